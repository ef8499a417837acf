"""Compile the C oracle (``oracle.c``) into a shared library with gcc.

Test infrastructure only.  ``mutant`` > 0 builds a copy with one deliberate
mistake compiled in (see ``ORACLE_MUTANT`` in oracle.c); the tests use those
copies to show that the oracle's pins reject each mistake.
"""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle.c"
DEFAULT_LIB = HERE / "liboracle.so"


# AddressSanitizer and UndefinedBehaviorSanitizer, host code only (gcc, no GPU
# code is involved); a process loading such a build needs libasan preloaded
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]


def build(out: Path | str | None = None, mutant: int = 0, openmp: bool = True,
          sanitize: bool = False) -> Path:
    out = Path(out) if out is not None else DEFAULT_LIB
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           f"-DORACLE_MUTANT={int(mutant)}", str(SRC), "-o", str(tmp), "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    if sanitize:
        cmd[1:1] = SANITIZE_FLAGS
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
