"""Build the gfx950 HIP library ``libidx.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libidx.so"
SOURCES = ["api.hip", "score.hip", "score_rows.hip", "topk.hip", "fp4_store.hip", "noalloc.hip",
           "probe.hip", "attn.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def build(out: Path | str | None = None, verbose: bool = False, extra_flags=(),
          csrc: Path | str | None = None) -> Path:
    """Compile the library to ``out``.  ``extra_flags`` (e.g. -D overrides of
    the score kernel's tuning knobs) and another source directory are for
    experiments; the default build uses neither."""
    out = Path(out) if out is not None else LIB
    src = Path(csrc) if csrc is not None else CSRC
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    flags = [f if f != f"-I{CSRC}" else f"-I{src}" for f in HIPCC_FLAGS]
    cmd = ["hipcc", *flags, *extra_flags, *[str(src / s) for s in SOURCES], "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
