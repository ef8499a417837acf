"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) must pass every pin: no out-of-bounds access, leak of
a freed buffer, signed overflow or other undefined behaviour on the pins'
inputs.  The pins run in a child process with the ASan runtime preloaded,
since the Python interpreter itself is not instrumented."""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

import pytest

from oracle import build as obuild

ROOT = Path(__file__).resolve().parents[1]

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import pins
from oracle.binding import Oracle
o = Oracle({lib!r})
for pin in pins.PINS:
    pin(o)
print("pins passed:", len(pins.PINS), flush=True)
"""


def test_pins_under_sanitizers(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not asan or not Path(asan).exists():
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = obuild.build(tmp_path / "liboracle_san.so", sanitize=True)
    env = dict(os.environ, LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = CHILD.format(root=str(ROOT), tests=str(ROOT / "tests"), lib=str(lib))
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, f"sanitized oracle failed its pins:\n{tail}"
    assert "pins passed" in res.stdout, tail
    assert "runtime error" not in res.stderr, tail
