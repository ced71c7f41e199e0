"""Build the host-side split-plan checker (tests/native/libsplitcheck.so), a
test helper compiled from the library's own planning header."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
from kv_cache_context_amd import build as _lib_build  # noqa: E402  (the library's compiler and flags)

SRC = os.path.join(HERE, "split_plan_check.hip")
LIB = os.path.join(HERE, "libsplitcheck.so")


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = [_lib_build.HIPCC, *_lib_build.CFLAGS, "-shared", "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"split-plan checker build failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
