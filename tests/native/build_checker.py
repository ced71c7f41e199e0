"""Build the host-side checkers (tests/native/libsplitcheck.so: the split plan;
tests/native/libgqalayout.so: the GQA tile layout), test helpers compiled from
the library's own headers."""
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
GQA_SRC = os.path.join(HERE, "gqa_layout_check.hip")
GQA_LIB = os.path.join(HERE, "libgqalayout.so")


def _build(src: str, lib: str) -> str:
    tmp = lib + ".tmp"
    cmd = [_lib_build.HIPCC, *_lib_build.CFLAGS, "-shared", "-o", tmp, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"checker build failed ({os.path.basename(src)}):\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build() -> str:
    return _build(SRC, LIB)


def build_gqa() -> str:
    return _build(GQA_SRC, GQA_LIB)


if __name__ == "__main__":
    print(build())
    print(build_gqa())
