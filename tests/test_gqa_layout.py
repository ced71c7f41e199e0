"""The GQA partial kernel's tile layout, checked on the host: the kernel's own
layout functions (compiled for the host from csrc/gqa_layout.hpp) must copy
every LDS chunk of a part exactly once from the right cache bytes, keep each
copy inside one 16-token sub-tile, and point every score and value operand
read at the bytes it means (see tests/native/gqa_layout_check.hip)."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

from kv_cache_context_amd import build as lib_build
from tests.native import build_checker

_lib = None


def checker():
    global _lib
    if _lib is None:
        if not os.path.exists(build_checker.GQA_LIB):
            build_checker.build_gqa()
        _lib = ctypes.CDLL(build_checker.GQA_LIB)
        _lib.dcp_gqa_layout_check.restype = ctypes.c_int
    return _lib


@pytest.mark.parametrize("hg,hkv", [(4, 4), (4, 8), (4, 64), (2, 2), (2, 6), (2, 10), (1, 1), (1, 3), (1, 7)])
def test_gqa_tile_layout(hg, hkv):
    msg = ctypes.create_string_buffer(256)
    assert checker().dcp_gqa_layout_check(hg, hkv, msg, 256) == 0, msg.value.decode()


def test_gqa_layout_check_rejects_unservable_head_count():
    """HG must divide Hkv (the launcher picks the largest of 4, 2, 1 that does)."""
    msg = ctypes.create_string_buffer(256)
    assert checker().dcp_gqa_layout_check(4, 6, msg, 256) != 0


# Plausible mistakes in the layout functions; each must make the check fail
# for at least one HG.
MUTANTS = [
    ("return (uint32_t)(rel * hkv * HROW + h * HROW + ((ch ^ swz(tok)) * 16));",
     "return (uint32_t)(rel * hkv * HROW + h * HROW + (ch * 16));"),                  # copy without the swizzle
    ("return Geo<HG>::SUB == 1 ? 4 * j + wave : 4 * wave + j;",
     "return 4 * j + wave;"),                                                           # slots interleaved for all HG
    ("const int rel = tok - 16 * (wave / HG);", "const int rel = tok;"),                # base of sub-tile 0, not the wave's
    ("return (16 * sub + 4 * g4 + (r16 >> 2)) * Geo<HG>::TROW + hk * HROW + (r16 & 1) * 8 +",
     "return (16 * sub + 4 * g4 + (r16 >> 2)) * Geo<HG>::TROW + hk * HROW + (r16 & 1) * 4 +"),  # wrong half chunk
]


@pytest.mark.parametrize("i", range(len(MUTANTS)))
def test_gqa_layout_check_catches_planted_mistakes(i):
    old, new = MUTANTS[i]
    header = os.path.join(lib_build.CSRC, "gqa_layout.hpp")
    src = open(header).read()
    assert old in src, "mutant no longer matches the header"
    with tempfile.TemporaryDirectory() as d:
        open(os.path.join(d, "gqa_layout.hpp"), "w").write(src.replace(old, new))
        shutil.copy(build_checker.GQA_SRC, d)
        lib = os.path.join(d, "libmut.so")
        cmd = [lib_build.HIPCC, *lib_build.CFLAGS, "-shared", "-o", lib, os.path.join(d, "gqa_layout_check.hip")]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        mut = ctypes.CDLL(lib)
        mut.dcp_gqa_layout_check.restype = ctypes.c_int
        msg = ctypes.create_string_buffer(256)
        results = [mut.dcp_gqa_layout_check(hg, hkv, msg, 256) for hg, hkv in ((4, 8), (2, 2), (1, 1))]
        assert any(rc != 0 for rc in results), f"mutant {i} passed the layout check"
