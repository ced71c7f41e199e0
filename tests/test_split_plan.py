"""The split plan of the partial kernels, checked on the host over many
configurations: the library's own planning functions (compiled for the host
from the same header) must give every tile to exactly one workgroup and hand
the reduce kernel exactly the segments that were written (see
tests/native/split_plan_check.hip for the invariants)."""
import ctypes
import os

import numpy as np
import pytest

from tests.native import build_checker

_lib = None


def checker():
    global _lib
    if _lib is None:
        if not os.path.exists(build_checker.LIB):
            build_checker.build()
        _lib = ctypes.CDLL(build_checker.LIB)
        _lib.dcp_split_plan_check.restype = ctypes.c_int
    return _lib


def check(lens, q_len=1, nshards=1, rank=0, layout=0, block_size=64, max_blocks=None, G=256, min_tiles=4,
          seg_cost=6, tile=32):
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if max_blocks is None:
        local = -(-int(max(lens.max(), 1)) // nshards)
        max_blocks = -(-local // block_size) + 1
    msg = ctypes.create_string_buffer(256)
    rc = checker().dcp_split_plan_check(
        ctypes.c_int(len(lens)), lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), q_len, nshards, rank, layout,
        block_size, max_blocks, G, min_tiles, seg_cost, tile, msg, 256)
    assert rc == 0, f"{msg.value.decode()} for lens={list(lens)[:8]} q_len={q_len} N={nshards} r={rank} " \
                    f"layout={layout} B={block_size} G={G} min_tiles={min_tiles} seg_cost={seg_cost} tile={tile}"


def test_workload_shapes():
    check([1024, 1024], nshards=4, rank=1, G=256, seg_cost=6)          # tiny MLA
    check([65536], nshards=8, rank=1)                                  # one request, one shard of 8
    check([65536] * 128, nshards=8, rank=1)                            # batch 128
    check([1 << 20], nshards=8, rank=7)                                # 1M tokens, last shard
    check([131072] * 16, nshards=4, rank=1, block_size=16, G=128, min_tiles=16, seg_cost=0, tile=16)  # GQA
    check([131072] * 16, nshards=2, rank=1, block_size=16, G=256, min_tiles=16, seg_cost=0, tile=64)  # GQA, 1 KV head
    check([70000, 3, 17, 64], nshards=2, rank=0, block_size=16, G=128, min_tiles=1, seg_cost=0, tile=32)  # 2 KV heads


def test_degenerate_plans():
    check([0])                                   # no work at all
    check([0, 0, 0], nshards=4)
    check([1, 2, 3], nshards=4, rank=3)          # L < N: empty slices
    check([5000, 0, 17, 0], nshards=2, G=1)      # one workgroup walks everything
    check([1], G=512, min_tiles=1, seg_cost=13)  # more charge positions than tiles
    check([33] * 300, G=7, min_tiles=1, seg_cost=1)


@pytest.mark.parametrize("seed", range(8))
def test_random_plans(seed):
    rng = np.random.default_rng([seed, 4242])
    for _ in range(250):
        nreq = int(rng.integers(1, 64))
        kind = rng.integers(0, 3)
        if kind == 0:
            lens = rng.integers(0, 3000, nreq)
        elif kind == 1:
            lens = np.exp(rng.uniform(0, np.log(300000), nreq)).astype(np.int64)
        else:
            lens = rng.choice([0, 1, 31, 32, 33, 4096, 65536], nreq)
        q_len = int(rng.choice([1, 1, 2, 4, 9]))
        lens = np.maximum(lens, 0)
        if q_len > 1:
            lens = np.where(lens > 0, np.maximum(lens, q_len), 0)
        nshards = int(rng.choice([1, 2, 3, 4, 8, 16]))
        check(lens, q_len=q_len, nshards=nshards, rank=int(rng.integers(0, nshards)), layout=int(rng.integers(0, 2)),
              block_size=int(rng.choice([16, 32, 48, 64, 128])), G=int(rng.integers(1, 513)),
              min_tiles=int(rng.integers(1, 17)), seg_cost=int(rng.integers(0, 14)), tile=int(rng.choice([16, 32, 64])))
