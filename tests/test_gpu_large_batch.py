"""Batches larger than one pass of the in-kernel split planner (512 requests per
prefix-sum pass, up to 2048 row sets) on the GPU vs the fp64 oracle."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_helpers import say
from tests.test_gpu_mla import check_case

pytestmark = pytest.mark.gpu


def _lens(n, lo, hi, seed):
    return tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi, size=n))


@pytest.mark.parametrize("batch,heads,n,bs", [(1500, 16, 2, 16), (2048, 16, 4, 32)])
def test_mla_large_batch(dev, batch, heads, n, bs):
    lens = _lens(batch, 1, 300, batch)
    say(f"mla large batch b={batch} H={heads} N={n} B={bs}")
    w = W.custom_workload(kind="mla", batch=batch, heads=heads, seq_lens=lens, num_shards=n, block_size=bs,
                          wid=210)
    check_case(W.Case(w, seed=11), dev)


def test_gqa_large_batch(dev):
    from tests.test_gpu_gqa import check
    lens = _lens(1100, 1, 200, 1100)
    say("gqa large batch b=1100")
    w = W.custom_workload(kind="gqa", batch=1100, heads=16, kv_heads=4, head_dim=128, seq_lens=lens, num_shards=2,
                          block_size=16, wid=211)
    check(W.Case(w, seed=12), dev)


def test_mtp_large_row_count(dev):
    """300 requests x 4 query tokens = 1200 row sets (three planner passes)."""
    from tests.test_gpu_mtp import _check_mtp
    _check_mtp(dev, "mla", 300, 16, 1, _lens(300, 4, 250, 300), 16, 2, 0, 4)
