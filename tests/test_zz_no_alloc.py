"""The no-allocation MLA entry point (fixed device scratch instead of a
caller workspace) against dcp_mla_decode_partial, through the C ABI: the same
kernels and split, so the results must be identical, also on a second call
with a smaller input that finds the previous call's data in the scratch."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import ShardRun, say
from kv_cache_context_amd import dcp, ops

pytestmark = pytest.mark.gpu


def _both(dev, case, r):
    sr = ShardRun(case, r, dev)
    o1, l1 = sr.run()
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    ops.dcp_mla_decode_partial_noalloc(sr.p, sr.q, sr.kv, sr.table, sr.seq_lens, o2, l2)
    torch.cuda.synchronize()
    return o1.cpu().numpy(), l1.cpu().numpy(), o2.cpu().numpy(), l2.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice(dev):
    # first call: 3 requests, a split one (9000 tokens), an empty shard slice
    # and a short one; second call: smaller, 2 requests
    calls = [
        W.custom_workload(batch=3, heads=64, seq_lens=(9000, 3, 4100), num_shards=4, wid=150),
        W.custom_workload(batch=2, heads=64, seq_lens=(700, 2500), num_shards=4, wid=151),
    ]
    for k, w in enumerate(calls):
        case = W.Case(w, seed=3)
        for r in (1, 3):
            say(f"no-alloc call {k}: lens {list(case.seq_lens)} shard {r}")
            o1, l1, o2, l2 = _both(dev, case, r)
            assert np.array_equal(np.isnan(o2), np.zeros_like(o2, bool)), "rows left unwritten"
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2, equal_nan=True), (k, r)


def test_noalloc_rejects_calls_beyond_the_scratch(dev):
    # 400 requests of 64 heads need more than the fixed scratch
    w = W.custom_workload(batch=400, heads=64, seq_lens=(64,) * 400, num_shards=1, wid=152)
    p = ops.mla_params(batch=400, num_heads=64, block_size=64, max_blocks_per_seq=1, num_blocks=400, shard_rank=0,
                       num_shards=1, layout=0, max_seq_len_hint=64, softmax_scale=w.scale)
    q = torch.zeros((400, 64, 576), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((400, 64, 576), dtype=torch.bfloat16, device=dev)
    table = torch.arange(400, dtype=torch.int32, device=dev).reshape(400, 1)
    lens = torch.full((400,), 64, dtype=torch.int32, device=dev)
    out = torch.zeros((400, 64, 512), dtype=torch.float32, device=dev)
    lse = torch.zeros((400, 64), dtype=torch.float32, device=dev)
    st = dcp.dcp_mla_decode_partial_noalloc(p, q.data_ptr(), kv.data_ptr(), table.data_ptr(), lens.data_ptr(),
                                            out.data_ptr(), lse.data_ptr(), 0)
    assert st == dcp.DCP_ERR_SCRATCH
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0  # nothing launched
