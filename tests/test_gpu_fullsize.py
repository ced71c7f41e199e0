"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (default split plan), on sampled (request, head) rows that the
oracle computes one by one.  Every shard's partial is produced by the HIP path
from its own paged cache; the combine merges all of them."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import ShardRun, assert_rows_close, oracle_rows, oracle_rows_merged, say
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu

SAMPLES = {
    "c2": ([0, 3, 11, 20, 31], [0, 17, 63]),
    "c3": ([0, 7, 15], [0, 9, 40, 63]),
    "c4a": ([0], [0, 21, 42, 63]),
    "c4b": ([0, 64, 127], [0, 31, 63]),
}


@pytest.mark.parametrize("name", ["c2", "c3", "c4a", "c4b"])
def test_full_size_sampled(dev, name):
    w = W.WORKLOADS[name]
    case = W.Case(w, seed=0)
    say(f"full-size {name}: {w.description}; generating {w.num_shards} shards")
    caches = case.shards(range(w.num_shards), max_blocks=case.max_blocks_per_seq())
    outs, lses = [], []
    for r in range(w.num_shards):
        say(f"  {name} shard {r} partial")
        sr = ShardRun(case, r, dev, cache=caches[r])
        caches[r] = None
        o, l = sr.run()
        torch.cuda.synchronize()
        outs.append(o)
        lses.append(l)
        del sr
    out_f = torch.empty_like(outs[0])
    lse = torch.empty_like(lses[0])
    out_bf = torch.empty(out_f.shape, dtype=torch.bfloat16, device=dev)
    ops.dcp_combine(torch.stack(outs), torch.stack(lses), out_bf, out_f, lse)
    torch.cuda.synchronize()
    reqs, heads = SAMPLES[name]
    for b in reqs:
        say(f"  {name} oracle rows for request {b} (L={int(case.seq_lens[b])})")
        for r in w.ranks:
            o_ref, l_ref = oracle_rows(case, b, heads, r)
            assert_rows_close(outs[r][b][heads].cpu().numpy(), lses[r][b][heads].cpu().numpy(), o_ref, l_ref,
                              f"{name} partial b={b} r={r}")
        o_ref, l_ref = oracle_rows_merged(case, b, heads)
        assert_rows_close(out_f[b][heads].cpu().numpy(), lse[b][heads].cpu().numpy(), o_ref, l_ref,
                          f"{name} combined b={b}")
