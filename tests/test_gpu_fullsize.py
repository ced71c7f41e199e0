"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (default split plan), on sampled (request, head) rows that the
oracle computes one by one.  Every shard's partial is produced by the HIP path
from its own paged cache; the combine merges all of them."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import ShardRun, assert_rows_close, oracle_all_shards, say
from workloads.device import bf16_tensor, int32_tensor
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu

# One head of each 16-head block: the MLA kernels give every block its own
# waves (and owner of the softmax), so each block is a separate code path.
MLA_HEADS = [0, 21, 42, 63]

SAMPLES = {
    "c1": ([0], MLA_HEADS),
    "c2": ([0, 3, 11, 20, 31], [0, 17, 40, 63]),
    "c3": ([0, 7, 15], [0, 9, 40, 63]),
    "c3kv1": ([0, 9, 15], list(range(8))),
    "c4a": ([0], MLA_HEADS),
    "c4b": ([0, 64, 127], MLA_HEADS),
}


@pytest.mark.parametrize("name,fp8", [("c2", False), ("c3", False), ("c3kv1", False), ("c4a", False), ("c4b", False),
                                      ("c4a", True), ("c1", True)])
def test_full_size_sampled(dev, name, fp8):
    """Every shard's partial (sampled rows) and the combine of all of them; the
    fp8 cases run the E4M3 cache (oracle: exact decoding times the scale)."""
    w = W.WORKLOADS[name]
    case = W.Case(w, seed=0, kv_fp8_scale=W.FP8_SCALE if fp8 else None)
    say(f"full-size {name}{' fp8' if fp8 else ''}: {w.description}; generating {w.num_shards} shards")
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
        ref = oracle_all_shards(case, b, heads)
        for r in w.ranks:
            o_ref, l_ref = ref[r]
            assert_rows_close(outs[r][b][heads].cpu().numpy(), lses[r][b][heads].cpu().numpy(), o_ref, l_ref,
                              f"{name} partial b={b} r={r}")
        # the combine against the oracle's merge of all shards
        o_ref, l_ref = ref[w.num_shards]
        assert_rows_close(out_f[b][heads].cpu().numpy(), lse[b][heads].cpu().numpy(), o_ref, l_ref,
                          f"{name} combined b={b}")


@pytest.mark.parametrize("name,q_len,reqs", [("c4b", 2, [0, 77, 127]), ("c4b", 4, [0, 127]), ("c2", 4, [0, 9, 31])])
def test_full_size_multi_token(dev, name, q_len, reqs):
    """q_len-token steps at full size on the timed shard: token j of request b
    attends the shard's positions below L - q_len + 1 + j; sampled (request,
    token, head) rows against the oracle over exactly those positions."""
    w = W.WORKLOADS[name]
    case = W.Case(w, seed=0)
    r = w.ranks[0]
    b, rows = w.batch, w.batch * q_len
    say(f"full-size {name} q_len={q_len}: generating shard {r}")
    mb = case.max_blocks_per_seq()
    sc = case.shard(r, max_blocks=mb)
    qbits = case.queries(q_len)
    p = ops.mla_params(batch=b, num_heads=w.heads, block_size=w.block_size, max_blocks_per_seq=mb,
                       num_blocks=sc.num_blocks, shard_rank=r, num_shards=w.num_shards, layout=w.layout,
                       max_seq_len_hint=max(1, case.max_seq_len), softmax_scale=w.scale, q_len=q_len)
    out = torch.full((rows, w.heads, w.dv), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((rows, w.heads), float("nan"), dtype=torch.float32, device=dev)
    say(f"  {name} q_len={q_len} partial")
    ops.dcp_mla_decode_partial(p, bf16_tensor(qbits.reshape(rows, w.heads, w.dk), dev),
                               bf16_tensor(sc.pools[0], dev), int32_tensor(sc.block_table, dev),
                               int32_tensor(case.seq_lens, dev), out, lse, ops.mla_workspace(p, dev))
    torch.cuda.synchronize()
    del sc
    for bb in reqs:
        L = int(case.seq_lens[bb])
        for j in range(q_len):
            say(f"  {name} q_len={q_len} oracle rows b={bb} j={j}")
            pos = oracle.query_positions(L, q_len, j, w.num_shards, r, w.layout)
            q = oracle.widen_bf16(qbits[bb, j, MLA_HEADS])
            kv = oracle.widen_bf16(case.rows_at(bb, pos)[0])
            o_ref, l_ref = oracle.mla_attention(q, kv, w.scale, w.kv_lora_rank)
            row = bb * q_len + j
            assert_rows_close(out[row][MLA_HEADS].cpu().numpy(), lse[row][MLA_HEADS].cpu().numpy(), o_ref, l_ref,
                              f"{name} q_len={q_len} b={bb} j={j}")
