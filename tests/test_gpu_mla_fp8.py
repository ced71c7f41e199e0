"""MLA shard partials over an fp8 (E4M3) latent cache on the GPU vs the fp64
oracle (``oracle.mla_attention_fp8``: exact decoding of the codes times the
cache's dequantization scale), then the combine of all shards."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import ShardRun, assert_rows_close, oracle_rows, say
from tests.test_gpu_mla import check_case
from workloads.device import bf16_tensor, fp8_tensor, int32_tensor
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu


def test_c0_fp8_all_shards(dev):
    w = W.WORKLOADS["c0"]
    check_case(W.Case(w, seed=0, kv_fp8_scale=W.FP8_SCALE), dev)


@pytest.mark.parametrize("lens,n,layout,heads,bs,scale", [
    ((1,), 1, 0, 16, 64, 1.0),
    ((1, 2, 3), 4, 0, 16, 64, W.FP8_SCALE),         # L < N: empty shards
    ((5, 31, 32, 33), 2, 0, 32, 16, 0.0125),
    ((63, 64, 65, 100), 3, 1, 48, 32, 3.0),          # most codes subnormal
    ((257, 1000, 64 * 7 + 3), 4, 1, 64, 128, 0.0125),
    ((2048, 17, 640), 8, 0, 64, 64, W.FP8_SCALE),
    ((4097,), 2, 0, 16, 48, 0.25),                   # block size not a power of two
])
def test_fp8_edge_lengths(dev, lens, n, layout, heads, bs, scale):
    w = W.custom_workload(kind="mla", batch=len(lens), heads=heads, seq_lens=lens, num_shards=n,
                          layout=layout, block_size=bs, wid=400)
    check_case(W.Case(w, seed=1, kv_fp8_scale=scale), dev)


@pytest.mark.parametrize("min_tiles,wgs,seg_cost", [(1, 256, 6), (3, 7, 3), (8, 1, 6), (2, 512, 0), (1, 64, 11)])
def test_fp8_split_plans(dev, monkeypatch, min_tiles, wgs, seg_cost):
    monkeypatch.setenv("DCP_MLA8_MIN_TILES", str(min_tiles))
    monkeypatch.setenv("DCP_SPLIT_WGS", str(wgs))
    monkeypatch.setenv("DCP_MLA8_SEG_COST", str(seg_cost))
    w = W.custom_workload(kind="mla", batch=5, heads=64, seq_lens=(3000, 1, 777, 5000, 64),
                          num_shards=2, wid=401)
    check_case(W.Case(w, seed=3, kv_fp8_scale=W.FP8_SCALE), dev)


def test_fp8_peaked_scores_and_needle(dev):
    """Sharper softmax and planted dominant keys (the reference-overflow rerun)."""
    w = W.custom_workload(kind="mla", batch=2, heads=64, seq_lens=(3000, 9000), num_shards=4, wid=402)
    case = W.Case(w, seed=4, q_scale_pow2=3, needles=[(0, 2500, 5), (1, 10, 63), (1, 8999, 0)],
                  kv_fp8_scale=W.FP8_SCALE)
    check_case(case, dev)


@pytest.mark.parametrize("bs", [16, 64])
def test_fp8_long_segment_table_window(dev, monkeypatch, bs):
    monkeypatch.setenv("DCP_SPLIT_WGS", "1")
    w = W.custom_workload(kind="mla", batch=2, heads=64, seq_lens=(70001, 33), num_shards=2, block_size=bs,
                          wid=403)
    check_case(W.Case(w, seed=6, kv_fp8_scale=W.FP8_SCALE), dev)


def test_fp8_deterministic_and_scale_linear(dev):
    """Repeated calls agree bit for bit; doubling the scale with halved codes'
    values is the same cache, so the results agree to rounding."""
    w = W.custom_workload(kind="mla", batch=3, heads=64, seq_lens=(5000, 300, 12000), num_shards=2, wid=404)
    case = W.Case(w, seed=5, kv_fp8_scale=0.02)
    sr = ShardRun(case, 1, dev)
    o1, l1 = sr.run(torch.empty_like(sr.out), torch.empty_like(sr.lse))
    o2, l2 = sr.run(torch.empty_like(sr.out), torch.empty_like(sr.lse))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_multi_token(dev):
    """A 3-token step over an fp8 cache: per-shard partials and the merge vs the oracle."""
    w = W.custom_workload(kind="mla", batch=2, heads=64, seq_lens=(900, 5), num_shards=4, layout=1, wid=405)
    case = W.Case(w, seed=7, kv_fp8_scale=W.FP8_SCALE)
    q_len, b, n = 3, 2, 4
    qbits = case.queries(q_len)
    q_d = bf16_tensor(qbits.reshape(b * q_len, 64, 576), dev)
    mb = case.max_blocks_per_seq()
    po = torch.full((n, b * q_len, 64, 512), float("nan"), dtype=torch.float32, device=dev)
    pl = torch.full((n, b * q_len, 64), float("nan"), dtype=torch.float32, device=dev)
    for r in range(n):
        sc = case.shard(r, max_blocks=mb)
        p = ops.mla_params(batch=b, num_heads=64, block_size=w.block_size, max_blocks_per_seq=mb,
                           num_blocks=sc.num_blocks, shard_rank=r, num_shards=n, layout=1, max_seq_len_hint=900,
                           softmax_scale=w.scale, q_len=q_len)
        ops.dcp_mla_decode_partial_fp8(p, q_d, fp8_tensor(sc.pools[0], dev), case.kv_fp8_scale,
                                       int32_tensor(sc.block_table, dev), int32_tensor(case.seq_lens, dev),
                                       po[r], pl[r], ops.mla_workspace(p, dev))
    merged = torch.empty((b * q_len, 64, 512), dtype=torch.float32, device=dev)
    mlse = torch.empty((b * q_len, 64), dtype=torch.float32, device=dev)
    ops.dcp_combine(po, pl, None, merged, mlse)
    torch.cuda.synchronize()
    po_h, pl_h, m_h, ml_h = po.cpu().numpy(), pl.cpu().numpy(), merged.cpu().numpy(), mlse.cpu().numpy()
    for bb in range(b):
        L = int(case.seq_lens[bb])
        for j in range(q_len):
            q = oracle.widen_bf16(qbits[bb, j])
            for r in range(n):
                pos = oracle.query_positions(L, q_len, j, n, r, 1)
                bits = case.rows_at(bb, pos)[0] if len(pos) else np.zeros((0, 576), np.uint8)
                o_ref, l_ref = oracle.mla_attention_fp8(q, bits, case.kv_fp8_scale, w.scale)
                assert_rows_close(po_h[r, bb * q_len + j], pl_h[r, bb * q_len + j], o_ref, l_ref,
                                  f"b={bb} j={j} r={r}")
            bits = case.rows_at(bb, np.arange(oracle.query_limit(L, q_len, j)))[0]
            o_ref, l_ref = oracle.mla_attention_fp8(q, bits, case.kv_fp8_scale, w.scale)
            assert_rows_close(m_h[bb * q_len + j], ml_h[bb * q_len + j], o_ref, l_ref, f"merged b={bb} j={j}")


@pytest.mark.parametrize("name,reqs,heads", [
    ("c4b", [0, 64, 127], [0, 21, 42, 63]),
    ("c2", [0, 11, 31], [0, 17, 40, 63]),
])
def test_fp8_full_size_sampled(dev, name, reqs, heads):
    """The fp8 cache at the benchmark workloads' full sizes (timed shard only;
    sampled rows against the oracle one by one)."""
    w = W.WORKLOADS[name]
    case = W.Case(w, seed=0, kv_fp8_scale=W.FP8_SCALE)
    r = w.ranks[0]
    say(f"fp8 full-size {name}: generating shard {r}")
    sr = ShardRun(case, r, dev, max_blocks=case.max_blocks_per_seq())
    o, l = sr.run()
    torch.cuda.synchronize()
    for b in reqs:
        say(f"  {name} fp8 oracle rows for request {b}")
        o_ref, l_ref = oracle_rows(case, b, heads, r)
        assert_rows_close(o[b][heads].cpu().numpy(), l[b][heads].cpu().numpy(), o_ref, l_ref,
                          f"{name} fp8 partial b={b}")
