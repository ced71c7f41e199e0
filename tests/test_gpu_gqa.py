"""GQA shard partials + combine on the GPU vs the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import ShardRun, assert_rows_close, oracle_rows, say
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu


def run_all(case, dev):
    w = case.w
    outs, lses = [], []
    for r in range(w.num_shards):
        say(f"  gqa partial b={w.batch} Hq={w.heads} Hkv={w.kv_heads} N={w.num_shards} r={r} B={w.block_size} "
            f"layout={w.layout} lens={list(case.seq_lens)[:6]}")
        o, l = ShardRun(case, r, dev).run()
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    return outs, lses


def check(case, dev, heads=None, reqs=None):
    w = case.w
    outs, lses = run_all(case, dev)
    heads = list(range(w.heads)) if heads is None else heads
    reqs = range(w.batch) if reqs is None else reqs
    for b in reqs:
        for r in range(w.num_shards):
            o_ref, l_ref = oracle_rows(case, b, heads, r)
            assert_rows_close(outs[r][b][heads].cpu().numpy(), lses[r][b][heads].cpu().numpy(), o_ref, l_ref,
                              f"gqa partial b={b} r={r}")
    out_f = torch.empty_like(outs[0])
    lse = torch.empty_like(lses[0])
    out_bf = torch.empty(out_f.shape, dtype=torch.bfloat16, device=dev)
    ops.dcp_combine(torch.stack(outs), torch.stack(lses), out_bf, out_f, lse)
    torch.cuda.synchronize()
    for b in reqs:
        o_ref, l_ref = oracle_rows(case, b, heads, None)
        assert_rows_close(out_f[b][heads].cpu().numpy(), lse[b][heads].cpu().numpy(), o_ref, l_ref,
                          f"gqa combined b={b}")


@pytest.mark.parametrize("hq,hkv,lens,n,layout,bs", [
    (64, 8, (1, 15, 16, 17, 100, 1000), 4, 0, 16),
    (32, 4, (5, 33, 2000), 2, 1, 32),
    (16, 16, (40, 300), 3, 0, 16),       # MHA: group of 1
    (64, 4, (77, 1500), 2, 0, 64),       # group of 16
    (24, 8, (129, 1), 4, 1, 48),         # group of 3
    (64, 8, (3,), 8, 0, 16),             # L < N
])
def test_gqa_shapes(dev, hq, hkv, lens, n, layout, bs):
    w = W.custom_workload(kind="gqa", batch=len(lens), heads=hq, kv_heads=hkv, head_dim=128, seq_lens=lens,
                          num_shards=n, layout=layout, block_size=bs, wid=300)
    check(W.Case(w, seed=1), dev)


@pytest.mark.parametrize("seg_cost", [0, 5])
def test_gqa_zero_lengths_and_splits(dev, monkeypatch, seg_cost):
    monkeypatch.setenv("DCP_GQA_MIN_TILES", "1")
    monkeypatch.setenv("DCP_SPLIT_WGS", "37")
    monkeypatch.setenv("DCP_GQA_SEG_COST", str(seg_cost))
    w = W.custom_workload(kind="gqa", batch=4, heads=64, kv_heads=8, seq_lens=(0, 5000, 17, 0), num_shards=2,
                          block_size=16, wid=301)
    check(W.Case(w, seed=2), dev)


def test_gqa_long_single_workgroup(dev, monkeypatch):
    """One workgroup walks > 1024 blocks (block-table window slides)."""
    monkeypatch.setenv("DCP_SPLIT_WGS", "1")
    w = W.custom_workload(kind="gqa", batch=1, heads=64, kv_heads=8, seq_lens=(40000,), num_shards=2,
                          block_size=16, wid=302)
    check(W.Case(w, seed=3), dev)


def test_gqa_peaked(dev):
    w = W.custom_workload(kind="gqa", batch=2, heads=64, kv_heads=8, seq_lens=(3000, 700), num_shards=4,
                          block_size=16, wid=303)
    check(W.Case(w, seed=4, q_scale_pow2=3), dev)


def test_gqa_deterministic(dev):
    w = W.custom_workload(kind="gqa", batch=3, heads=64, kv_heads=8, seq_lens=(5000, 300, 9000), num_shards=2,
                          block_size=16, wid=304)
    sr = ShardRun(W.Case(w, seed=5), 1, dev)
    o1, l1 = sr.run(torch.empty_like(sr.out), torch.empty_like(sr.lse))
    o2, l2 = sr.run(torch.empty_like(sr.out), torch.empty_like(sr.lse))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("hq,hkv,lens,n,layout,bs", [
    (8, 1, (1, 15, 16, 17, 63, 64, 65, 1000), 2, 0, 16),  # one KV head per rank: 64-token tiles over 16-token blocks
    (16, 2, (5, 31, 32, 33, 2000), 2, 1, 32),             # two KV heads per rank: 32-token tiles
    (64, 1, (100, 3000), 2, 0, 64),                       # MQA: 64 query heads on one KV head
    (32, 1, (49, 700), 4, 1, 48),                         # 2 query blocks, block size not a power of two
    (48, 1, (17, 1200), 2, 0, 16),                        # 3 query blocks
    (24, 3, (129, 1, 400), 4, 1, 16),                     # odd Hkv: one KV head per workgroup, groups of 8
    (36, 6, (300, 2), 2, 0, 32),                          # Hkv 6: two KV heads per workgroup, groups of 6
    (64, 2, (3,), 8, 0, 16),                              # L < N
])
def test_gqa_few_kv_heads(dev, hq, hkv, lens, n, layout, bs):
    """Fewer than 4 KV heads per workgroup: the waves split each tile's tokens
    and merge their states at the end of a segment."""
    w = W.custom_workload(kind="gqa", batch=len(lens), heads=hq, kv_heads=hkv, head_dim=128, seq_lens=lens,
                          num_shards=n, layout=layout, block_size=bs, wid=305)
    check(W.Case(w, seed=6), dev)


@pytest.mark.parametrize("hkv,seg_cost", [(1, 0), (1, 5), (2, 3)])
def test_gqa_few_kv_heads_splits(dev, monkeypatch, hkv, seg_cost):
    monkeypatch.setenv("DCP_GQA_MIN_TILES", "1")
    monkeypatch.setenv("DCP_SPLIT_WGS", "37")
    monkeypatch.setenv("DCP_GQA_SEG_COST", str(seg_cost))
    w = W.custom_workload(kind="gqa", batch=5, heads=8 * hkv, kv_heads=hkv, seq_lens=(0, 5000, 17, 0, 130),
                          num_shards=2, block_size=16, wid=306)
    check(W.Case(w, seed=7), dev)


@pytest.mark.parametrize("hq,hkv", [(8, 1), (64, 1), (16, 2)])
def test_gqa_few_kv_heads_long_single_workgroup(dev, monkeypatch, hq, hkv):
    """One workgroup walks > 1024 blocks (the block-table window slides while
    the sub-tiles of one tile sit in different blocks)."""
    monkeypatch.setenv("DCP_SPLIT_WGS", "1")
    w = W.custom_workload(kind="gqa", batch=1, heads=hq, kv_heads=hkv, seq_lens=(40001,), num_shards=2,
                          block_size=16, wid=307)
    check(W.Case(w, seed=8), dev)


def test_gqa_one_kv_head_peaked(dev):
    w = W.custom_workload(kind="gqa", batch=2, heads=64, kv_heads=1, seq_lens=(3000, 700), num_shards=4,
                          block_size=16, wid=308)
    check(W.Case(w, seed=9, q_scale_pow2=3), dev)
