"""MLA shard partials + combine on the GPU vs the fp64 oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import ShardRun, assert_rows_close, oracle_rows, say
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu


def run_all_shards(case, dev, ranks=None):
    w = case.w
    ranks = range(w.num_shards) if ranks is None else ranks
    outs, lses = [], []
    for r in ranks:
        say(f"  mla partial {w.name} b={w.batch} H={w.heads} N={w.num_shards} r={r} B={w.block_size} "
            f"layout={w.layout} lens={list(case.seq_lens)[:6]}")
        sr = ShardRun(case, r, dev)
        o, l = sr.run()
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    return outs, lses


def check_case(case, dev, check_partials=True):
    w = case.w
    outs, lses = run_all_shards(case, dev)
    heads = list(range(w.heads))
    for b in range(w.batch):
        if check_partials:
            for r in range(w.num_shards):
                o_ref, l_ref = oracle_rows(case, b, heads, r)
                assert_rows_close(outs[r][b].cpu().numpy(), lses[r][b].cpu().numpy(), o_ref, l_ref,
                                  f"partial b={b} r={r}")
    po = torch.stack(outs)
    pl = torch.stack(lses)
    out_f = torch.empty_like(outs[0])
    lse = torch.empty_like(lses[0])
    out_bf = torch.empty(out_f.shape, dtype=torch.bfloat16, device=dev)
    ops.dcp_combine(po, pl, out_bf, out_f, lse)
    torch.cuda.synchronize()
    for b in range(w.batch):
        o_ref, l_ref = oracle_rows(case, b, heads, None)
        assert_rows_close(out_f[b].cpu().numpy(), lse[b].cpu().numpy(), o_ref, l_ref, f"combined b={b}")
        # the bf16 output is the device's own fp32 result rounded to nearest even
        assert np.array_equal(out_bf[b].view(torch.int16).cpu().numpy().view(np.uint16),
                              oracle.bf16_rne_bits(out_f[b].cpu().numpy()))
    return outs, lses


def test_c0_tiny_mla_all_shards(dev):
    say("c0")
    check_case(W.Case(W.WORKLOADS["c0"], seed=0), dev)


@pytest.mark.parametrize("lens,n,layout,heads,bs", [
    ((1,), 1, 0, 16, 64),
    ((1, 2, 3), 4, 0, 16, 64),               # L < N: empty shards
    ((5, 31, 32, 33), 2, 0, 32, 16),
    ((63, 64, 65, 100), 3, 1, 48, 32),
    ((257, 1000, 64 * 7 + 3), 4, 1, 64, 128),
    ((2048, 17, 640), 8, 0, 64, 64),
    ((4097,), 2, 0, 16, 48),                 # block size not a power of two
])
def test_edge_lengths(dev, lens, n, layout, heads, bs):
    w = W.custom_workload(kind="mla", batch=len(lens), heads=heads, seq_lens=lens, num_shards=n,
                          layout=layout, block_size=bs, wid=200)
    check_case(W.Case(w, seed=1), dev)


def test_zero_length_requests(dev):
    w = W.custom_workload(kind="mla", batch=4, heads=16, seq_lens=(0, 40, 0, 7), num_shards=2, wid=201)
    outs, lses = run_all_shards(W.Case(w, seed=2), dev)
    for r in range(2):
        l = lses[r].cpu().numpy()
        o = outs[r].cpu().numpy()
        assert np.all(np.isneginf(l[0])) and np.all(np.isneginf(l[2])), "empty requests need lse=-inf"
        assert np.all(o[0] == 0) and np.all(o[2] == 0)
    check_case(W.Case(w, seed=2), dev)


@pytest.mark.parametrize("min_tiles,wgs,seg_cost", [(1, 256, 6), (3, 7, 1), (8, 1, 6), (2, 512, 0), (1000, 256, 6),
                                                    (1, 64, 13), (1, 300, 5)])
def test_split_plans(dev, monkeypatch, min_tiles, wgs, seg_cost):
    """Same answer whatever the split of the tile list over workgroups,
    including segment charges that put workgroup boundaries inside a
    request's charge positions (odd and even charges split unevenly)."""
    monkeypatch.setenv("DCP_MLA_MIN_TILES", str(min_tiles))
    monkeypatch.setenv("DCP_SPLIT_WGS", str(wgs))
    monkeypatch.setenv("DCP_MLA_SEG_COST", str(seg_cost))
    w = W.custom_workload(kind="mla", batch=5, heads=64, seq_lens=(3000, 1, 777, 5000, 64),
                          num_shards=2, wid=202)
    check_case(W.Case(w, seed=3), dev)


def test_peaked_scores_and_needle(dev):
    """Sharper softmax (q x 8) and planted dominant keys stress the running max."""
    w = W.custom_workload(kind="mla", batch=2, heads=64, seq_lens=(3000, 9000), num_shards=4, wid=203)
    case = W.Case(w, seed=4, q_scale_pow2=3, needles=[(0, 2500, 5), (1, 10, 63), (1, 8999, 0)])
    check_case(case, dev)


def test_deterministic(dev):
    w = W.custom_workload(kind="mla", batch=3, heads=64, seq_lens=(5000, 300, 12000), num_shards=2, wid=204)
    case = W.Case(w, seed=5)
    sr = ShardRun(case, 1, dev)
    o1, l1 = sr.run(torch.empty_like(sr.out), torch.empty_like(sr.lse))
    o2, l2 = sr.run(torch.empty_like(sr.out), torch.empty_like(sr.lse))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_c1_full(dev):
    """64 heads, 64K context, shard 1 of 8: every shard's partial and the combine."""
    say("c1 full")
    check_case(W.Case(W.WORKLOADS["c1"], seed=0), dev)


@pytest.mark.parametrize("bs", [16, 48])
def test_long_segment_table_window(dev, monkeypatch, bs):
    """One workgroup walks > 1024 cache blocks of one request, so the staged
    block-table window has to slide; small blocks also split tiles."""
    monkeypatch.setenv("DCP_SPLIT_WGS", "1")
    w = W.custom_workload(kind="mla", batch=2, heads=64, seq_lens=(70001, 33), num_shards=2, block_size=bs,
                          wid=205)
    check_case(W.Case(w, seed=6), dev)


def test_workspace_reuse_across_shapes(dev):
    """One workspace (sized for the largest call) serves calls of different
    batch sizes and split counts in a row, with the same results each time."""
    big = W.custom_workload(kind="mla", batch=8, heads=64, seq_lens=(4000, 9000, 1, 300, 7000, 64, 2500, 10),
                            num_shards=2, wid=207)
    small = W.custom_workload(kind="mla", batch=1, heads=64, seq_lens=(30000,), num_shards=2, wid=208)
    rb = ShardRun(W.Case(big, seed=8), 0, dev)
    rs = ShardRun(W.Case(small, seed=9), 0, dev, workspace=rb.ws)
    ref_b = [o.clone() for o in rb.run()]
    ref_s = [o.clone() for o in rs.run()]
    for _ in range(3):
        ob, lb = rb.run(torch.empty_like(rb.out), torch.empty_like(rb.lse))
        os_, ls = rs.run(torch.empty_like(rs.out), torch.empty_like(rs.lse))
        torch.cuda.synchronize()
        assert torch.equal(ob, ref_b[0]) and torch.equal(lb, ref_b[1])
        assert torch.equal(os_, ref_s[0]) and torch.equal(ls, ref_s[1])
    for b in range(big.batch):
        o_ref, l_ref = oracle_rows(rb.case, b, list(range(64)), 0)
        assert_rows_close(ref_b[0][b].cpu().numpy(), ref_b[1][b].cpu().numpy(), o_ref, l_ref, f"big b={b}")
