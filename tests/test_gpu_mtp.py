"""Multi-token decode steps (q_len > 1) on the GPU vs the oracle.

Query token j of a request with L cached positions attends the causal prefix
t <= L - q_len + j.  Every shard's partial of every (request, token) row set is
checked against the oracle over exactly the positions that shard holds in that
prefix (``oracle.query_positions``), and the merge of all shards (dcp_combine)
against unsharded attention over the prefix.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_rows_close, say
from workloads.device import bf16_tensor, int32_tensor
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu


def _oracle(case, qbits, b, j, positions):
    w = case.w
    q = oracle.widen_bf16(qbits[b, j])
    if w.kind == "mla":
        kv = oracle.widen_bf16(case.rows_at(b, positions)[0]) if len(positions) else np.zeros((0, w.dk))
        return oracle.mla_attention(q, kv, w.scale, w.kv_lora_rank)
    if len(positions):
        k, v = (oracle.widen_bf16(x) for x in case.rows_at(b, positions))
    else:
        k = v = np.zeros((0, w.kv_heads, w.head_dim))
    return oracle.gqa_attention(q, k, v, w.scale)


def _run_shards(case, q_len, dev):
    """All shards' partials; returns out [N, b*Q, H, dv], lse [N, b*Q, H] (device)."""
    w = case.w
    b, n = w.batch, w.num_shards
    rows = b * q_len
    qbits = case.queries(q_len)
    q_d = bf16_tensor(qbits.reshape(rows, w.heads, w.dk), dev)
    lens = int32_tensor(case.seq_lens, dev)
    mb = case.max_blocks_per_seq()
    po = torch.full((n, rows, w.heads, w.dv), float("nan"), dtype=torch.float32, device=dev)
    pl = torch.full((n, rows, w.heads), float("nan"), dtype=torch.float32, device=dev)
    for r in range(n):
        sc = case.shard(r, max_blocks=mb)
        common = dict(batch=b, block_size=w.block_size, max_blocks_per_seq=mb, num_blocks=sc.num_blocks,
                      shard_rank=r, num_shards=n, layout=w.layout, max_seq_len_hint=max(1, case.max_seq_len),
                      softmax_scale=w.scale, q_len=q_len)
        table = int32_tensor(sc.block_table, dev)
        if w.kind == "mla":
            p = ops.mla_params(num_heads=w.heads, **common)
            ops.dcp_mla_decode_partial(p, q_d, bf16_tensor(sc.pools[0], dev), table, lens, po[r], pl[r],
                                       ops.mla_workspace(p, dev))
        else:
            p = ops.gqa_params(num_q_heads=w.heads, num_kv_heads=w.kv_heads, **common)
            ops.dcp_gqa_decode_partial(p, q_d, bf16_tensor(sc.pools[0], dev), bf16_tensor(sc.pools[1], dev),
                                       table, lens, po[r], pl[r], ops.gqa_workspace(p, dev))
    return qbits, po, pl


CASES = [
    # kind, batch, heads, kv_heads, seq_lens, block, shards, layout, q_len
    ("mla", 3, 64, 1, (1000, 37, 5), 64, 4, 0, 4),
    ("mla", 2, 16, 1, (777, 130), 16, 3, 1, 9),
    ("mla", 2, 64, 1, (2, 300), 64, 8, 0, 2),      # L < N and L = q_len
    ("gqa", 2, 64, 8, (700, 19), 16, 4, 0, 3),
    ("gqa", 1, 32, 4, (513,), 32, 2, 1, 16),
    ("mla", 2, 16, 1, (3, 50), 16, 2, 1, 5),       # L < q_len, contiguous
    ("gqa", 2, 16, 4, (2, 40), 16, 4, 0, 4),       # L < q_len, round-robin
    ("gqa", 2, 8, 1, (700, 19), 16, 2, 0, 3),      # one KV head per rank
    ("gqa", 2, 16, 2, (333, 64), 32, 2, 1, 4),     # two KV heads per rank, contiguous
]


@pytest.mark.parametrize("kind,batch,heads,kvh,lens,block,n,layout,q_len", CASES)
def test_mtp_partials_and_merge(dev, kind, batch, heads, kvh, lens, block, n, layout, q_len):
    _check_mtp(dev, kind, batch, heads, kvh, lens, block, n, layout, q_len)


@pytest.mark.parametrize("wgs", [64, 60])
def test_mtp_xcd_grouped_ranges(dev, monkeypatch, wgs):
    """Multi-token MLA steps whose split width is a multiple of 8 (64) number
    their ranges per XCD; the same results as a split that is not (60)."""
    monkeypatch.setenv("DCP_SPLIT_WGS", str(wgs))
    monkeypatch.setenv("DCP_MLA_MIN_TILES", "1")
    _check_mtp(dev, "mla", 3, 64, 1, (4000, 2500, 700), 64, 2, 0, 3)


def _check_mtp(dev, kind, batch, heads, kvh, lens, block, n, layout, q_len):
    say(f"mtp {kind} b={batch} H={heads} lens={lens} B={block} N={n} layout={layout} q_len={q_len}")
    w = W.custom_workload(kind, batch=batch, heads=heads, kv_heads=kvh, seq_lens=lens, block_size=block,
                          num_shards=n, layout=layout, wid=300 + q_len)
    case = W.Case(w, seed=q_len)
    qbits, po, pl = _run_shards(case, q_len, dev)
    merged = torch.empty((batch * q_len, heads, w.dv), dtype=torch.float32, device=dev)
    mlse = torch.empty((batch * q_len, heads), dtype=torch.float32, device=dev)
    ops.dcp_combine(po, pl, None, merged, mlse)
    torch.cuda.synchronize()
    po_h, pl_h = po.cpu().numpy(), pl.cpu().numpy()
    m_h, ml_h = merged.cpu().numpy(), mlse.cpu().numpy()
    for b in range(batch):
        L = int(case.seq_lens[b])
        for j in range(q_len):
            row = b * q_len + j
            for r in range(n):
                pos = oracle.query_positions(L, q_len, j, n, r, layout)
                o_ref, l_ref = _oracle(case, qbits, b, j, pos)
                assert_rows_close(po_h[r, row], pl_h[r, row], o_ref, l_ref, f"b={b} j={j} r={r}")
            lim = oracle.query_limit(L, q_len, j)
            o_ref, l_ref = _oracle(case, qbits, b, j, np.arange(lim))
            assert_rows_close(m_h[row], ml_h[row], o_ref, l_ref, f"merged b={b} j={j}")


def test_mtp_q_len_one_equals_single_token(dev):
    """q_len = 1 (and the 0 spelling of it) reproduces the single-token call bit for bit."""
    w = W.custom_workload("mla", batch=2, heads=64, seq_lens=(900, 333), block_size=64, num_shards=4, wid=320)
    case = W.Case(w, seed=1)
    outs = []
    for ql in (1, 0):
        sc = case.shard(2, max_blocks=case.max_blocks_per_seq())
        p = ops.mla_params(batch=2, num_heads=64, block_size=64, max_blocks_per_seq=sc.block_table.shape[1],
                           num_blocks=sc.num_blocks, shard_rank=2, num_shards=4, layout=0,
                           max_seq_len_hint=900, softmax_scale=w.scale, q_len=ql)
        out = torch.empty((2, 64, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((2, 64), dtype=torch.float32, device=dev)
        ops.dcp_mla_decode_partial(p, bf16_tensor(case.q, dev), bf16_tensor(sc.pools[0], dev),
                                   int32_tensor(sc.block_table, dev), int32_tensor(case.seq_lens, dev), out, lse,
                                   ops.mla_workspace(p, dev))
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
