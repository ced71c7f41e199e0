"""Seeded random shapes through the whole path on the GPU against the oracle:
every shard's partial and the combine of all shards, every row, for MLA (bf16
and fp8 caches) and GQA (1 to 16 KV heads per rank, groups of 1 to 64 query
heads), ragged and empty requests, block sizes 16 to 128, 1 to 8 shards, both
layouts and 1 to 4 query tokens per request.  The shapes are drawn once from a
fixed seed, so every run checks the same cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_rows_close, say
from workloads.device import bf16_tensor, fp8_tensor, int32_tensor
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu

GQA_SHAPES = [(8, 1), (16, 2), (64, 1), (24, 3), (32, 4), (48, 6), (64, 8), (64, 16), (128, 2), (12, 12)]


def _draw(i):
    rng = np.random.default_rng([2026, i])
    kind = "mla" if i % 2 == 0 else "gqa"
    batch = int(rng.integers(1, 6))
    lens = [int(x) for x in np.where(rng.random(batch) < 0.3, rng.integers(0, 70, batch),
                                     rng.integers(70, 7000, batch))]
    n = int(rng.integers(1, 9))
    layout = int(rng.integers(0, 2))
    q_len = int(rng.choice([1, 1, 2, 4]))
    bs = int(rng.choice([16, 32, 48, 64, 128]))
    spec = dict(kind=kind, batch=batch, seq_lens=tuple(lens), num_shards=n, layout=layout, block_size=bs)
    fp8 = False
    if kind == "mla":
        spec["heads"] = int(rng.choice([16, 32, 48, 64]))
        fp8 = bool(rng.random() < 0.4) and q_len == 1
    else:
        hq, hkv = GQA_SHAPES[int(rng.integers(0, len(GQA_SHAPES)))]
        spec.update(heads=hq, kv_heads=hkv)
    return spec, q_len, fp8


def _oracle(case, q, b, positions, fp8):
    w = case.w
    if w.kind == "mla":
        if fp8:
            bits = case.rows_at(b, positions)[0] if len(positions) else np.zeros((0, w.dk), np.uint8)
            return oracle.mla_attention_fp8(q, bits, case.kv_fp8_scale, w.scale, w.kv_lora_rank)
        kv = oracle.widen_bf16(case.rows_at(b, positions)[0]) if len(positions) else np.zeros((0, w.dk))
        return oracle.mla_attention(q, kv, w.scale, w.kv_lora_rank)
    if len(positions):
        k, v = (oracle.widen_bf16(x) for x in case.rows_at(b, positions))
    else:
        k = v = np.zeros((0, w.kv_heads, w.head_dim))
    return oracle.gqa_attention(q, k, v, w.scale)


@pytest.mark.parametrize("i", range(48))
def test_random_shape(dev, i):
    spec, q_len, fp8 = _draw(i)
    say(f"random shape {i}: {spec} q_len={q_len} fp8={fp8}")
    w = W.custom_workload(wid=800 + i, **spec)
    case = W.Case(w, seed=i, kv_fp8_scale=W.FP8_SCALE if fp8 else None)
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
            if fp8:
                ops.dcp_mla_decode_partial_fp8(p, q_d, fp8_tensor(sc.pools[0], dev), case.kv_fp8_scale, table, lens,
                                               po[r], pl[r], ops.mla_workspace(p, dev))
            else:
                ops.dcp_mla_decode_partial(p, q_d, bf16_tensor(sc.pools[0], dev), table, lens, po[r], pl[r],
                                           ops.mla_workspace(p, dev))
        else:
            p = ops.gqa_params(num_q_heads=w.heads, num_kv_heads=w.kv_heads, **common)
            ops.dcp_gqa_decode_partial(p, q_d, bf16_tensor(sc.pools[0], dev), bf16_tensor(sc.pools[1], dev),
                                       table, lens, po[r], pl[r], ops.gqa_workspace(p, dev))
    merged = torch.empty((rows, w.heads, w.dv), dtype=torch.float32, device=dev)
    mlse = torch.empty((rows, w.heads), dtype=torch.float32, device=dev)
    ops.dcp_combine(po, pl, None, merged, mlse)
    torch.cuda.synchronize()
    po_h, pl_h, m_h, ml_h = po.cpu().numpy(), pl.cpu().numpy(), merged.cpu().numpy(), mlse.cpu().numpy()
    for bb in range(b):
        L = int(case.seq_lens[bb])
        for j in range(q_len):
            row = bb * q_len + j
            q = oracle.widen_bf16(qbits[bb, j])
            for r in range(n):
                pos = oracle.query_positions(L, q_len, j, n, r, w.layout)
                o_ref, l_ref = _oracle(case, q, bb, pos, fp8)
                assert_rows_close(po_h[r, row], pl_h[r, row], o_ref, l_ref, f"case {i} b={bb} j={j} r={r}")
            o_ref, l_ref = _oracle(case, q, bb, np.arange(oracle.query_limit(L, q_len, j)), fp8)
            assert_rows_close(m_h[row], ml_h[row], o_ref, l_ref, f"case {i} merged b={bb} j={j}")
