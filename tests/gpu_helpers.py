"""Helpers for the GPU parity tests: run the HIP path through the C ABI on seeded
inputs and compare with the fp64 oracle.

The HIP side sees only the paged pools and tables built by ``workloads``; the
oracle side sees only the logical (unsharded) per-request tensors from the same
generator.  Neither side's results feed the other.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as W
from workloads.device import bf16_tensor, fp8_tensor, int32_tensor
from kv_cache_context_amd import ops

# Parity bar: per (request, head) row, max|o - o_ref| / max|o_ref| <= 1e-2
# (fp32 output before the bf16 cast); |lse - lse_ref| <= 1e-3 absolute.
O_TOL = 1e-2
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class ShardRun:
    """Device tensors and results of one shard's partial call."""

    def __init__(self, case: W.Case, r: int, dev, stream=None, max_blocks=None, workspace=None, cache=None):
        w = case.w
        self.case, self.r = case, r
        sc = cache if cache is not None else case.shard(r, max_blocks=max_blocks)
        self.sc = sc
        b = w.batch
        self.seq_lens = int32_tensor(case.seq_lens, dev)
        self.table = int32_tensor(sc.block_table, dev)
        self.q = bf16_tensor(case.q, dev)
        common = dict(block_size=w.block_size, max_blocks_per_seq=sc.block_table.shape[1],
                      num_blocks=sc.num_blocks, shard_rank=r, num_shards=w.num_shards, layout=w.layout,
                      max_seq_len_hint=max(1, case.max_seq_len), softmax_scale=w.scale)
        if w.kind == "mla":
            self.kv = bf16_tensor(sc.pools[0], dev) if case.kv_fp8_scale is None else fp8_tensor(sc.pools[0], dev)
            self.p = ops.mla_params(batch=b, num_heads=w.heads, **common)
            self.ws = workspace if workspace is not None else ops.mla_workspace(self.p, dev)
        else:
            self.k = bf16_tensor(sc.pools[0], dev)
            self.v = bf16_tensor(sc.pools[1], dev)
            self.p = ops.gqa_params(batch=b, num_q_heads=w.heads, num_kv_heads=w.kv_heads, **common)
            self.ws = workspace if workspace is not None else ops.gqa_workspace(self.p, dev)
        self.out = torch.full((b, w.heads, w.dv), float("nan"), dtype=torch.float32, device=dev)
        self.lse = torch.full((b, w.heads), float("nan"), dtype=torch.float32, device=dev)
        self.stream = stream

    def run(self, out=None, lse=None):
        out = self.out if out is None else out
        lse = self.lse if lse is None else lse
        if self.case.w.kind == "mla" and self.case.kv_fp8_scale is not None:
            ops.dcp_mla_decode_partial_fp8(self.p, self.q, self.kv, self.case.kv_fp8_scale, self.table,
                                           self.seq_lens, out, lse, self.ws, self.stream)
        elif self.case.w.kind == "mla":
            ops.dcp_mla_decode_partial(self.p, self.q, self.kv, self.table, self.seq_lens, out, lse, self.ws,
                                       self.stream)
        else:
            ops.dcp_gqa_decode_partial(self.p, self.q, self.k, self.v, self.table, self.seq_lens, out, lse,
                                       self.ws, self.stream)
        return out, lse


def oracle_rows_merged(case: W.Case, b: int, heads):
    """Oracle of the combined result built from the oracle's own shard partials
    and merge (equal to unsharded attention: pinned by the merge invariant);
    used where one request is too long to widen in one piece."""
    w = case.w
    parts = [oracle_rows(case, b, heads, r) for r in range(w.num_shards)]
    return oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))


def oracle_rows(case: W.Case, b: int, heads, r: int | None):
    """Oracle (o, lse) for request b, the given heads, over shard r's slice
    (r=None: the whole sequence)."""
    w = case.w
    L = int(case.seq_lens[b])
    if r is None:
        pos = np.arange(L)
    else:
        pos = oracle.shard_positions(L, w.num_shards, r, w.layout)
    rows = case.rows_at(b, pos) if len(pos) else None
    return oracle_on_rows(case, b, heads, rows)


def oracle_all_shards(case: W.Case, b: int, heads):
    """Oracle (o, lse) of every shard's slice of request b, from one pass over
    the request's stored rows, and (last) the oracle's merge of them, which
    equals unsharded attention (pinned by the merge invariant); the merge avoids
    widening a whole 1M-token request at once."""
    w = case.w
    L = int(case.seq_lens[b])
    logical = case.kv_logical(b)
    if w.kind == "mla":
        logical = [logical]
    res = []
    for r in range(w.num_shards):
        pos = oracle.shard_positions(L, w.num_shards, r, w.layout)
        say(f"    oracle b={b} shard {r}: {len(pos)} positions")
        res.append(oracle_on_rows(case, b, heads, [x[pos] for x in logical] if len(pos) else None))
    res.append(oracle.merge(np.stack([p[0] for p in res]), np.stack([p[1] for p in res])))
    return res


def oracle_on_rows(case: W.Case, b: int, heads, rows):
    """Oracle (o, lse) for request b and the given heads over the stored rows
    ``rows`` (as ``Case.rows_at`` returns them; None: no tokens)."""
    w = case.w
    q = oracle.widen_bf16(case.q[b, heads])
    if w.kind == "mla" and case.kv_fp8_scale is not None:
        bits = rows[0] if rows is not None else np.zeros((0, w.dk), np.uint8)
        return oracle.mla_attention_fp8(q, bits, case.kv_fp8_scale, w.scale, w.kv_lora_rank)
    if w.kind == "mla":
        kv = oracle.widen_bf16(rows[0]) if rows is not None else np.zeros((0, w.dk))
        return oracle.mla_attention(q, kv, w.scale, w.kv_lora_rank)
    k, v = rows if rows is not None else (np.zeros((0, w.kv_heads, w.head_dim), np.uint16),) * 2
    k = oracle.widen_bf16(k)
    v = oracle.widen_bf16(v)
    hq = w.heads
    o = np.zeros((len(heads), w.head_dim))
    lse = np.zeros(len(heads))
    for i, h in enumerate(heads):
        g = (h * w.kv_heads) // hq
        oh, lh = oracle.softmax_attention(q[i:i + 1], k[:, g, :], v[:, g, :], w.scale)
        o[i], lse[i] = oh[0], lh[0]
    return o, lse


def assert_rows_close(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    """Row-wise parity check; returns (worst normwise error, worst lse error)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), f"{what}: empty-slice pattern differs"
    if empty.any():
        assert np.all(o_gpu[empty] == 0.0), f"{what}: empty rows must be zero"
    worst_o = 0.0
    worst_l = 0.0
    if (~empty).any():
        num = np.abs(o_gpu[~empty] - o_ref[~empty]).max(axis=-1)
        den = np.abs(o_ref[~empty]).max(axis=-1)
        rel = num / np.maximum(den, 1e-30)
        worst_o = float(rel.max())
        worst_l = float(np.abs(lse_gpu[~empty] - lse_ref[~empty]).max())
    assert worst_o <= O_TOL, f"{what}: output rel err {worst_o:.3e} > {O_TOL}"
    assert worst_l <= LSE_TOL, f"{what}: lse abs err {worst_l:.3e} > {LSE_TOL}"
    return worst_o, worst_l
