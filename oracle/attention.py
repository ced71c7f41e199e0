"""fp64 reference arithmetic for DCP decode attention (test infrastructure only).

Plain numpy, float64 throughout, no blocking or fusion.  Sources of each step
are given per function; all refer to the vLLM blog post on Decode Context
Parallelism (DCP) unless stated otherwise.

Readings taken where the post is silent (each one is also listed in the design
notes):
* the LSE is the natural log of the sum of exp of the scaled scores, and
  partial outputs are normalized by their own softmax sum;
* an empty local slice yields (o = 0, lse = -inf), which the merge treats as
  the identity;
* MLA works in absorbed latent space: score over [c_kv | k_rope], value c_kv;
* GQA query head h reads KV head floor(h * Hkv / Hq).
"""
from __future__ import annotations

import numpy as np

ROUND_ROBIN = 0
CONTIGUOUS = 1


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of one query per head over L keys.

    q [H, Dk], k [L, Dk], v [L, Dv] (float64).  Returns (o [H, Dv], lse [H]):
      z[h, t] = scale * <q_h, k_t>
      lse[h]  = log(sum_t exp(z[h, t]))          (natural log)
      o[h]    = sum_t exp(z[h, t] - lse[h]) * v_t
    Computed with the usual max shift so large scores do not overflow.
    With L = 0 the result is (0, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    H = q.shape[0]
    L = k.shape[0]
    if L == 0:
        return np.zeros((H, v.shape[1])), np.full(H, -np.inf)
    z = scale * (q @ k.T)                       # [H, L]
    m = z.max(axis=1)                           # [H]
    e = np.exp(z - m[:, None])                  # [H, L]
    s = e.sum(axis=1)                           # [H]
    o = (e @ v) / s[:, None]                    # [H, Dv]
    lse = m + np.log(s)
    return o, lse


def mla_attention(q: np.ndarray, kv: np.ndarray, scale: float, kv_lora_rank: int = 512):
    """MLA decode attention in absorbed form (section 5.3 "MLA Backend").

    q [H, R + P] absorbed queries, kv [L, R + P] latent rows [c_kv | k_rope].
    Keys are the whole latent row; values are c_kv = kv[:, :R].  All H heads
    read the same latent rows (one effective KV head).
    """
    kv = np.asarray(kv, dtype=np.float64)
    return softmax_attention(q, kv, kv[:, :kv_lora_rank], scale)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """GQA decode attention (section 5.4 "GQA Backend").

    q [Hq, D], k and v [L, Hkv, D].  KV head g serves the consecutive query heads
    h with floor(h * Hkv / Hq) = g.
    """
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    hkv = k.shape[1]
    o = np.zeros((hq, v.shape[2]))
    lse = np.zeros(hq)
    for h in range(hq):
        g = (h * hkv) // hq
        oh, lh = softmax_attention(q[h:h + 1], k[:, g, :], v[:, g, :], scale)
        o[h] = oh[0]
        lse[h] = lh[0]
    return o, lse


def decode_e4m3fn(bits) -> np.ndarray:
    """8-bit float codes of the OCP E4M3 format ("e4m3fn") -> exact float64.

    Bit 7 is the sign, bits 6..3 the exponent E (bias 7), bits 2..0 the
    mantissa M.  E = 0 encodes subnormals M/8 * 2^-6; otherwise the value is
    (1 + M/8) * 2^(E - 7).  The code with E = 15 and M = 7 (either sign) is
    NaN; the format has no infinities, so its largest finite magnitude is
    1.75 * 2^8 = 448.  This is the fp8 KV-cache format read here (the Kimi K3
    optimizations page runs its cache in fp8; the pages fix no encoding).
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where((b >> 7) == 1, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (b & 7 == 7), np.nan, mag)
    return sign * mag


def mla_attention_fp8(q: np.ndarray, kv_bits: np.ndarray, kv_scale: float, scale: float,
                      kv_lora_rank: int = 512):
    """MLA decode attention over an fp8 latent cache with one dequantization
    scale for the whole cache: each stored latent row stands for
    kv_scale * decode_e4m3fn(row), used as both key (all 576) and value (first
    512) exactly as in ``mla_attention``."""
    kv = float(kv_scale) * decode_e4m3fn(kv_bits)
    return mla_attention(q, kv, scale, kv_lora_rank)


def shard_positions(L: int, n: int, r: int, layout: int = ROUND_ROBIN) -> np.ndarray:
    """Global token positions held by shard r of n (section 4 "What is DCP?").

    Round-robin: positions t with t mod n == r.  Contiguous: the r-th run of
    ceil(L / n) consecutive positions (the post's 4-GPU example splits a long
    request into equal consecutive ranges).
    """
    t = np.arange(L)
    if layout == ROUND_ROBIN:
        return t[t % n == r]
    c = -(-L // n)
    return t[(t >= r * c) & (t < (r + 1) * c)]


def query_limit(L: int, q_len: int, j: int) -> int:
    """Number of leading cache positions query token j of a q_len-token decode
    step attends (multi-token decode for speculative verification, DCP post
    section 6 "Future Work"): the cache holds L positions whose last q_len are
    the step's own tokens, and token j sees the positions before it and itself,
    i.e. t <= L - q_len + j.  Clamped at 0."""
    return max(0, L - q_len + 1 + j)


def query_positions(L: int, q_len: int, j: int, n: int, r: int, layout: int = ROUND_ROBIN) -> np.ndarray:
    """Shard r's positions attended by query token j: the shard's part of the
    cache of length L (the sharding is a property of the cache, so the
    contiguous layout cuts by ceil(L / n)) below query j's causal limit."""
    t = shard_positions(L, n, r, layout)
    return t[t < query_limit(L, q_len, j)]


def mla_shard_partial(q, kv_full, scale, n, r, layout=ROUND_ROBIN, kv_lora_rank=512):
    """Shard r's partial (o, lse): MLA attention over its local slice only."""
    idx = shard_positions(kv_full.shape[0], n, r, layout)
    return mla_attention(q, np.asarray(kv_full, dtype=np.float64)[idx], scale, kv_lora_rank)


def gqa_shard_partial(q, k_full, v_full, scale, n, r, layout=ROUND_ROBIN):
    idx = shard_positions(k_full.shape[0], n, r, layout)
    return gqa_attention(q, np.asarray(k_full, dtype=np.float64)[idx],
                         np.asarray(v_full, dtype=np.float64)[idx], scale)


def merge(o_parts, lse_parts):
    """LSE-weighted merge of N partials into the exact result (section 4.1).

    o_parts [N, ..., Dv], lse_parts [N, ...].  With M = max_i lse_i:
      lse = M + log(sum_i exp(lse_i - M))
      o   = sum_i exp(lse_i - lse) * o_i
    If every lse_i is -inf the result is (0, -inf).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])                 # exp(-inf) = 0
    s = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, s)))
    wn = np.where(empty[None], 0.0, w / np.where(empty, 1.0, s)[None])
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse


def combine_vproj_gate(o_parts, lse_parts, w_uv_t, gate):
    """DCP merge followed by the per-head value up-projection and a sigmoid
    output gate, the epilogue that the Kimi K3 GB300 decode page fuses into its
    combine kernel (DCP partials combined together with v-proj and gating).

    o_parts [N, b, H, Dv] latent partials and lse_parts [N, b, H] as for
    ``merge``; w_uv_t [H, Dvo, Dv] holds each head's up-projection with the
    latent index last (row n of head h maps the latent vector to output
    column n); gate [b, H, Dvo] holds gate logits.  Returns (y [b, H, Dvo],
    lse [b, H]) with
      o = merge(o_parts, lse_parts)[0]
      y[b, h, n] = sigmoid(gate[b, h, n]) * sum_k o[b, h, k] * w_uv_t[h, n, k].
    """
    o, lse = merge(o_parts, lse_parts)
    w = np.asarray(w_uv_t, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    y = np.empty(g.shape)
    for h in range(w.shape[0]):
        y[:, h, :] = o[:, h, :] @ w[h].T
    sig = 1.0 / (1.0 + np.exp(-g))
    return sig * y, lse


def bf16_rne_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    Works on the float32 value itself: the bf16 neighbours below and above are
    found by truncating the low 16 bits, and the nearer one is taken; on an
    exact tie the one with an even last bit is taken.  Infinities pass through.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lo = (bits & np.uint32(0xFFFF0000))            # truncation toward zero (in magnitude)
    rem = bits & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    up = (rem > half) | ((rem == half) & (((lo >> np.uint32(16)) & np.uint32(1)) == 1))
    res = (lo >> np.uint32(16)) + up.astype(np.uint32)
    res = np.where(np.isinf(x), bits >> np.uint32(16), res)
    return res.astype(np.uint16)


def bf16_rne(x) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned widened to float64."""
    return widen_bf16(bf16_rne_bits(x))
