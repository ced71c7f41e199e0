"""Pins that tie the fp64 oracle to facts outside itself.

Each ``pin_*`` function takes an implementation (the ``oracle.attention``
module, or a copy of it with a planted mistake) and raises AssertionError if
the implementation disagrees with:

* hand-derived closed forms (``tests/golden/closed_forms.json``);
* closed forms valid at any size (one key, uniform scores, equal keys);
* independent library implementations of the same definition (torch's
  ``scaled_dot_product_attention`` and ``logsumexp`` in float64 on the CPU,
  including its grouped-query mode);
* a 50-digit mpmath evaluation on tiny inputs;
* invariants of the method: merging the N shard partials gives unsharded
  attention for every N and both layouts, N = 1 is the identity, a dropped
  shard gives attention over the surviving tokens, the merge is associative,
  token order does not matter, adding a constant to all scores shifts only the
  LSE (also at magnitudes where an unshifted exp overflows);
* MLA absorbed form equal to explicit per-head up-projection;
* the fp8 cache format: OCP E4M3 code values from the format's published table
  (``tests/golden/fp8_e4m3fn.json``), torch's float8_e4m3fn decoding of all 256
  codes, and the scaling identity of attention over a scaled cache;
* the fused combine epilogue (merge, value up-projection, sigmoid gate):
  a column-selecting projection with a saturated gate returns columns of the
  plain merge, a zero gate halves the projection, and torch's batched fp64
  matmul and sigmoid give the same result.

``tests/test_oracle_mutants.py`` plants mistakes in copies of the oracle and
checks that each one fails at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")
GOLDEN_FP8 = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8_e4m3fn.json")
TIGHT = 1e-12


def _f(x):
    if isinstance(x, str):
        return float(x)
    if isinstance(x, list):
        return [_f(y) for y in x]
    return float(x)


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    inf_a, inf_b = np.isinf(a), np.isinf(b)
    assert np.array_equal(inf_a, inf_b) and np.array_equal(a[inf_a], b[inf_b]), f"{what}: inf pattern"
    fa, fb = a[~inf_a], b[~inf_b]
    assert np.all(np.isfinite(fa)), f"{what}: non-finite values"
    if fa.size:
        err = np.max(np.abs(fa - fb) / np.maximum(1.0, np.abs(fb)))
        assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


def _rng(*key):
    return np.random.default_rng([20260, *key])


# ------------------------------------------------------------------ closed forms

def pin_golden_closed_forms(impl):
    g = json.load(open(GOLDEN))
    for c in g["attention"]:
        o, lse = impl.softmax_attention(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), c["scale"])
        _close(o, c["o"], 1e-14, c["name"])
        _close(lse, _f(c["lse"]), 1e-14, c["name"])
    for c in g["merge"]:
        o, lse = impl.merge(np.array(_f(c["o"])), np.array(_f(c["lse"])))
        _close(o, c["o_merged"], 1e-14, c["name"])
        _close(lse, _f(c["lse_merged"]), 1e-14, c["name"])


def pin_single_key(impl):
    """L = 1: the output is that key's value and the LSE is its score."""
    r = _rng(1)
    for d, dv in ((3, 2), (576, 512), (128, 128)):
        q = r.standard_normal((4, d))
        k = r.standard_normal((1, d))
        v = r.standard_normal((1, dv))
        s = 0.37
        o, lse = impl.softmax_attention(q, k, v, s)
        _close(o, np.repeat(v, 4, axis=0), 1e-13, "L=1 o")
        _close(lse, s * np.array([float(np.dot(q[h], k[0])) for h in range(4)]), 1e-13, "L=1 lse")


def pin_uniform_scores(impl):
    """q = 0: every score is 0, so lse = ln L and o = mean of V."""
    r = _rng(2)
    for L in (1, 2, 5, 64, 1000):
        k = r.standard_normal((L, 8))
        v = r.standard_normal((L, 6))
        o, lse = impl.softmax_attention(np.zeros((3, 8)), k, v, 0.9)
        _close(lse, np.full(3, math.log(L)), 1e-14, "uniform lse")
        _close(o, np.repeat(v.mean(axis=0, keepdims=True), 3, axis=0), 1e-12, "uniform o")


def pin_equal_keys(impl):
    """All keys equal k: lse = s<q,k> + ln L, o = mean of V."""
    r = _rng(3)
    L, d = 37, 10
    q = r.standard_normal((2, d))
    k1 = r.standard_normal(d)
    v = r.standard_normal((L, 4))
    o, lse = impl.softmax_attention(q, np.tile(k1, (L, 1)), v, 0.5)
    _close(lse, 0.5 * (q @ k1) + math.log(L), 1e-13, "equal keys lse")
    _close(o, np.repeat(v.mean(axis=0, keepdims=True), 2, axis=0), 1e-12, "equal keys o")


# ------------------------------------------------------------------ library routines

def _torch_attention(q, k, v, scale, enable_gqa=False):
    import torch
    qt = torch.from_numpy(np.array(q, dtype=np.float64))
    kt = torch.from_numpy(np.array(k, dtype=np.float64))
    vt = torch.from_numpy(np.array(v, dtype=np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=enable_gqa)
    return o.numpy()


def pin_torch_sdpa(impl):
    """Generic attention equals torch SDPA (fp64, CPU); LSE equals torch.logsumexp."""
    import torch
    r = _rng(4)
    for H, L, d, dv in ((1, 1, 4, 4), (4, 7, 16, 8), (3, 300, 64, 32), (2, 129, 576, 512)):
        q = r.standard_normal((H, d))
        k = r.standard_normal((L, d))
        v = r.standard_normal((L, dv))
        s = 1.0 / math.sqrt(d)
        o, lse = impl.softmax_attention(q, k, v, s)
        o_ref = _torch_attention(q[None, :, None, :], np.broadcast_to(k, (H, L, d))[None],
                                 np.broadcast_to(v, (H, L, dv))[None], s)[0, :, 0, :]
        _close(o, o_ref, 1e-12, "sdpa o")
        z = torch.from_numpy(q) @ torch.from_numpy(k).T * s
        _close(lse, torch.logsumexp(z, dim=1).numpy(), 1e-12, "logsumexp")


def pin_gqa_torch(impl):
    """GQA equals torch SDPA with grouped-query broadcasting (consecutive groups)."""
    import torch
    r = _rng(5)
    for hq, hkv, L, d in ((8, 2, 33, 16), (64, 8, 70, 128), (6, 3, 5, 8), (4, 4, 9, 8), (4, 1, 9, 8)):
        q = r.standard_normal((hq, d))
        k = r.standard_normal((L, hkv, d))
        v = r.standard_normal((L, hkv, d))
        s = 1.0 / math.sqrt(d)
        o, lse = impl.gqa_attention(q, k, v, s)
        o_ref = _torch_attention(q[None, :, None, :], np.transpose(k, (1, 0, 2))[None],
                                 np.transpose(v, (1, 0, 2))[None], s, enable_gqa=True)[0, :, 0, :]
        _close(o, o_ref, 1e-12, "gqa o")
        kk = torch.from_numpy(np.ascontiguousarray(np.transpose(k, (1, 0, 2))))
        kk = kk.repeat_interleave(hq // hkv, dim=0)          # [hq, L, d]
        z = torch.einsum("hd,hld->hl", torch.from_numpy(q), kk) * s
        _close(lse, torch.logsumexp(z, dim=1).numpy(), 1e-12, "gqa lse")


def pin_mpmath(impl):
    """50-digit evaluation of the definition on tiny inputs."""
    import mpmath as mp
    mp.mp.dps = 50
    r = _rng(6)
    for H, L, d, dv in ((1, 1, 2, 1), (2, 3, 3, 2), (2, 6, 5, 3)):
        q = r.standard_normal((H, d))
        k = r.standard_normal((L, d))
        v = r.standard_normal((L, dv))
        s = 0.61
        o, lse = impl.softmax_attention(q, k, v, s)
        for h in range(H):
            z = [mp.mpf(s) * mp.fsum(mp.mpf(q[h, i]) * mp.mpf(k[t, i]) for i in range(d)) for t in range(L)]
            lse_ref = mp.log(mp.fsum(mp.exp(zt) for zt in z))
            assert abs(lse[h] - float(lse_ref)) <= 1e-13 * max(1, abs(float(lse_ref))), "mpmath lse"
            for j in range(dv):
                oj = mp.fsum(mp.exp(z[t] - lse_ref) * mp.mpf(v[t, j]) for t in range(L))
                assert abs(o[h, j] - float(oj)) <= 1e-13 * max(1, abs(float(oj))), "mpmath o"


# ------------------------------------------------------------------ invariants

def _mla_case(r, H, L, R=24, P=8):
    return r.standard_normal((H, R + P)), r.standard_normal((L, R + P))


def pin_merge_equals_unsharded(impl):
    """merge(shard partials) == unsharded attention, every N, both layouts."""
    r = _rng(7)
    for layout in (0, 1):
        for L in (1, 2, 5, 16, 33, 100):
            q, kv = _mla_case(r, 3, L)
            o_ref, lse_ref = impl.mla_attention(q, kv, 0.3, kv_lora_rank=24)
            for n in (1, 2, 3, 4, 7, 8, 16, L + 3):
                parts = [impl.mla_shard_partial(q, kv, 0.3, n, rr, layout, kv_lora_rank=24) for rr in range(n)]
                o, lse = impl.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
                _close(o, o_ref, 1e-12, f"merge o L={L} N={n} layout={layout}")
                _close(lse, lse_ref, 1e-12, f"merge lse L={L} N={n} layout={layout}")
                # every position is held by exactly one shard
                pos = np.concatenate([impl.shard_positions(L, n, rr, layout) for rr in range(n)])
                assert np.array_equal(np.sort(pos), np.arange(L)), "shards do not partition the sequence"
        # GQA too
        hq, hkv, L, d = 8, 2, 29, 8
        q = r.standard_normal((hq, d))
        k = r.standard_normal((L, hkv, d))
        v = r.standard_normal((L, hkv, d))
        o_ref, lse_ref = impl.gqa_attention(q, k, v, 0.4)
        for n in (1, 2, 4, 5, 40):
            parts = [impl.gqa_shard_partial(q, k, v, 0.4, n, rr, layout) for rr in range(n)]
            o, lse = impl.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            _close(o, o_ref, 1e-12, "gqa merge o")
            _close(lse, lse_ref, 1e-12, "gqa merge lse")


def pin_round_robin_layout(impl):
    """Round-robin: shard r holds t = r, r+N, r+2N, ... (in that order)."""
    for L, n in ((10, 3), (7, 8), (64, 8)):
        for rr in range(n):
            assert list(impl.shard_positions(L, n, rr, 0)) == list(range(rr, L, n))
    # contiguous: consecutive runs of ceil(L/N)
    assert [list(impl.shard_positions(10, 4, rr, 1)) for rr in range(4)] == \
        [[0, 1, 2], [3, 4, 5], [6, 7, 8], [9]]


def pin_merge_identity(impl):
    """N = 1: the merge returns its single partial exactly."""
    r = _rng(8)
    o1 = r.standard_normal((1, 3, 5, 7))
    l1 = r.standard_normal((1, 3, 5)) * 10
    o, lse = impl.merge(o1, l1)
    assert np.array_equal(o, o1[0]) and np.array_equal(lse, l1[0]), "N=1 merge is not the identity"


def pin_shift_invariance(impl):
    """Adding c to every score moves the LSE by c and leaves o unchanged."""
    r = _rng(9)
    L, d = 50, 6
    q = r.standard_normal((2, d))
    k = r.standard_normal((L, d))
    v = r.standard_normal((L, 3))
    o0, l0 = impl.softmax_attention(q, k, v, 1.0)
    for c in (-3.0, 7.5, 1.0e4, -1.0e4):
        # an extra coordinate with q = c and k = 1 adds c to each score
        qx = np.concatenate([q, np.full((2, 1), c)], axis=1)
        kx = np.concatenate([k, np.ones((L, 1))], axis=1)
        o, lse = impl.softmax_attention(qx, kx, v, 1.0)
        _close(o, o0, 1e-11, f"shift o c={c}")
        _close(lse - c, l0, 1e-11 * max(1.0, abs(c)), f"shift lse c={c}")


def pin_dropped_shard(impl):
    """A shard whose LSE is -inf drops out: exact attention over the rest."""
    r = _rng(10)
    L, n = 40, 4
    q, kv = _mla_case(r, 2, L)
    parts = [impl.mla_shard_partial(q, kv, 0.25, n, rr, 0, kv_lora_rank=24) for rr in range(n)]
    os_ = np.stack([p[0] for p in parts])
    ls = np.stack([p[1] for p in parts])
    for drop in range(n):
        ls2 = ls.copy()
        ls2[drop] = -np.inf
        o, lse = impl.merge(os_, ls2)
        keep = np.array([t for t in range(L) if t % n != drop])
        o_ref, lse_ref = impl.mla_attention(q, kv[keep], 0.25, kv_lora_rank=24)
        _close(o, o_ref, 1e-12, "dropped o")
        _close(lse, lse_ref, 1e-12, "dropped lse")


def pin_associativity(impl):
    """merge(merge(A,B),C) == merge(A,merge(B,C)) == merge(A,B,C)."""
    r = _rng(11)
    o = r.standard_normal((3, 4, 6))
    lse = r.standard_normal((3, 4)) * 5
    lse[1, 2] = -np.inf
    ab = impl.merge(o[:2], lse[:2])
    left = impl.merge(np.stack([ab[0], o[2]]), np.stack([ab[1], lse[2]]))
    bc = impl.merge(o[1:], lse[1:])
    right = impl.merge(np.stack([o[0], bc[0]]), np.stack([lse[0], bc[1]]))
    flat = impl.merge(o, lse)
    for x in (left, right):
        _close(x[0], flat[0], 1e-13, "assoc o")
        _close(x[1], flat[1], 1e-13, "assoc lse")


def pin_permutation(impl):
    """Token order does not change the result."""
    r = _rng(12)
    q, kv = _mla_case(r, 3, 45)
    o, lse = impl.mla_attention(q, kv, 0.2, kv_lora_rank=24)
    p = r.permutation(45)
    o2, lse2 = impl.mla_attention(q, kv[p], 0.2, kv_lora_rank=24)
    _close(o2, o, 1e-13, "perm o")
    _close(lse2, lse, 1e-13, "perm lse")


def pin_absorbed_equals_unabsorbed(impl):
    """MLA absorbed form == explicit up-projection of the latent per head.

    Unabsorbed: per head h, key = [c_kv W_UK[h] | k_rope], query = [q_nope_h | q_rope_h],
    value = c_kv W_UV[h]; standard attention (torch SDPA, fp64).  Absorbed: the
    query becomes [W_UK[h] q_nope_h | q_rope_h] against the latent row
    [c_kv | k_rope], the value is c_kv, and W_UV[h] is applied afterwards.
    """
    r = _rng(13)
    H, L, R, P, dn, dv = 4, 23, 16, 4, 6, 5
    c_kv = r.standard_normal((L, R))
    k_rope = r.standard_normal((L, P))
    w_uk = r.standard_normal((H, R, dn)) / math.sqrt(R)
    w_uv = r.standard_normal((H, R, dv)) / math.sqrt(R)
    q_nope = r.standard_normal((H, dn))
    q_rope = r.standard_normal((H, P))
    s = 1.0 / math.sqrt(dn + P)
    # explicit per-head keys/values
    keys = np.stack([np.concatenate([c_kv @ w_uk[h], k_rope], axis=1) for h in range(H)])   # [H, L, dn+P]
    vals = np.stack([c_kv @ w_uv[h] for h in range(H)])                                      # [H, L, dv]
    qs = np.concatenate([q_nope, q_rope], axis=1)[:, None, :]                               # [H, 1, dn+P]
    o_ref = _torch_attention(qs[None], keys[None], vals[None], s)[0, :, 0, :]
    # absorbed
    q_abs = np.stack([np.concatenate([w_uk[h] @ q_nope[h], q_rope[h]]) for h in range(H)])  # [H, R+P]
    latent = np.concatenate([c_kv, k_rope], axis=1)
    o_lat, _ = impl.mla_attention(q_abs, latent, s, kv_lora_rank=R)
    o_abs = np.stack([o_lat[h] @ w_uv[h] for h in range(H)])
    _close(o_abs, o_ref, 1e-12, "absorbed vs unabsorbed")


def pin_bf16_cast(impl):
    """fp32 -> bf16 round-to-nearest-even equals torch's conversion."""
    import torch
    r = _rng(14)
    x = (r.standard_normal(200000) * np.exp(r.uniform(-20, 20, 200000))).astype(np.float32)
    # exact ties, both parities, and a few specials
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x7F7FFFFF, 0x00008000, 0x00018000],
                    dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = impl.bf16_rne_bits(x)
    assert np.array_equal(got, ref), "bf16 RNE bits differ from torch"
    # widening is exact
    w = impl.widen_bf16(ref)
    assert np.array_equal(w, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def pin_fp8_table(impl):
    """E4M3 codes decode to the values of the format's published table."""
    for c in json.load(open(GOLDEN_FP8))["codes"]:
        got = float(impl.decode_e4m3fn(np.array([int(c["code"], 16)], np.uint8))[0])
        want = float(c["value"])
        if math.isnan(want):
            assert math.isnan(got), c
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), (c, got)


def pin_fp8_torch(impl):
    """All 256 codes decode as torch's float8_e4m3fn does (NaN at the same codes),
    and the positive finite codes are strictly increasing."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = impl.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert np.all(np.diff(got[:0x7F]) > 0)


def pin_fp8_attention_scale(impl):
    """Attention over an fp8 cache with dequantization scale s: scores see
    s * K, values s * V, so o = s * o' and lse = lse' where (o', lse') is
    attention over the decoded codes with the softmax scale multiplied by s."""
    r = _rng(45)
    H, L, R, P = 5, 23, 24, 8
    q = r.standard_normal((H, R + P))
    bits = r.integers(0, 256, size=(L, R + P)).astype(np.uint8)
    bits[(bits & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    for s in (1.0, 0.0125, 3.5):
        o, lse = impl.mla_attention_fp8(q, bits, s, 0.3, R)
        dec = impl.decode_e4m3fn(bits)
        o2, lse2 = impl.mla_attention(q, dec, 0.3 * s, R)
        _close(o, s * o2, what=f"fp8 scale {s} o")
        _close(lse, lse2, what=f"fp8 scale {s} lse")
    # and against the plain route on explicitly dequantized rows
    o3, lse3 = impl.softmax_attention(q, 0.0125 * dec, 0.0125 * dec[:, :R], 0.3)
    o4, lse4 = impl.mla_attention_fp8(q, bits, 0.0125, 0.3, R)
    _close(o4, o3, what="fp8 plain o")
    _close(lse4, lse3, what="fp8 plain lse")


def _vproj_case(r, N=3, b=4, H=3, Dv=20, Dvo=6):
    o = r.standard_normal((N, b, H, Dv))
    lse = r.standard_normal((N, b, H)) * 2.0
    lse[0, 1, 2] = -np.inf
    lse[:, 3, 0] = -np.inf  # an all-empty row
    w = r.standard_normal((H, Dvo, Dv))
    g = r.standard_normal((b, H, Dvo))
    return o, lse, w, g


def pin_vproj_selection(impl):
    """Projection rows that pick latent columns, gate logits of 60 (sigmoid is
    1 to 1e-26): the result is those columns of the plain merge, per head."""
    r = _rng(41)
    o, lse, _, _ = _vproj_case(r)
    N, b, H, Dv = o.shape
    cols = [[3, 0, 19, 7, 7, 11], [1, 2, 3, 4, 5, 6], [19, 18, 0, 1, 10, 9]]
    w = np.zeros((H, 6, Dv))
    for h in range(H):
        for n, c in enumerate(cols[h]):
            w[h, n, c] = 1.0
    y, lse2 = impl.combine_vproj_gate(o, lse, w, np.full((b, H, 6), 60.0))
    om, lm = impl.merge(o, lse)
    _close(lse2, lm, what="vproj lse")
    for h in range(H):
        _close(y[:, h, :], om[:, h, cols[h]], what=f"vproj selection head {h}")


def pin_vproj_gate_half(impl):
    """Zero gate logits halve the projection; a gate logit g scales by 1/(1+e^-g)."""
    r = _rng(42)
    o, lse, w, _ = _vproj_case(r)
    b, H, Dvo = o.shape[1], o.shape[2], w.shape[1]
    y0, _ = impl.combine_vproj_gate(o, lse, w, np.zeros((b, H, Dvo)))
    y1, _ = impl.combine_vproj_gate(o, lse, w, np.full((b, H, Dvo), 60.0))
    _close(y0, 0.5 * y1, what="zero gate")
    ym, _ = impl.combine_vproj_gate(o, lse, w, np.full((b, H, Dvo), -math.log(3.0)))
    _close(ym, 0.25 * y1, what="gate logit -ln 3")


def pin_vproj_torch(impl):
    """torch fp64: bmm over heads of the merged latent with the transposed
    projection, times torch.sigmoid of the gate."""
    import torch
    r = _rng(43)
    o, lse, w, g = _vproj_case(r)
    om, _ = impl.merge(o, lse)
    ot = torch.from_numpy(np.ascontiguousarray(om.transpose(1, 0, 2)))           # [H, b, Dv]
    wt = torch.from_numpy(np.ascontiguousarray(w.transpose(0, 2, 1)))            # [H, Dv, Dvo]
    ref = torch.bmm(ot, wt).numpy().transpose(1, 0, 2) * torch.sigmoid(torch.from_numpy(g)).numpy()
    y, _ = impl.combine_vproj_gate(o, lse, w, g)
    _close(y, ref, tol=1e-11, what="vproj vs torch")


def pin_query_positions(impl):
    """Multi-token steps: for every query token, the shards' attended positions
    are disjoint and together are exactly the causal prefix 0 .. L - q_len + j
    (enumerated by brute force), for both layouts; q_len = 1 is the whole cache."""
    for L in (1, 2, 5, 17, 64, 100):
        for n in (1, 2, 3, 8):
            for layout in (0, 1):
                assert np.array_equal(np.sort(np.concatenate([impl.query_positions(L, 1, 0, n, r, layout)
                                                              for r in range(n)])), np.arange(L))
                for q_len in (2, 3, 9):
                    for j in range(q_len):
                        want = [t for t in range(L) if t <= L - q_len + j]
                        parts = [impl.query_positions(L, q_len, j, n, r, layout) for r in range(n)]
                        got = np.sort(np.concatenate(parts))
                        assert got.tolist() == want, (L, n, layout, q_len, j)
                        assert sum(len(p) for p in parts) == len(want)
                        # and each shard's part lies inside that shard's slice of the cache
                        for r in range(n):
                            assert set(parts[r].tolist()) <= set(impl.shard_positions(L, n, r, layout).tolist())


def pin_query_merge(impl):
    """Merging the shards' per-query partials gives attention over that query's
    causal prefix, for each query token of a 3-token step."""
    r_ = _rng(44)
    q, kv = _mla_case(r_, 3, 29)
    L, q_len, n = 29, 3, 4
    for layout in (0, 1):
        for j in range(q_len):
            lim = impl.query_limit(L, q_len, j)
            o_ref, lse_ref = impl.mla_attention(q, kv[:lim], 0.4, 24)
            parts = [impl.mla_attention(q, kv[impl.query_positions(L, q_len, j, n, r, layout)], 0.4, 24)
                     for r in range(n)]
            o, lse = impl.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            _close(o, o_ref, what="query merge o")
            _close(lse, lse_ref, what="query merge lse")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
