"""Plant mistakes in copies of the oracle; each must fail at least one pin.

Every mutant is a textual edit of ``oracle/attention.py`` (a dropped term, a
wrong sign, index or operand), executed as a fresh module on the CPU.  The
real oracle is never modified.
"""
import os
import types

import pytest

from tests import oracle_pins

SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "attention.py")).read()

MUTANTS = {
    "no max shift": ("e = np.exp(z - m[:, None])", "e = np.exp(z)"),
    "lse drops max": ("lse = m + np.log(s)", "lse = np.log(s)"),
    "lse base 2": ("lse = m + np.log(s)", "lse = m + np.log2(s)"),
    "unnormalized o": ("o = (e @ v) / s[:, None]", "o = (e @ v)"),
    "scale on sqrt": ("z = scale * (q @ k.T)", "z = np.sqrt(scale) * (q @ k.T)"),
    "reversed values": ("o = (e @ v) / s[:, None]", "o = (e @ v[::-1]) / s[:, None]"),
    "MLA value = last 512": ("return softmax_attention(q, kv, kv[:, :kv_lora_rank], scale)",
                             "return softmax_attention(q, kv, kv[:, -kv_lora_rank:], scale)"),
    "MLA key = c_kv only": ("return softmax_attention(q, kv, kv[:, :kv_lora_rank], scale)",
                            "return softmax_attention(q[:, :kv_lora_rank], kv[:, :kv_lora_rank], kv[:, :kv_lora_rank], scale)"),
    "GQA interleaved heads": ("g = (h * hkv) // hq", "g = h % hkv"),
    "round-robin by quotient": ("return t[t % n == r]", "return t[t // n == r]"),
    "contiguous floor": ("c = -(-L // n)\n    return t[(t >= r * c)", "c = L // n\n    return t[(t >= r * c)"),
    "merge unnormalized weights": ("wn = np.where(empty[None], 0.0, w / np.where(empty, 1.0, s)[None])",
                                   "wn = np.where(empty[None], 0.0, w)"),
    "merge lse drops log": ("m_safe + np.log(np.where(empty, 1.0, s))", "m_safe + np.where(empty, 1.0, s)"),
    "merge weight sign": ("w = np.exp(lse_parts - m_safe[None])", "w = np.exp(m_safe[None] - lse_parts)"),
    "merge mean": ("o = (wn[..., None] * o_parts).sum(axis=0)", "o = o_parts.mean(axis=0)"),
    "merge all-empty lse 0": ("lse = np.where(empty, -np.inf, m_safe", "lse = np.where(empty, 0.0, m_safe"),
    "bf16 truncates": ("res = (lo >> np.uint32(16)) + up.astype(np.uint32)", "res = (lo >> np.uint32(16))"),
    "bf16 ties away": ("up = (rem > half) | ((rem == half) & (((lo >> np.uint32(16)) & np.uint32(1)) == 1))",
                       "up = (rem >= half)"),
    "widen shift 8": ("b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
                      "b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(8)"),
    "empty slice lse 0": ("return np.zeros((H, v.shape[1])), np.full(H, -np.inf)",
                          "return np.zeros((H, v.shape[1])), np.zeros(H)"),
    "vproj untransposed": ("y[:, h, :] = o[:, h, :] @ w[h].T", "y[:, h, :] = (o[:, h, :] @ w[h].T[::-1])[:, ::-1]"),
    "vproj wrong head": ("y[:, h, :] = o[:, h, :] @ w[h].T", "y[:, h, :] = o[:, h, :] @ w[(h + 1) % w.shape[0]].T"),
    "gate sign": ("sig = 1.0 / (1.0 + np.exp(-g))", "sig = 1.0 / (1.0 + np.exp(g))"),
    "gate missing": ("return sig * y, lse", "return y, lse"),
    "fp8 exponent bias 8": ("(1.0 + m / 8.0) * np.exp2(e - 7.0)", "(1.0 + m / 8.0) * np.exp2(e - 8.0)"),
    "fp8 subnormals as normals": ("mag = np.where(e == 0, m / 8.0 * 2.0 ** -6,", "mag = np.where(e == -1, m / 8.0 * 2.0 ** -6,"),
    "fp8 sign dropped": ("sign = np.where((b >> 7) == 1, -1.0, 1.0)", "sign = 1.0"),
    "fp8 NaN code as a number": ("mag = np.where((e == 15) & (b & 7 == 7), np.nan, mag)", "pass"),
    "fp8 scale on scores only": ("    kv = float(kv_scale) * decode_e4m3fn(kv_bits)\n    return mla_attention(q, kv, scale, kv_lora_rank)",
                                 "    return mla_attention(q, decode_e4m3fn(kv_bits), scale * kv_scale, kv_lora_rank)"),
    "fp8 scale ignored": ("    kv = float(kv_scale) * decode_e4m3fn(kv_bits)", "    kv = decode_e4m3fn(kv_bits)"),
    "query limit excludes itself": ("return max(0, L - q_len + 1 + j)", "return max(0, L - q_len + j)"),
    "query limit from the front": ("return max(0, L - q_len + 1 + j)", "return max(0, min(L, q_len + j))"),
    "query positions re-sharded by prefix": ("    t = shard_positions(L, n, r, layout)\n    return t[t < query_limit(L, q_len, j)]",
                                            "    return shard_positions(query_limit(L, q_len, j), n, r, layout)"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash caused by the mistake
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name!r} passes every pin"
