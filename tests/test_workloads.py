"""Seeded input generator: determinism, paged layout, length statistics."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as O


def test_bf16_bits_match_torch():
    r = np.random.default_rng(1)
    x = r.standard_normal(100000).astype(np.float32) * 3
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), ref)
    assert np.array_equal(W.bf16_bits_to_f32(ref).astype(np.float64), O.widen_bf16(ref))


def test_generation_is_deterministic_and_chunk_independent():
    w = W.custom_workload(batch=2, heads=4, seq_lens=(W.CHUNK + 77, 5), num_shards=3)
    a = W.Case(w, seed=3)
    b = W.Case(w, seed=3)
    assert np.array_equal(a.q, b.q)
    full = a.kv_logical(0)
    assert full.shape == (W.CHUNK + 77, 576)
    assert np.array_equal(full[W.CHUNK - 5: W.CHUNK + 9], b.kv_logical(0, W.CHUNK - 5, W.CHUNK + 9))
    pos = [W.CHUNK + 3, 2, W.CHUNK - 1, 0]
    assert np.array_equal(a.rows_at(0, pos)[0], full[pos])
    assert not np.array_equal(W.Case(w, seed=4).q, a.q)


@pytest.mark.parametrize("layout", [W.ROUND_ROBIN, W.CONTIGUOUS])
@pytest.mark.parametrize("kind", ["mla", "gqa"])
def test_pool_gathers_back_to_oracle_slices(layout, kind):
    """Reading each shard's pool through its table gives exactly the tokens the
    oracle assigns to that shard, in order."""
    lens = (1, 3, 17, 64, 65, 200)
    n = 4
    if kind == "mla":
        w = W.custom_workload(kind="mla", batch=len(lens), heads=2, seq_lens=lens, num_shards=n,
                              layout=layout, block_size=16)
    else:
        w = W.custom_workload(kind="gqa", batch=len(lens), heads=8, kv_heads=2, head_dim=16,
                              seq_lens=lens, num_shards=n, layout=layout, block_size=16)
    case = W.Case(w, seed=0)
    seen_blocks = []
    for r in range(n):
        sc = case.shard(r)
        used = []
        for b, L in enumerate(lens):
            idx = O.shard_positions(L, n, r, layout)
            assert sc.local_lens[b] == len(idx)
            j = np.arange(len(idx))
            blk = sc.block_table[b, j // w.block_size]
            used.extend(sorted(set(blk.tolist())))
            logical = case.kv_logical(b)
            logical = (logical,) if kind == "mla" else logical
            for pool, ref in zip(sc.pools, logical):
                assert np.array_equal(pool[blk, j % w.block_size], ref[idx])
        # block ids of one shard are a permutation of its pool
        assert sorted(used) == list(range(len(used))) or len(used) == 0
        seen_blocks.append(len(used))


def test_block_table_is_shuffled():
    case = W.Case(W.WORKLOADS["c0"])
    t, nb = case.block_table(1)
    assert nb == 2 * 4 and sorted(t[:, :4].ravel().tolist()) == list(range(8))
    assert t[:, :4].ravel().tolist() != list(range(8))


def test_bimodal_sampler_statistics():
    L = W.sample_bimodal_lengths(20000, np.random.default_rng(0))
    k = 1024
    assert 0.16 < np.mean(L < 8 * k) < 0.20
    assert 0.45 < np.mean(L < 64 * k) < 0.49
    assert 62 * k < np.median(L) < 72 * k
    assert 0.02 < np.mean(L > 256 * k) < 0.05
    assert L.max() <= 512 * k and L.min() >= k


def test_c2_lengths_fixed_by_seed():
    a = W.Case(W.WORKLOADS["c2"], seed=0).seq_lens
    assert a.shape == (32,) and np.array_equal(a, W.Case(W.WORKLOADS["c2"], seed=0).seq_lens)


def test_workload_shapes():
    w = W.WORKLOADS
    assert (w["c1"].heads, w["c1"].dk, w["c1"].dv, w["c1"].num_shards) == (64, 576, 512, 8)
    assert abs(w["c0"].scale - 192 ** -0.5) < 1e-15 and abs(w["c3"].scale - 128 ** -0.5) < 1e-15
    c3 = W.Case(w["c3"])
    assert c3.max_blocks_per_seq() == 2048 and c3.local_lens(1)[0] == 32768
    c4b = W.Case(w["c4b"])
    assert c4b.local_lens(1).sum() == 128 * 8192
    kv1 = W.Case(w["c3kv1"])
    assert (w["c3kv1"].heads, w["c3kv1"].kv_heads, w["c3kv1"].num_shards) == (8, 1, 2)
    assert kv1.local_lens(1)[0] == 65536 and kv1.max_blocks_per_seq() == 4096


def test_e4m3_encoder_matches_torch():
    """The fp8 cache encoder is torch's float -> float8_e4m3fn rounding (nearest,
    ties to even) on in-range values, clamps beyond 448, and maps every finite
    code's own value back to that code."""
    import torch
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-9, 6, 100000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = W.f32_to_e4m3_bits(x)
    assert np.array_equal(got, ref)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(W.f32_to_e4m3_bits(vals), codes)
    # midpoints between neighbouring codes go to the even code
    mids = (vals[1:0x7E] + vals[2:0x7F]) / 2
    m_codes = W.f32_to_e4m3_bits(mids)
    assert np.all(m_codes % 2 == 0)
    assert W.f32_to_e4m3_bits(np.array([1e4, -1e4, 449.0], np.float32)).tolist() == [0x7E, 0xFE, 0x7E]


def test_fp8_case_quantizes_the_bf16_draws():
    """An fp8 case stores the E4M3 codes of the same normal draws divided by the
    scale; shard pools gather back to the logical codes."""
    w = W.custom_workload("mla", batch=2, heads=16, seq_lens=(300, 77), block_size=16, num_shards=3, wid=77)
    c8 = W.Case(w, seed=4, kv_fp8_scale=0.0125)
    cb = W.Case(w, seed=4)
    lb = W.bf16_bits_to_f32(cb.kv_logical(0))
    l8 = c8.kv_logical(0)
    assert l8.dtype == np.uint8 and l8.shape == (300, 576)
    import torch
    dec = torch.from_numpy(l8).view(torch.float8_e4m3fn).float().numpy() * 0.0125
    # bf16 rounding and fp8 rounding of the same draw: both within their half-ulps
    assert np.all(np.abs(dec - lb) <= np.abs(lb) * (2.0 ** -4 + 2.0 ** -8) + 2.0 ** -10 * 0.0125)
    sc = c8.shard(1)
    assert sc.pools[0].dtype == np.uint8
    pos = list(W.local_positions(300, 3, 1, 0))
    for j, t in enumerate(pos):
        blk = sc.block_table[0, j // 16]
        assert np.array_equal(sc.pools[0][blk, j % 16], l8[t])


def test_e4m3_fast_encoder_equals_grid_search():
    """The bit-level encoder gives the codes of the nearest-value search over
    the code table on every code, every midpoint and its neighbours, clamped
    magnitudes and random draws at the workloads' scale."""
    grid = W._E4M3.astype(np.float32)
    mids = ((grid[1:].astype(np.float64) + grid[:-1]) / 2).astype(np.float32)
    edge = np.concatenate([grid, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           np.array([0.0, 448, 449, 464, 479.9, 480, 1e30, 2.0 ** -6, 2.0 ** -10, 1e-45], np.float32)])
    rng = np.random.default_rng(11)
    for x in (edge, -edge, rng.standard_normal(1 << 21, dtype=np.float32) / np.float32(W.FP8_SCALE),
              rng.standard_normal(1 << 20, dtype=np.float32) * np.float32(0.01)):
        assert np.array_equal(W.f32_to_e4m3_bits(x), W.f32_to_e4m3_bits_grid(x))
