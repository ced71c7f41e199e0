"""Seeded synthetic inputs for shard-local decode attention.

This module is shared by the oracle side and the HIP side of the tests and the
benchmark.  It only *draws and lays out* inputs; it holds none of the attention,
softmax or merge arithmetic.

What it produces, per workload:

* queries ``q``: bf16 bit patterns (uint16), ``[batch][heads][dk]``;
* per-request global context lengths ``seq_lens`` (int32);
* for every shard rank ``r`` a paged cache holding that shard's local slice of
  each request's tokens, plus a shuffled block table that maps local block
  index -> physical block id in that shard's pool.

The sequence split is the one the decode-context-parallel design uses (vLLM
blog post on Decode Context Parallelism, section "What is DCP?": each rank keeps
the cache of its own subset of one sequence's token positions).  Two layouts are
supported: round-robin (token t lives on rank t mod N, local index t div N)
and contiguous (rank r holds positions [r*C, (r+1)*C) with C = ceil(L/N), the
example given in that section).

Input recipe (all values are standard normal draws rounded to bf16):

* every tensor is drawn from ``numpy.random.default_rng(key)`` (PCG64) where
  ``key = [seed, workload_id, tensor_id, request, chunk]``; draws are float32
  (``Generator.standard_normal(dtype=float32)``) rounded to bf16 with
  round-to-nearest-even.  The bf16 bit patterns are the ground truth that both
  sides read.
* the K/V of one request is drawn in chunks of ``CHUNK`` global token
  positions, so any request, any token range and any shard can be regenerated
  independently and in parallel.
* block tables: shard r's blocks are numbered 0..nb-1 in request order and then
  relabelled by ``rng.permutation(nb)`` keyed ``[seed, workload_id, PERM, r]``.
  Table entries past a request's last local block hold 0 (a valid block that
  belongs to some other request, so a stray read shows up as a wrong result).
* fp8 caches (MLA): the same float32 draws divided by the cache's
  dequantization scale and rounded to the nearest OCP E4M3 code (ties to the
  even code, magnitudes clamped to 448); the uint8 codes are the ground truth.
* the ragged-length workload draws lengths from a bimodal mixture shaped like
  the agentic trace the DCP post benchmarks on (section 2.1 "Dataset": median
  near 67k, about half the requests at 64k and above with a long tail, about
  18% under 8k, a few percent above 256k).  The trace itself is not used.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor ids inside the RNG key
T_Q, T_KV, T_K, T_V, T_LEN, T_PERM, T_PART_O, T_PART_LSE, T_WUV, T_GATE = 1, 2, 3, 4, 5, 6, 7, 8, 9, 10
CHUNK = 1 << 16  # global token positions per RNG chunk

ROUND_ROBIN = 0
CONTIGUOUS = 1


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite normal draws, so NaN handling is not needed.
    Rounding adds 0x7FFF plus the kept part's lowest bit to the float32 bits
    and drops the low 16 bits.  Done in pieces of 2^20 values so the
    temporaries stay in the host caches (large caches are generated in
    chunks of tens of millions of values).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, np.uint16)
    step = 1 << 20
    tmp = np.empty(min(step, flat.size), np.uint32)
    for i in range(0, flat.size, step):
        u = flat[i:i + step]
        t = tmp[:u.size]
        np.right_shift(u, np.uint32(16), out=t)
        np.bitwise_and(t, np.uint32(1), out=t)
        np.add(t, np.uint32(0x7FFF), out=t)
        np.add(t, u, out=t)
        np.right_shift(t, np.uint32(16), out=t)
        out[i:i + u.size] = t
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(key, shape) -> np.ndarray:
    """bf16 bits of float32 standard normal draws from the generator keyed
    ``key``, in C order.  The draws are taken in consecutive pieces of the one
    stream (the same values as a single call) so no full-size float32
    temporary is needed."""
    rng = np.random.default_rng(list(key))
    out = np.empty(shape, np.uint16)
    flat = out.reshape(-1)
    step = 1 << 20
    buf = np.empty(min(step, flat.size), np.float32)
    for i in range(0, flat.size, step):
        x = buf[:min(step, flat.size - i)]
        rng.standard_normal(out=x, dtype=np.float32)
        flat[i:i + x.size] = f32_to_bf16_bits(x)
    return out


# ---------------------------------------------------------------- fp8 (E4M3) codes

def _e4m3_grid() -> np.ndarray:
    """Magnitudes of the non-negative finite E4M3 codes 0x00..0x7E, in code order."""
    c = np.arange(0x7F)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))


_E4M3 = _e4m3_grid()

# Dequantization scale of the fp8 workloads: the largest code (448) stands for
# 6 standard deviations of the N(0, 1) cache values.
FP8_SCALE = 6.0 / 448.0


def f32_to_e4m3_bits_grid(x: np.ndarray) -> np.ndarray:
    """Round values to the nearest E4M3 code (ties to the even code), clamping
    magnitudes to 448; returns uint8 codes.  Inputs are finite.  Reference form:
    a search over the table of code values (slow; ``f32_to_e4m3_bits`` gives the
    same codes)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(448.0))
    grid = _E4M3.astype(np.float32)  # exact: every E4M3 value is a float32 value
    i = np.clip(np.searchsorted(grid, a), 1, len(grid) - 1)
    lo, hi = grid[i - 1], grid[i]
    up = (a - lo > hi - a) | ((a - lo == hi - a) & (i % 2 == 0))
    code = np.where(up, i, i - 1).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def _e4m3_codes(a: np.ndarray) -> np.ndarray:
    """E4M3 codes of magnitudes 0 <= a <= 448 (float32), nearest, ties to even."""
    # normal range (a >= 2^-6): round the float32 significand to 3 bits, ties to
    # even, on the bit pattern (a carry out of the significand bumps the exponent)
    bits = a.view(np.uint32)
    r = (bits + np.uint32(0x7FFFF) + ((bits >> np.uint32(20)) & np.uint32(1))) >> np.uint32(20)
    # r = (biased float32 exponent << 3) | 3-bit significand; E4M3 bias is 7, float32's 127
    normal = (r - np.uint32((127 - 7) << 3)).astype(np.int64)
    # below 2^-6 the codes are multiples of 2^-9 (code 8 is 2^-6 itself)
    sub = np.rint(a * np.float32(512.0)).astype(np.int64)
    return np.where(a < np.float32(2.0 ** -6), sub, normal).astype(np.uint8)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round values to the nearest E4M3 code (ties to the even code), clamping
    magnitudes to 448; returns uint8 codes.  Inputs are finite."""
    x = np.asarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    flat_x, flat_o = x.reshape(-1), out.reshape(-1)
    step = 1 << 20
    for i in range(0, flat_x.size, step):
        xs = flat_x[i:i + step]
        a = np.minimum(np.abs(xs), np.float32(448.0))
        code = _e4m3_codes(a)
        flat_o[i:i + step] = np.where(np.signbit(xs), code | np.uint8(0x80), code)
    return out


# ---------------------------------------------------------------- layouts

def local_len(L: int, n: int, r: int, layout: int) -> int:
    """Number of a request's L tokens that live on shard r (input layout)."""
    if layout == ROUND_ROBIN:
        return len(range(r, L, n))
    c = -(-L // n)
    return len(range(r * c, min(L, (r + 1) * c)))


def local_positions(L: int, n: int, r: int, layout: int) -> range:
    """Global token positions stored on shard r, in local order."""
    if layout == ROUND_ROBIN:
        return range(r, L, n)
    c = -(-L // n)
    return range(r * c, min(L, (r + 1) * c))


# ---------------------------------------------------------------- length sampler

def sample_bimodal_lengths(n: int, rng: np.random.Generator, cap: int = 512 * 1024) -> np.ndarray:
    """Bimodal context-length mixture standing in for an agentic trace.

    18%: log-uniform on [1K, 8K); 29%: log-uniform on [8K, 64K); 53%: log-normal
    with median 67K and sigma 0.75, redrawn while below 64K, capped at ``cap``.
    K = 1024 tokens.
    """
    k = 1024
    out = np.empty(n, dtype=np.int64)
    for i in range(n):
        u = rng.random()
        if u < 0.18:
            v = math.exp(rng.uniform(math.log(1 * k), math.log(8 * k)))
        elif u < 0.47:
            v = math.exp(rng.uniform(math.log(8 * k), math.log(64 * k)))
        else:
            while True:
                v = 67 * k * math.exp(0.75 * rng.standard_normal())
                if v >= 64 * k:
                    break
            v = min(v, cap)
        out[i] = int(v)
    return out


# ---------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # id inside the RNG key
    kind: str                # "mla" or "gqa"
    batch: int
    heads: int               # query heads
    block_size: int
    num_shards: int
    ranks: tuple             # shard ranks whose partial a step computes and times
    seq_lens: tuple | None   # fixed lengths, or None for the bimodal sampler
    kv_lora_rank: int = 512  # MLA c_kv width
    rope_dim: int = 64       # MLA k_rope width
    kv_heads: int = 1        # GQA KV heads
    head_dim: int = 128      # GQA head width
    layout: int = ROUND_ROBIN
    scale: float = 1.0
    description: str = ""

    @property
    def dk(self) -> int:
        return self.kv_lora_rank + self.rope_dim if self.kind == "mla" else self.head_dim

    @property
    def dv(self) -> int:
        return self.kv_lora_rank if self.kind == "mla" else self.head_dim


MLA_SCALE = 1.0 / math.sqrt(192.0)
GQA_SCALE = 1.0 / math.sqrt(128.0)

WORKLOADS = {
    "c0": Workload("c0", 0, "mla", batch=2, heads=16, block_size=64, num_shards=4, ranks=(0, 1, 2, 3),
                   seq_lens=(1024, 1024), scale=MLA_SCALE,
                   description="tiny MLA: b=2, H=16, L=1024, B=64, N=4 round-robin, all 4 partials + combine"),
    "c1": Workload("c1", 1, "mla", batch=1, heads=64, block_size=64, num_shards=8, ranks=(1,),
                   seq_lens=(65536,), scale=MLA_SCALE,
                   description="MLA b=1, H=64, L=64K, shard 1 of 8 (8K local), B=64, combine over 8"),
    "c2": Workload("c2", 2, "mla", batch=32, heads=64, block_size=64, num_shards=8, ranks=(1,),
                   seq_lens=None, scale=MLA_SCALE,
                   description="MLA b=32, H=64, bimodal ragged lengths, shard 1 of 8, B=64, combine over 8"),
    "c3": Workload("c3", 3, "gqa", batch=16, heads=64, kv_heads=8, head_dim=128, block_size=16,
                   num_shards=4, ranks=(1,), seq_lens=(131072,) * 16, scale=GQA_SCALE,
                   description="GQA b=16, 64 q / 8 KV heads, D=128, L=128K, shard 1 of 4, B=16, combine over 4"),
    "c4a": Workload("c4a", 4, "mla", batch=1, heads=64, block_size=64, num_shards=8, ranks=tuple(range(8)),
                    seq_lens=(1 << 20,), scale=MLA_SCALE,
                    description="MLA b=1, H=64, L=1M, all 8 shards (128K local each), combine over 8"),
    "c4b": Workload("c4b", 5, "mla", batch=128, heads=64, block_size=64, num_shards=8, ranks=(1,),
                    seq_lens=(65536,) * 128, scale=MLA_SCALE,
                    description="MLA b=128, H=64, L=64K, shard 1 of 8 (8K local), B=64, combine over 8"),
    # the DCP post's GQA deployment example (4 KV heads, tp 8, dcp 2): each rank
    # holds 8 query heads and one KV head; C3's lengths and block size
    "c3kv1": Workload("c3kv1", 6, "gqa", batch=16, heads=8, kv_heads=1, head_dim=128, block_size=16,
                      num_shards=2, ranks=(1,), seq_lens=(131072,) * 16, scale=GQA_SCALE,
                      description="GQA b=16, 8 q / 1 KV head per rank, D=128, L=128K, shard 1 of 2, B=16, "
                                  "combine over 2"),
}


def custom_workload(kind="mla", batch=1, heads=16, seq_lens=(100,), block_size=64, num_shards=1,
                    layout=ROUND_ROBIN, kv_heads=1, head_dim=128, scale=None, wid=100,
                    kv_lora_rank=512, rope_dim=64, name="custom") -> Workload:
    if scale is None:
        scale = MLA_SCALE if kind == "mla" else 1.0 / math.sqrt(head_dim)
    return Workload(name, wid, kind, batch=batch, heads=heads, block_size=block_size,
                    num_shards=num_shards, ranks=tuple(range(num_shards)), seq_lens=tuple(seq_lens),
                    kv_heads=kv_heads, head_dim=head_dim, layout=layout, scale=scale,
                    kv_lora_rank=kv_lora_rank, rope_dim=rope_dim)


@dataclass
class ShardCache:
    """One shard's paged cache: pool(s) of bf16 bits and its block table."""
    rank: int
    local_lens: np.ndarray           # int64 [batch]
    block_table: np.ndarray          # int32 [batch][max_blocks]
    pools: list = field(default_factory=list)  # MLA: [kv]; GQA: [k, v]; uint16 (bf16) or uint8 (fp8) arrays

    @property
    def num_blocks(self) -> int:
        return int(self.pools[0].shape[0]) if self.pools else 0


class Case:
    """A seeded instance of a workload."""

    def __init__(self, w: Workload, seed: int = 0, q_scale_pow2: int = 0, needles=(),
                 kv_fp8_scale: float | None = None):
        """``q_scale_pow2`` multiplies every query by 2**k (exact in bf16), which
        sharpens the softmax.  ``needles`` is a list of (request, position,
        head): the K/V row at that global position is replaced by that head's
        query, planting one dominant key (MLA only).  ``kv_fp8_scale`` makes
        the latent cache fp8 (MLA only): rows hold E4M3 codes of value / scale."""
        assert kv_fp8_scale is None or w.kind == "mla"
        self.w = w
        self.seed = seed
        self.kv_fp8_scale = None if kv_fp8_scale is None else float(kv_fp8_scale)
        self.q_scale_pow2 = int(q_scale_pow2)
        self.needles = tuple(needles)
        if w.seq_lens is None:
            rng = np.random.default_rng([seed, w.wid, T_LEN])
            self.seq_lens = sample_bimodal_lengths(w.batch, rng).astype(np.int32)
        else:
            assert len(w.seq_lens) == w.batch
            self.seq_lens = np.asarray(w.seq_lens, dtype=np.int32)
        self._q = None

    # ---- queries
    @property
    def q(self) -> np.ndarray:
        if self._q is None:
            w = self.w
            q = np.stack([normal_bf16((self.seed, w.wid, T_Q, b, 0), (w.heads, w.dk))
                          for b in range(w.batch)]) if w.batch else np.zeros((0, w.heads, w.dk), np.uint16)
            if self.q_scale_pow2:
                # add k to the bf16 exponent field (values stay normal for N(0,1) draws)
                nz = (q & 0x7F80) != 0
                q = np.where(nz, q + np.uint16((self.q_scale_pow2 & 0xFF) << 7), q).astype(np.uint16)
            self._q = q
        return self._q

    def queries(self, q_len: int) -> np.ndarray:
        """Queries of a q_len-token decode step, bf16 bits [batch][q_len][heads][dk]
        (the head width is dk for MLA and head_dim for GQA); token 0 is ``q``."""
        w = self.w
        out = np.empty((w.batch, q_len, w.heads, w.dk), np.uint16)
        for b in range(w.batch):
            out[b, 0] = self.q[b]
            for j in range(1, q_len):
                out[b, j] = normal_bf16((self.seed, w.wid, T_Q, b, j), (w.heads, w.dk))
        return out

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    def max_blocks_per_seq(self) -> int:
        w = self.w
        m = max((local_len(int(L), w.num_shards, r, w.layout)
                 for L in self.seq_lens for r in range(w.num_shards)), default=0)
        return max(1, -(-m // w.block_size))

    # ---- logical (unsharded) K/V of one request
    def _tensor_ids(self):
        return (T_KV,) if self.w.kind == "mla" else (T_K, T_V)

    def _row_shape(self):
        w = self.w
        return (w.dk,) if w.kind == "mla" else (w.kv_heads, w.head_dim)

    @property
    def kv_dtype(self):
        return np.uint16 if self.kv_fp8_scale is None else np.uint8

    def _chunk(self, tid: int, b: int, c: int, L: int) -> np.ndarray:
        t0 = c * CHUNK
        n = min(CHUNK, L - t0)
        if self.kv_fp8_scale is not None:
            rng = np.random.default_rng([self.seed, self.w.wid, tid, b, c])
            x = rng.standard_normal((n,) + self._row_shape(), dtype=np.float32)
            for nb, pos, head in self.needles:
                if nb == b and t0 <= pos < t0 + n:
                    x[pos - t0] = bf16_bits_to_f32(self.q[b, head])
            return f32_to_e4m3_bits(x / np.float32(self.kv_fp8_scale))
        a = normal_bf16((self.seed, self.w.wid, tid, b, c), (n,) + self._row_shape())
        for nb, pos, head in self.needles:
            if nb == b and t0 <= pos < t0 + n:
                a[pos - t0] = self.q[b, head]
        return a

    def kv_logical(self, b: int, t0: int = 0, t1: int | None = None):
        """Stored bits of request b's tokens [t0, t1) in global order (bf16
        bits, or E4M3 codes for an fp8 cache).

        MLA: one array [n][576]; GQA: (K, V) each [n][kv_heads][head_dim].
        """
        L = int(self.seq_lens[b])
        t1 = L if t1 is None else min(t1, L)
        outs = []
        for tid in self._tensor_ids():
            parts = []
            for c in range(t0 // CHUNK, -(-t1 // CHUNK)):
                a = self._chunk(tid, b, c, L)
                lo = max(t0, c * CHUNK) - c * CHUNK
                hi = min(t1, (c + 1) * CHUNK) - c * CHUNK
                parts.append(a[lo:hi])
            outs.append(np.concatenate(parts) if parts else np.zeros((0,) + self._row_shape(), self.kv_dtype))
        return outs[0] if self.w.kind == "mla" else tuple(outs)

    def rows_at(self, b: int, positions) -> list:
        """Stored bits of request b at the given global token positions (any order)."""
        pos = np.asarray(positions, dtype=np.int64)
        L = int(self.seq_lens[b])
        res = []
        for tid in self._tensor_ids():
            out = np.empty((len(pos),) + self._row_shape(), self.kv_dtype)
            for c in np.unique(pos // CHUNK):
                sel = np.nonzero(pos // CHUNK == c)[0]
                out[sel] = self._chunk(tid, b, int(c), L)[pos[sel] - c * CHUNK]
            res.append(out)
        return res

    # ---- one shard's paged cache
    def local_lens(self, r: int) -> np.ndarray:
        w = self.w
        return np.array([local_len(int(L), w.num_shards, r, w.layout) for L in self.seq_lens], dtype=np.int64)

    def block_table(self, r: int, max_blocks: int | None = None) -> tuple[np.ndarray, int]:
        """(table int32 [batch][max_blocks], number of pool blocks) for shard r."""
        w = self.w
        ll = self.local_lens(r)
        nblk = -(-ll // w.block_size)
        total = int(nblk.sum())
        mb = self.max_blocks_per_seq() if max_blocks is None else max_blocks
        perm = np.random.default_rng([self.seed, w.wid, T_PERM, r]).permutation(max(total, 1)).astype(np.int32)
        table = np.zeros((w.batch, mb), dtype=np.int32)
        off = 0
        for b in range(w.batch):
            n = int(nblk[b])
            table[b, :n] = perm[off:off + n]
            off += n
        return table, max(total, 1)

    def shard(self, r: int, max_blocks: int | None = None, threads: int | None = None) -> ShardCache:
        """Build shard r's pool(s) and table (host memory, stored bits)."""
        return self.shards([r], max_blocks, threads)[0]

    def shards(self, ranks, max_blocks: int | None = None, threads: int | None = None) -> list:
        """Build several shards' pools in one pass over the generated K/V."""
        w = self.w
        B = w.block_size
        ranks = list(ranks)
        out = []
        for r in ranks:
            table, nb = self.block_table(r, max_blocks)
            pools = [np.zeros((nb, B) + self._row_shape(), self.kv_dtype) for _ in self._tensor_ids()]
            out.append(ShardCache(rank=r, local_lens=self.local_lens(r), block_table=table, pools=pools))
        jobs = [(b, c) for b in range(w.batch) for c in range(-(-int(self.seq_lens[b]) // CHUNK))]

        def fill(job):
            b, c = job
            L = int(self.seq_lens[b])
            t0, t1 = c * CHUNK, min(L, (c + 1) * CHUNK)
            chunks = [self._chunk(tid, b, c, L) for tid in self._tensor_ids()]
            for sc in out:
                r = sc.rank
                pos = local_positions(L, w.num_shards, r, w.layout)
                if w.layout == ROUND_ROBIN:
                    j0 = len(range(r, t0, w.num_shards))
                    j1 = len(range(r, t1, w.num_shards))
                else:
                    j0 = min(max(t0 - pos.start, 0), len(pos))
                    j1 = min(max(t1 - pos.start, 0), len(pos))
                if j1 <= j0:
                    continue
                j = np.arange(j0, j1)
                g = np.asarray(pos[j0:j1], dtype=np.int64) - t0
                blk = sc.block_table[b, j // B]
                off = j % B
                for p, a in zip(sc.pools, chunks):
                    p[blk, off] = a[g]

        n = threads or _threads()
        if n > 1 and len(jobs) > 1:
            with ThreadPoolExecutor(n) as ex:
                list(ex.map(fill, jobs))
        else:
            for jb in jobs:
                fill(jb)
        return out


def random_partials(num_shards: int, batch: int, heads: int, dv: int, seed: int = 0,
                    empty_frac: float = 0.0, lse_spread: float = 4.0):
    """Synthetic shard partials (o fp32 [N][b][H][dv], lse fp32 [N][b][H]) for combine tests.

    ``empty_frac`` of the (shard, b, h) slots get lse = -inf and o = 0, the way
    an empty local slice reports itself.
    """
    rng = np.random.default_rng([seed, 99, T_PART_O])
    o = rng.standard_normal((num_shards, batch, heads, dv), dtype=np.float32)
    rng2 = np.random.default_rng([seed, 99, T_PART_LSE])
    lse = (rng2.standard_normal((num_shards, batch, heads)) * lse_spread).astype(np.float32)
    if empty_frac > 0:
        mask = rng2.random((num_shards, batch, heads)) < empty_frac
        lse[mask] = -np.inf
        o[mask] = 0.0
    return o, lse


def random_vproj(batch: int, heads: int, dvo: int, dv: int, seed: int = 0):
    """Synthetic value up-projection and gate logits for the fused combine
    epilogue, as bf16 bit patterns: w_uv_t [heads][dvo][dv] ~ N(0, 1/dv) (so
    projected outputs stay O(1)) and gate [batch][heads][dvo] ~ N(0, 1)."""
    rw = np.random.default_rng([seed, 98, T_WUV])
    w = rw.standard_normal((heads, dvo, dv), dtype=np.float32) * np.float32(1.0 / math.sqrt(dv))
    rg = np.random.default_rng([seed, 98, T_GATE])
    g = rg.standard_normal((batch, heads, dvo), dtype=np.float32)
    return f32_to_bf16_bits(w), f32_to_bf16_bits(g)
