// Shard-local MLA decode attention (absorbed form) for gfx950.
//
// What one shard computes (vLLM blog post on Decode Context Parallelism,
// sections 4.1 and 5.3): every query head attends its request's local latent
// rows [c_kv | k_rope] (576 bf16); the value is c_kv (512).  The output is the
// normalized partial attention and its natural-log LSE, merged across shards
// by dcp_combine.
//
// Structure (per split workgroup of 4 waves, one per 16 query heads):
//  * The workgroup streams its tile range of the shard's paged cache from HBM
//    into LDS with direct global->LDS copies (no register staging), 32 tokens
//    (36 KiB) per tile, 4 tiles in LDS; every latent byte crosses HBM once for
//    all 64 heads.
//  * Scores, transposed: S^T[32 tok x 16 heads] = K_tile[32 x 576] . q^T with
//    v_mfma_f32_16x16x32_bf16; the wave's q stays in registers for the whole
//    segment.
//  * Online softmax in base 2 (scale * log2 e folded into one FMA); the score
//    tile layout puts one head per lane column, so the running max needs two
//    cross-lane steps and the output rescale is lane-local.
//  * Values, transposed: O^T[512 x 16 heads] += V^T[512 x 32 tok] . P^T with
//    V^T read straight from the row-major tile by ds_read_b64_tr_b16.
//  * LDS rows are 1152 B; 16-byte chunks are XOR-swizzled per row so both the
//    row-wise K reads and the transposing V reads hit distinct banks.
//  * Split-K partials go to the workspace and a small kernel merges them.
#include "dcp_device.hpp"
#include "dcp_internal.hpp"
#include "dcp_split.hpp"

namespace dcp {
namespace mla {

constexpr int R = 512, P = 64, DK = R + P;
constexpr int ROW = DK * 2;           // bytes per latent row
constexpr int TILE = 32;              // tokens per pipeline tile
constexpr int STAGE = TILE * ROW;     // 36864 bytes
#ifndef DCP_MLA_NST
#define DCP_MLA_NST 4
#endif
constexpr int NST = DCP_MLA_NST;      // tiles resident in LDS (NST - 1 in flight)
static_assert(NST >= 2 && NST <= 4, "ring depth");
constexpr int CPR = ROW / 16;         // 16-byte chunks per row (72)
constexpr int THREADS = 256;
constexpr int DMA_N = TILE * CPR / THREADS;  // copies per thread per tile (9)
constexpr int KS = DK / 32;           // k-steps of the score contraction (18)
constexpr int VB = R / 16;            // 16-column blocks of the value contraction (32)
static_assert(TILE * CPR % THREADS == 0, "tile copy split");

// Chunk swizzle of LDS row r: 16-byte chunk c of row r is stored at chunk
// (c & ~7) | ((c & 7) ^ swz(r)), so a row's 72 chunks stay inside their aligned
// groups of 8.  swz(r) = r mod 8 was selected on gfx950 by counting LDS bank
// conflicts (SQ_LDS_BANK_CONFLICT) for the two read patterns of this kernel
// across a set of candidate swizzles: it is conflict-free for both the row-wise
// score reads (ds_read_b128, 16 rows x 4 chunks per instruction) and the
// transposing value reads (ds_read_b64_tr_b16, 16 rows x 2 chunks).
__host__ __device__ constexpr int swz(int r) { return r & 7; }

constexpr int TBL = 1024;  // block-table entries staged in LDS per window

struct Smem {
  char tiles[NST * STAGE];
  int pref[kMaxBatch + 1];
  int tbl[TBL];
  int wsum[THREADS / 64];
  int flag;
};

// Where the copies of one tile go: source block(s) and LDS stage.  All fields
// are wave-uniform.
struct TileCopy {
  const char* base0;  // source of tile row 0 (block pg0)
  const char* base1;  // source such that base1 + goff is right for rows >= split
  DCP_LDS char* stage;
  int split;          // rows [0, split) come from block pg0, the rest from pg0 + 1
  bool valid;
};

// The segment's block-table entries live in an LDS window, so the per-tile
// lookup is an LDS read rather than a dependent load from HBM.  Entries are
// clamped to the pool when staged.
struct TableWin {
  int lo;   // first local block held
  int end;  // one past the last block held
};

__device__ __forceinline__ void load_window(const MlaArgs& a, const int32_t* trow, Smem& sm, int lo, int hi) {
  const SplitArgs& s = a.s;
  const int n = min(hi - lo, TBL);
  for (int i = (int)threadIdx.x; i < n; i += THREADS) {
    const int j = min(lo + i, s.max_blocks - 1);
    sm.tbl[i] = min(max(trow[j], 0), s.num_blocks - 1);
  }
}

__device__ __forceinline__ TileCopy plan_copy(const MlaArgs& a, const int32_t* trow, Smem& sm, TableWin& win,
                                              int pg_hi, int k, DCP_LDS char* stage, bool valid) {
  TileCopy t;
  t.valid = valid;
  t.stage = stage;
  const SplitArgs& s = a.s;
  const int B = s.block_size;
  const int tok0 = k * TILE;
  const int pg0 = uni(tok0 / B);
  const int in0 = tok0 - pg0 * B;
  t.split = B - in0;
  int e0 = 0, e1 = 0;
  if (valid) {
    // rows past `split` need block pg0 + 1 only if the request has one; else
    // they are past the request's end (zeroed later) and read block pg0 again
    const bool two = t.split < TILE && pg0 + 1 < pg_hi;
    const int need = two ? pg0 + 1 : pg0;
    if (need >= win.end) {  // slide the window (rare: every TBL blocks)
      barrier();
      load_window(a, trow, sm, pg0, pg_hi);
      wait_vmcnt<0>();
      wait_lgkm0();
      barrier();
      win.lo = pg0;
      win.end = min(pg_hi, pg0 + TBL);
    }
    e0 = uni(sm.tbl[pg0 - win.lo]);
    e1 = two ? uni(sm.tbl[pg0 + 1 - win.lo]) : e0;
  }
  const char* kv = (const char*)a.kv;
  t.base0 = kv + ((int64_t)e0 * B + in0) * ROW;
  t.base1 = kv + ((int64_t)e1 * B - t.split) * ROW;
  return t;
}

// Issue copy i (0 <= i < DMA_N) of a planned tile: 1 KiB per wave.
__device__ __forceinline__ void copy_part(const TileCopy& t, int i, const int (&goff)[DMA_N],
                                          const int (&grow)[DMA_N]) {
  if (!t.valid) return;
  const int wave = uni(threadIdx.x >> 6);
  DCP_LDS char* dst = t.stage + (i * (THREADS / 64) + wave) * 1024;
  if (t.split >= TILE) {
    dma16_sbase(t.base0, (uint32_t)goff[i], dst);
  } else {
    dma16((grow[i] < t.split ? t.base0 : t.base1) + goff[i], dst);
  }
}

__device__ __forceinline__ void copy_all(const TileCopy& t, const int (&goff)[DMA_N], const int (&grow)[DMA_N]) {
#pragma unroll
  for (int i = 0; i < DMA_N; ++i) copy_part(t, i, goff, grow);
}

// Zero the tile rows at and past `valid` (the unused end of the last block),
// so stale cache contents can never reach the value contraction.
__device__ __forceinline__ void zero_tail(DCP_LDS char* stage, int valid) {
  const int start = valid * CPR;
  for (int c = start + (int)threadIdx.x; c < TILE * CPR; c += THREADS)
    *(DCP_LDS f32x4*)(stage + c * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// One 32-token tile for the wave's 16 heads: scores, softmax, P.V.
// EXACT = false: the softmax reference m is the segment's first-tile maximum
//   and never moves; tiles whose maximum exceeds it by more than `thr` (p would
//   pass 2^64) only raise `ovf`, and the caller recomputes the segment with
//   EXACT = true.  No branch touches the output accumulators, so they stay in
//   the matrix-core registers.
// EXACT = true: classic online softmax, rescaling the output whenever the
//   running maximum grows.
template <bool EXACT>
__device__ __forceinline__ void compute_tile(const DCP_LDS char* st, int tok0, int lr, bool first,
                                             const bf16x8 (&qf)[KS], f32x4 (&acc)[VB], float& m,
                                             float& l, float c, float thr, bool& ovf,
                                             const TileCopy& nxt, const int (&goff)[DMA_N],
                                             const int (&grow)[DMA_N]) {
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, r16 = lane & 15;

  // ---- scores S^T[tok][head], two 16-token blocks.  K operands are read in
  // groups of KG k-steps, one group ahead of the MFMAs that use them; the
  // scheduling fences keep that shape (unbounded look-ahead spills registers).
  const int fz = swz(r16);
  const int offE = ((g4) ^ fz) * 16;
  const int offO = ((4 | g4) ^ fz) * 16;
  const DCP_LDS char* k0p = st + r16 * ROW;
  const DCP_LDS char* k1p = st + (16 + r16) * ROW;
  constexpr int KG = 3;
  static_assert(KS % KG == 0, "k groups");
  static_assert(KS / KG + VB / 8 >= DMA_N, "copy slots");
  bf16x8 ka[2][KG], kb[2][KG];
  auto load_group = [&](int grp, int buf) {
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const int ks = grp * KG + j;
      const int off = (ks >> 1) * 128 + ((ks & 1) ? offO : offE);
      ka[buf][j] = *(const DCP_LDS bf16x8*)(k0p + off);
      kb[buf][j] = *(const DCP_LDS bf16x8*)(k1p + off);
    }
  };
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  load_group(0, 0);
#pragma unroll
  for (int grp = 0; grp < KS / KG; ++grp) {
    __builtin_amdgcn_sched_barrier(0);
    // the next tile's copies are spread over the MFMA groups so that their
    // issue latency hides behind matrix work
    copy_part(nxt, grp, goff, grow);
    if (grp + 1 < KS / KG) load_group(grp + 1, (grp + 1) & 1);
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      s0 = mfma_16x16x32(ka[grp & 1][j], qf[grp * KG + j], s0);
      s1 = mfma_16x16x32(kb[grp & 1][j], qf[grp * KG + j], s1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- online softmax (base 2).  Lane holds head r16, tokens 4*g4+i and 16+4*g4+i.
  float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  if (tok0 + TILE > lr) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = tok0 + (j < 4 ? 4 * g4 + j : 16 + 4 * g4 + (j - 4));
      if (t >= lr) sv[j] = -__builtin_inff();
    }
  }
  float mt = sv[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mt = fmaxf(mt, sv[j]);
  mt = wave_max16(mt);
  if constexpr (!EXACT) {
    if (first) m = mt;
    else ovf = ovf || (mt > m + thr);
  } else {
    const float mnew = fmaxf(m, mt);
    const float alpha = exp2_fast((m - mnew) * c);  // 0 while m is still -inf
    l *= alpha;
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int cb = 0; cb < VB; ++cb) acc[cb] *= alpha;
    }
    m = mnew;
  }
  const float mc = m * c;
  float p[8];
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = exp2_fast(fmaf(sv[j], c, -mc));
    ps += p[j];
  }
  l += ps;
  bf16x8 pt;
#pragma unroll
  for (int j = 0; j < 8; ++j) pt[j] = (__bf16)p[j];

  // ---- values O^T[col][head] += V^T[col][tok] . P^T[tok][head]
  // V^T operands come from transposing LDS reads, VG column blocks per group,
  // one group ahead of their MFMAs.
  const int rowa = 4 * g4 + (r16 >> 2);
  const int fa = swz(rowa);
  const int hb = (r16 & 3) >> 1;
  const int byte = (r16 & 1) * 8;
  const DCP_LDS char* va = st + rowa * ROW + byte;
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) voff[q] = (((2 * q) | hb) ^ fa) * 16;
  constexpr int VG = 4;
  static_assert(VB % VG == 0, "v groups");
  i16x4 vlo[2][VG], vhi[2][VG];
  auto load_v = [&](int grp, int buf) {
#pragma unroll
    for (int j = 0; j < VG; ++j) {
      const int cb = grp * VG + j;
      const DCP_LDS char* p0 = va + (cb >> 2) * 128 + voff[cb & 3];
      vlo[buf][j] = lds_read_tr16(p0);
      vhi[buf][j] = lds_read_tr16(p0 + 16 * ROW);
    }
  };
  load_v(0, 0);
#pragma unroll
  for (int grp = 0; grp < VB / VG; ++grp) {
    __builtin_amdgcn_sched_barrier(0);
    if ((grp & 1) == 0 && KS / KG + grp / 2 < DMA_N) copy_part(nxt, KS / KG + grp / 2, goff, grow);
    if (grp + 1 < VB / VG) load_v(grp + 1, (grp + 1) & 1);
#pragma unroll
    for (int j = 0; j < VG; ++j) {
      const int cb = grp * VG + j;
      const i16x8 v8 = __builtin_shufflevector(vlo[grp & 1][j], vhi[grp & 1][j], 0, 1, 2, 3, 4, 5, 6, 7);
      acc[cb] = mfma_16x16x32(__builtin_bit_cast(bf16x8, v8), pt, acc[cb]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <bool EXACT>
__device__ __attribute__((always_inline)) inline bool run_segment_body(
    const MlaArgs& a, Smem& sm, int b, int t0, int t1, int ntiles_b, int g) {
  const SplitArgs& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int heads = a.heads;
  const bool active = wave * 16 < heads;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int head = wave * 16 + r16;
  DCP_LDS char* tiles = (DCP_LDS char*)sm.tiles;
  const float thr = 64.f / s.c;  // raw-score headroom of the fixed reference (p < 2^64)
  const int n = t1 - t0;
  const int lr = uni(clamped_local_len(s, b));
  const int32_t* trow = s.table + (int64_t)b * s.max_blocks;

  // per-thread copy pattern of a tile: LDS chunk slot -> source chunk (swizzled)
  int goff[DMA_N], grow[DMA_N];
#pragma unroll
  for (int i = 0; i < DMA_N; ++i) {
    const int slot = (i * (THREADS / 64) + wave) * 64 + lane;
    const int r = slot / CPR, ch = slot % CPR;
    grow[i] = r;
    goff[i] = r * ROW + ((ch ^ swz(r)) * 16);
  }

  bf16x8 qf[KS];
  if (active) {
    const bf16x8* qp = (const bf16x8*)(a.q + ((int64_t)b * heads + head) * DK + 8 * g4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qp[4 * ks];
    // Make the compiler wait for q here, before any tile copy is in flight;
    // otherwise its wait lands inside the tile loop and drains the prefetch.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }
  f32x4 acc[VB];
#pragma unroll
  for (int cb = 0; cb < VB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;
  bool ovf = false;

  // stage the segment's block-table entries: local blocks [pg_lo, pg_hi)
  const int pg_lo = uni((t0 * TILE) / s.block_size);
  const int pg_hi = uni(min(s.max_blocks, (min(t1 * TILE, lr) - 1) / s.block_size + 1));
  TableWin win{pg_lo, min(pg_hi, pg_lo + TBL)};
  load_window(a, trow, sm, pg_lo, pg_hi);
  wait_vmcnt<0>();
  wait_lgkm0();
  barrier();

  copy_all(plan_copy(a, trow, sm, win, pg_hi, t0, tiles, true), goff, grow);
#pragma unroll
  for (int j = 1; j < NST - 1; ++j)
    if (n > j) copy_all(plan_copy(a, trow, sm, win, pg_hi, t0 + j, tiles + j * STAGE, true), goff, grow);
  for (int i = 0; i < n; ++i) {
    const int k = t0 + i;
    const int rem = n - 1 - i;
    // copies issued after tile k: min(NST - 2, rem) tiles
    if (NST >= 4 && rem >= 2) wait_vmcnt<(NST >= 4 ? 2 : 0) * DMA_N>();
    else if (NST >= 3 && rem >= 1) wait_vmcnt<DMA_N>();
    else wait_vmcnt<0>();
    barrier();
    DCP_LDS char* cur = tiles + (i % NST) * STAGE;
    const int valid = lr - k * TILE;
    if (valid < TILE) {  // last tile of the request: clear rows past the end
      zero_tail(cur, valid);
      wait_lgkm0();
      barrier();
    }
    const TileCopy nxt = plan_copy(a, trow, sm, win, pg_hi, k + NST - 1, tiles + ((i + NST - 1) % NST) * STAGE,
                                   i + NST - 1 < n);
    if (active) compute_tile<EXACT>(cur, k * TILE, lr, i == 0, qf, acc, m, l, s.c, thr, ovf, nxt, goff, grow);
    else copy_all(nxt, goff, grow);
  }
  if constexpr (!EXACT) {
    if (tid == 0) sm.flag = 0;
    barrier();
    if (active && __any(ovf) && lane == 0) sm.flag = 1;
    barrier();
    const bool redo = uni(sm.flag) != 0;
    barrier();  // also: every wave is done with the tiles before they are refilled
    if (redo) return true;
  } else {
    barrier();
  }

  if (active) {
    const float lt = wave_sum16(l);
    if (t0 == 0 && t1 == ntiles_b) {
      // the whole request is in this workgroup: write the final result
      const float inv = 1.f / lt;
      float* dst = s.out + ((size_t)b * heads + head) * R + 4 * g4;
#pragma unroll
      for (int cb = 0; cb < VB; ++cb) *(f32x4*)(dst + 16 * cb) = acc[cb] * inv;
      if (g4 == 0) s.lse[(size_t)b * heads + head] = (m * s.c + __log2f(lt)) * kLn2;
    } else {
      const int slot = g + b;
      float* dst = s.ws_o + ((size_t)slot * heads + head) * R + 4 * g4;
#pragma unroll
      for (int cb = 0; cb < VB; ++cb) *(f32x4*)(dst + 16 * cb) = acc[cb];
      if (g4 == 0) {
        float* ml = s.ws_ml + ((size_t)slot * heads + head) * 2;
        ml[0] = m;
        ml[1] = lt;
      }
    }
  }
  return false;
}

template <bool EXACT>
__device__ inline bool run_segment(const MlaArgs& a, Smem& sm, int b, int t0, int t1, int ntiles_b, int g);
template <>
__device__ __attribute__((always_inline)) inline bool run_segment<false>(
    const MlaArgs& a, Smem& sm, int b, int t0, int t1, int ntiles_b, int g) {
  return run_segment_body<false>(a, sm, b, t0, t1, ntiles_b, g);
}
// The exact path is rare; keep it out of line so its rescaling code does not
// shape register allocation of the fast path.
template <>
__device__ __attribute__((noinline)) bool run_segment<true>(
    const MlaArgs& a, Smem& sm, int b, int t0, int t1, int ntiles_b, int g) {
  return run_segment_body<true>(a, sm, b, t0, t1, ntiles_b, g);
}

__global__ __launch_bounds__(THREADS, 1) void partial_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem sm;
  const SplitArgs& s = a.s;
  const int tid = threadIdx.x;
  const int g = blockIdx.x;

  const int T = plan_tiles<THREADS>(s, TILE, sm.pref, sm.wsum);
  const int geff = split_wgs(s, T);
  if (g == 0) {
    for (int i = tid; i <= s.batch; i += THREADS) s.ws_meta[1 + i] = sm.pref[i];
    if (tid == 0) s.ws_meta[0] = geff;
  }
  if (g >= geff) return;
  const int p0 = uni((int)((int64_t)g * T / geff));
  const int p1 = uni((int)((int64_t)(g + 1) * T / geff));

  int b = find_request(sm.pref, s.batch, p0);
  for (;;) {
    const int pb = uni(sm.pref[b]), pe = uni(sm.pref[b + 1]);
    if (pe > pb) {
      const int t0 = (p0 > pb ? p0 : pb) - pb;
      const int t1 = (p1 < pe ? p1 : pe) - pb;
      if (run_segment<false>(a, sm, b, t0, t1, pe - pb, g))
        run_segment<true>(a, sm, b, t0, t1, pe - pb, g);
    }
    if (pe >= p1 || b + 1 >= s.batch) break;
    ++b;
  }
}

// Rows (request, head) are visited grid-stride by a bounded grid, so a batch in
// which no request was split costs a short launch, not one block per row.
__global__ __launch_bounds__(R / 2) void reduce_kernel(MlaArgs a) {
  __shared__ float s_w[kMaxSplitWGs];
  reduce_request<R>(a.s, a.heads, blockIdx.y, blockIdx.x, gridDim.x, s_w);
}

}  // namespace mla

hipError_t launch_mla_partial(const MlaArgs& a, hipStream_t stream) {
  if (a.s.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(mla::partial_kernel, dim3(a.s.G), dim3(mla::THREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla::reduce_kernel, reduce_grid(a.s.batch, a.heads), dim3(mla::R / 2), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dcp
