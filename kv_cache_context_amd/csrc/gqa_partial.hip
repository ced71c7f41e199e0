// Shard-local GQA decode attention for gfx950.
//
// What one shard computes (vLLM blog post on Decode Context Parallelism,
// sections 4.1 and 5.4): query head h attends KV head g = floor(h * Hkv / Hq)
// over the shard's local tokens; the result is the normalized partial output and
// its natural-log LSE, merged across shards by dcp_combine.
//
// Structure (per split workgroup of 4 waves, one per KV head of a group of 4):
//  * A 16-token tile holds, per token, the 4 KV heads' K rows (1 KiB contiguous
//    in the cache) and V rows; both are streamed HBM -> LDS with direct
//    global->LDS copies, 4 tiles (32 KiB each) resident.  Each K/V byte is read
//    from HBM once and from LDS once.
//  * Scores, transposed: S^T[16 tok x 16] = K[16 x 128] . q^T with
//    v_mfma_f32_16x16x32_bf16; the KV head's group of query heads fills the 16
//    columns (zero-padded when the group is smaller).
//  * Online softmax in base 2 with rescaling when a head's maximum grows (the
//    output block is only 32 registers per lane).
//  * Values: O^T[128 x 16] += V^T[128 x 16 tok] . P^T with
//    v_mfma_f32_16x16x16_bf16; V^T comes from ds_read_b64_tr_b16, and the score
//    tile's register layout is already the P^T operand layout.
//  * Stream-K split over tiles and the split reduce are shared with MLA.
#include "dcp_device.hpp"
#include "dcp_internal.hpp"
#include "dcp_split.hpp"

namespace dcp {
namespace gqa {

constexpr int D = 128;                 // head dim
constexpr int HROW = D * 2;            // bytes per (token, head) row
constexpr int QH = 4;                  // KV heads per workgroup (one per wave)
constexpr int TROW = QH * HROW;        // bytes per token in a tile (1 KiB)
constexpr int TILE = 16;               // tokens per tile
constexpr int HALF = TILE * TROW;      // 16 KiB: the K (or V) part of a stage
constexpr int STAGE = 2 * HALF;        // K then V
constexpr int NST = 4;
constexpr int THREADS = 256;
constexpr int CPI = TILE / 4;          // copy instructions per wave per part (4)
constexpr int DMA_N = 2 * CPI;         // per wave per tile (8)
constexpr int KS = D / 32;             // score k-steps (4)
constexpr int VB = D / 16;             // value column blocks (8)
constexpr int TBL = 1024;

// Chunk swizzle of token row t inside one head's 16 chunks of 16 bytes.
__host__ __device__ constexpr int swz(int t) { return t & 15; }

struct Smem {
  char tiles[NST * STAGE];
  int pref[kMaxBatch + 1];
  int tbl[TBL];
  int wsum[THREADS / 64];
};

struct TileCopy {
  const char* kbase;  // K cache address of (tile token 0, head 4*quad)
  const char* vbase;
  DCP_LDS char* stage;
  bool valid;
};

__device__ __forceinline__ void load_window(const GqaArgs& a, const int32_t* trow, Smem& sm, int lo, int hi) {
  const SplitArgs& s = a.s;
  const int n = min(hi - lo, TBL);
  for (int i = (int)threadIdx.x; i < n; i += THREADS) {
    const int j = min(lo + i, s.max_blocks - 1);
    sm.tbl[i] = min(max(trow[j], 0), s.num_blocks - 1);
  }
}

struct TableWin {
  int lo, end;
};

__device__ __forceinline__ TileCopy plan_copy(const GqaArgs& a, const int32_t* trow, Smem& sm, TableWin& win,
                                              int pg_hi, int quad, int k, DCP_LDS char* stage, bool valid) {
  TileCopy t;
  t.valid = valid;
  t.stage = stage;
  const SplitArgs& s = a.s;
  const int B = s.block_size;
  const int tok0 = k * TILE;
  const int pg = uni(tok0 / B);  // B is a multiple of 16: a tile never spans two blocks
  const int in0 = tok0 - pg * B;
  int e = 0;
  if (valid) {
    if (pg >= win.end) {  // slide the window (rare)
      barrier();
      load_window(a, trow, sm, pg, pg_hi);
      wait_vmcnt<0>();
      wait_lgkm0();
      barrier();
      win.lo = pg;
      win.end = min(pg_hi, pg + TBL);
    }
    e = uni(sm.tbl[pg - win.lo]);
  }
  const int64_t off = (((int64_t)e * B + in0) * a.hkv + (int64_t)quad * QH) * HROW;
  t.kbase = (const char*)a.k + off;
  t.vbase = (const char*)a.v + off;
  return t;
}

// Copy i of a tile for this wave: i < CPI -> K of token 4*i + wave, else V.
__device__ __forceinline__ void copy_part(const TileCopy& t, int i, const uint32_t (&voff)[CPI]) {
  if (!t.valid) return;
  const int wave = uni(threadIdx.x >> 6);
  const int j = i % CPI;
  const int tok = 4 * j + wave;
  DCP_LDS char* dst = t.stage + (i < CPI ? 0 : HALF) + tok * TROW;
  dma16_sbase(i < CPI ? t.kbase : t.vbase, voff[j], dst);
}

__device__ __forceinline__ void copy_all(const TileCopy& t, const uint32_t (&voff)[CPI]) {
#pragma unroll
  for (int i = 0; i < DMA_N; ++i) copy_part(t, i, voff);
}

__device__ __forceinline__ void zero_tail(DCP_LDS char* stage, int valid) {
  // rows past the end, in both the K and the V half
  for (int c = valid * (TROW / 16) + (int)threadIdx.x; c < TILE * (TROW / 16); c += THREADS) {
    *(DCP_LDS f32x4*)(stage + c * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
    *(DCP_LDS f32x4*)(stage + HALF + c * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

__device__ __forceinline__ void compute_tile(const DCP_LDS char* st, int tok0, int lr, int hk,
                                             const bf16x8 (&qf)[KS], f32x4 (&acc)[VB], float& m, float& l,
                                             float c, const TileCopy& nxt, const uint32_t (&voff)[CPI]) {
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, r16 = lane & 15;
  // ---- scores S^T[tok][head col]: A = K row (token r16), B = q^T
  const DCP_LDS char* kp = st + r16 * TROW + hk * HROW;
  const int fz = swz(r16);
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const DCP_LDS bf16x8*)(kp + (((4 * ks + g4) ^ fz) * 16));
  copy_part(nxt, 0, voff);
  copy_part(nxt, 1, voff);
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) sc = mfma_16x16x32(kf[ks], qf[ks], sc);
  copy_part(nxt, 2, voff);
  copy_part(nxt, 3, voff);

  // ---- online softmax: lane holds head col r16, tokens 4*g4 + i
  float sv[4] = {sc[0], sc[1], sc[2], sc[3]};
  if (tok0 + TILE > lr) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (tok0 + 4 * g4 + i >= lr) sv[i] = -__builtin_inff();
  }
  float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mt = wave_max16(mt);
  const float mnew = fmaxf(m, mt);
  const float alpha = exp2_fast((m - mnew) * c);  // 0 while m is -inf
  l *= alpha;
  if (!__all(alpha == 1.f)) {
#pragma unroll
    for (int cb = 0; cb < VB; ++cb) acc[cb] *= alpha;
  }
  m = mnew;
  const float mc = m * c;
  i16x4 pt;
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = exp2_fast(fmaf(sv[i], c, -mc));
    ps += p;
    pt[i] = __builtin_bit_cast(short, (__bf16)p);
  }
  l += ps;
  copy_part(nxt, 4, voff);
  copy_part(nxt, 5, voff);

  // ---- values O^T[col][head] += V^T[col][tok] . P^T[tok][head]
  const int row = 4 * g4 + (r16 >> 2);  // token this lane addresses
  const int fv = swz(row);
  const int hb = (r16 & 3) >> 1;
  const int byte = (r16 & 1) * 8;
  const DCP_LDS char* vp = st + HALF + row * TROW + hk * HROW + byte;
  i16x4 vt[VB];
#pragma unroll
  for (int cb = 0; cb < VB; ++cb) vt[cb] = lds_read_tr16(vp + (((2 * cb + hb) ^ fv) * 16));
  copy_part(nxt, 6, voff);
  copy_part(nxt, 7, voff);
#pragma unroll
  for (int cb = 0; cb < VB; ++cb) acc[cb] = mfma_16x16x16(vt[cb], pt, acc[cb]);
}

__device__ __forceinline__ void run_segment(const GqaArgs& a, Smem& sm, int quad, int b, int t0, int t1,
                                            int ntiles_b, int g) {
  const SplitArgs& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gs = a.hq / a.hkv;               // query heads per KV head (<= 16)
  const int hk = wave;                        // KV head within the quad
  const int kvh = quad * QH + hk;             // KV head index
  const int g4 = lane >> 4, r16 = lane & 15;
  const bool col_ok = r16 < gs;
  const int qh = kvh * gs + r16;              // query head of this lane's column
  DCP_LDS char* tiles = (DCP_LDS char*)sm.tiles;
  const int n = t1 - t0;
  const int lr = uni(clamped_local_len(s, b));
  const int32_t* trow = table_row(s, b);

  // lane offsets of the copies: token 4*j + wave of the tile, chunk `lane` of its
  // 1 KiB (4 heads x 16 chunks), chunk index swizzled per token
  uint32_t voff[CPI];
#pragma unroll
  for (int j = 0; j < CPI; ++j) {
    const int tok = 4 * j + wave;
    const int h = lane >> 4, ch = lane & 15;
    voff[j] = (uint32_t)(tok * a.hkv * HROW + h * HROW + ((ch ^ swz(tok)) * 16));
  }

  bf16x8 qf[KS];
  {
    const bf16x8* qp = (const bf16x8*)(a.q + ((int64_t)b * a.hq + (col_ok ? qh : 0)) * D + 8 * g4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = qp[4 * ks];
      if (!col_ok) qf[ks] = bf16x8{};
    }
  }
  f32x4 acc[VB];
#pragma unroll
  for (int cb = 0; cb < VB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;

  const int pg_lo = uni((t0 * TILE) / s.block_size);
  const int pg_hi = uni(min(s.max_blocks, (min(t1 * TILE, lr) - 1) / s.block_size + 1));
  TableWin win{pg_lo, min(pg_hi, pg_lo + TBL)};
  load_window(a, trow, sm, pg_lo, pg_hi);  // in flight together with the q loads
  wait_vmcnt<0>();
  wait_lgkm0();
  barrier();
  // q has arrived (vmcnt 0); tie it here so the compiler places no wait for it
  // inside the tile loop, where it would drain the copy prefetch.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));

  copy_all(plan_copy(a, trow, sm, win, pg_hi, quad, t0, tiles, true), voff);
  if (n > 1) copy_all(plan_copy(a, trow, sm, win, pg_hi, quad, t0 + 1, tiles + STAGE, true), voff);
  if (n > 2) copy_all(plan_copy(a, trow, sm, win, pg_hi, quad, t0 + 2, tiles + 2 * STAGE, true), voff);
  for (int i = 0; i < n; ++i) {
    const int k = t0 + i;
    const int rem = n - 1 - i;
    if (rem >= 2) wait_vmcnt<2 * DMA_N>();
    else if (rem == 1) wait_vmcnt<DMA_N>();
    else wait_vmcnt<0>();
    barrier();
    DCP_LDS char* cur = tiles + (i % NST) * STAGE;
    const int valid = lr - k * TILE;
    if (valid < TILE) {
      zero_tail(cur, valid);
      wait_lgkm0();
      barrier();
    }
    const TileCopy nxt = plan_copy(a, trow, sm, win, pg_hi, quad, k + 3, tiles + ((i + 3) % NST) * STAGE, i + 3 < n);
    compute_tile(cur, k * TILE, lr, hk, qf, acc, m, l, s.c, nxt, voff);
  }
  barrier();

  const float lt = wave_sum16(l);
  if (col_ok) {
    if (t0 == 0 && t1 == ntiles_b) {
      const float inv = 1.f / lt;
      float* dst = s.out + ((size_t)b * a.hq + qh) * D + 4 * g4;
#pragma unroll
      for (int cb = 0; cb < VB; ++cb) *(f32x4*)(dst + 16 * cb) = acc[cb] * inv;
      if (g4 == 0) s.lse[(size_t)b * a.hq + qh] = (m * s.c + __log2f(lt)) * kLn2;
    } else {
      const int slot = g + b;
      float* dst = (float*)s.ws_o + ((size_t)slot * a.hq + qh) * D + 4 * g4;
#pragma unroll
      for (int cb = 0; cb < VB; ++cb) *(f32x4*)(dst + 16 * cb) = acc[cb];
      if (g4 == 0) {
        float* ml = s.ws_ml + ((size_t)slot * a.hq + qh) * 2;
        ml[0] = m;
        ml[1] = lt;
      }
    }
  }
}

__global__ __launch_bounds__(THREADS, 1) void partial_kernel(GqaArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem sm;
  const SplitArgs& s = a.s;
  const int tid = threadIdx.x;
  const int g = blockIdx.x, quad = blockIdx.y;
  const int T = plan_tiles<THREADS>(s, TILE, sm.pref, sm.wsum);
  const int geff = split_wgs(s, T);
  if (g == 0 && quad == 0) {
    for (int i = tid; i <= s.batch; i += THREADS) s.ws_meta[1 + i] = sm.pref[i];
    if (tid == 0) s.ws_meta[0] = geff;
  }
  if (g >= geff) return;
  const int p0 = uni((int)((int64_t)g * T / geff));
  const int p1 = uni((int)((int64_t)(g + 1) * T / geff));
  int b = find_request(sm.pref, s.batch, p0);
  for (;;) {
    const int pb = uni(sm.pref[b]), pe = uni(sm.pref[b + 1]);
    const SegTiles st = seg_tiles(s, pb, pe, p0, p1);
    if (pe > pb && st.t1 > st.t0) run_segment(a, sm, quad, b, st.t0, st.t1, st.ntiles, g);
    if (pe >= p1 || b + 1 >= s.batch) break;
    ++b;
  }
}

constexpr int RED_COL_PARTS = 1;  // column parts of the by-segments reduce

__global__ __launch_bounds__(REDUCE_THREADS) void reduce_kernel(GqaArgs a, int by_segments) {
  __shared__ ReduceSmem sm;
  if (by_segments) reduce_by_segments<D, RED_COL_PARTS, float>(a.s, a.hq, blockIdx.z, blockIdx.y, blockIdx.x, sm);
  else reduce_by_heads<D, float>(a.s, a.hq, blockIdx.y, blockIdx.x, sm);
}

}  // namespace gqa

hipError_t launch_gqa_partial(const GqaArgs& a, hipStream_t stream) {
  if (a.s.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(gqa::partial_kernel, dim3(a.s.G, a.hkv / gqa::QH), dim3(gqa::THREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const ReducePlan rp = reduce_plan(a.s.batch, a.hq, a.s.G, gqa::RED_COL_PARTS);
  hipLaunchKernelGGL(gqa::reduce_kernel, rp.grid, dim3(REDUCE_THREADS), 0, stream, a, rp.by_segments ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dcp
