// Shard-local GQA decode attention for gfx950.
//
// What one shard computes (vLLM blog post on Decode Context Parallelism,
// sections 4.1 and 5.4): query head h attends KV head g = floor(h * Hkv / Hq)
// over the shard's local tokens; the result is the normalized partial output and
// its natural-log LSE, merged across shards by dcp_combine.
//
// Structure (per split workgroup of 4 waves, one per SIMD):
//  * A workgroup owns HG consecutive KV heads (HG = 4, 2 or 1: the largest that
//    divides Hkv) and streams 16 KiB of K and 16 KiB of V per tile: 16 * SUB
//    tokens x HG heads, SUB = 4 / HG.  The 4 waves are (KV head of the group,
//    16-token sub-tile): with 4 heads every wave takes the whole tile of its
//    head; with 1 head (the DCP post's example of one KV head per rank) the
//    four waves take a quarter of the tokens each.  Copies go HBM -> LDS with
//    direct global->LDS copies, 4 tiles (32 KiB each) resident; each K/V byte is
//    read from HBM once and from LDS once.
//  * Scores, transposed: S^T[16 tok x 16] = K[16 x 128] . q^T with
//    v_mfma_f32_16x16x32_bf16, for each 16-head block of the KV head's query
//    group (up to 4 blocks: 64 query heads per KV head); a group smaller than 16
//    zero-pads the block's columns.
//  * Online softmax in base 2 with rescaling when a head's maximum grows.
//  * Values: O^T[128 x 16] += V^T[128 x 16 tok] . P^T with
//    v_mfma_f32_16x16x16_bf16; V^T comes from ds_read_b64_tr_b16, and the score
//    tile's register layout is already the P^T operand layout.
//  * Waves of one KV head that took different sub-tiles merge their (max, sum,
//    output) states through LDS at the end of a segment (the same rule as the
//    split and shard merges).
//  * Stream-K split over tiles and the split reduce are shared with MLA.
#include "dcp_device.hpp"
#include "dcp_internal.hpp"
#include "dcp_split.hpp"
#include "gqa_layout.hpp"

namespace dcp {
namespace gqa {

// (head dim, part size, copy slots and the operand offsets: gqa_layout.hpp)
constexpr int STAGE = 2 * HALF;        // K then V
constexpr int NST = 4;
constexpr int THREADS = 256;
constexpr int DMA_N = 2 * CPI;         // copies per wave per tile (8)
constexpr int KS = D / 32;             // score k-steps (4)
constexpr int VB = D / 16;             // value column blocks (8)
constexpr int TBL = 1024;

// Segment-end exchange of the waves of one KV head (SUB > 1): per (head,
// sub-tile >= 1, query block) slot, the output block and each column's
// reference and sum.  Overlays the tile ring, which is idle by then.
struct MergeSlot {
  f32x4 acc[VB][64];
  float m[16], l[16];
};
static_assert(12 * sizeof(MergeSlot) <= NST * STAGE, "merge slots fit the tile ring");

struct Smem {
  char tiles[NST * STAGE];
  int pref[kMaxBatch + 1];
  int tbl[TBL];
  int wsum[THREADS / 64];
};

struct TileCopy {
  const char* kbase;  // K cache address of (token 0 of the wave's copy sub-tile, head HG*group)
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

// Addresses of tile k's copies for this wave.  The wave copies (part of) one
// 16-token sub-tile, which lies in one cache block (B is a multiple of 16); a
// sub-tile past the request's end copies sub-tile 0's rows instead (in bounds;
// the rows are zeroed before use), so every wave issues the same copies.
template <int HG>
__device__ __forceinline__ TileCopy plan_copy(const GqaArgs& a, const int32_t* trow, Smem& sm, TableWin& win,
                                              int pg_hi, int lr, int group, int k, DCP_LDS char* stage,
                                              bool valid) {
  using G = Geo<HG>;
  TileCopy t;
  t.valid = valid;
  t.stage = stage;
  const SplitArgs& s = a.s;
  const int B = s.block_size;
  const int wave = uni(threadIdx.x >> 6);
  const int tok0 = k * G::TILE;
  int sub_tok = tok0 + 16 * (wave / HG);  // first token of the wave's copy sub-tile
  if (sub_tok >= lr) sub_tok = tok0;
  const int pg = uni(sub_tok / B);
  const int in0 = sub_tok - pg * B;
  int e = 0;
  if (valid) {
    // the window must hold every valid sub-tile's block (a workgroup-uniform test)
    const int pg_need = uni(min((min(tok0 + G::TILE, lr) - 1) / B, pg_hi - 1));
    if (pg_need >= win.end) {  // slide the window (rare)
      barrier();
      const int lo = uni(tok0 / B);
      load_window(a, trow, sm, lo, pg_hi);
      wait_vmcnt<0>();
      wait_lgkm0();
      barrier();
      win.lo = lo;
      win.end = min(pg_hi, lo + TBL);
    }
    e = uni(sm.tbl[pg - win.lo]);
  }
  const int64_t off = (((int64_t)e * B + in0) * a.hkv + (int64_t)group * HG) * HROW;
  t.kbase = (const char*)a.k + off;
  t.vbase = (const char*)a.v + off;
  return t;
}

// Copy i of a tile for this wave: i < CPI -> K, else V.
template <int HG>
__device__ __forceinline__ void copy_part(const TileCopy& t, int i, const uint32_t (&voff)[CPI]) {
  if (!t.valid) return;
  const int wave = uni(threadIdx.x >> 6);
  const int j = i % CPI;
  DCP_LDS char* dst = t.stage + (i < CPI ? 0 : HALF) + copy_dst_offset<HG>(wave, j, 0);
  dma16_sbase(i < CPI ? t.kbase : t.vbase, voff[j], dst);
}

template <int HG>
__device__ __forceinline__ void copy_all(const TileCopy& t, const uint32_t (&voff)[CPI]) {
#pragma unroll
  for (int i = 0; i < DMA_N; ++i) copy_part<HG>(t, i, voff);
}

template <int HG>
__device__ __forceinline__ void zero_tail(DCP_LDS char* stage, int valid) {
  using G = Geo<HG>;
  // rows past the end, in both the K and the V half
  for (int c = valid * (G::TROW / 16) + (int)threadIdx.x; c < G::TILE * (G::TROW / 16); c += THREADS) {
    *(DCP_LDS f32x4*)(stage + c * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
    *(DCP_LDS f32x4*)(stage + HALF + c * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// One 16-token sub-tile for the wave's KV head hk: `st` is the tile's stage,
// `sub` the wave's sub-tile and tok0 its first token.
template <int HG, int NQB>
__device__ __forceinline__ void compute_tile(const DCP_LDS char* st, int sub, int tok0, int lr, int hk,
                                             const bf16x8 (&qf)[NQB][KS], f32x4 (&acc)[NQB][VB],
                                             float (&m)[NQB], float (&l)[NQB], float c, const TileCopy& nxt,
                                             const uint32_t (&voff)[CPI]) {
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, r16 = lane & 15;
  // ---- scores S^T[tok][head col]: A = K row (token r16 of the sub-tile), B = q^T
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const DCP_LDS bf16x8*)(st + k_read_offset<HG>(sub, r16, hk, 4 * ks + g4));
  copy_part<HG>(nxt, 0, voff);
  copy_part<HG>(nxt, 1, voff);
  f32x4 sc[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    sc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc[qb] = mfma_16x16x32(kf[ks], qf[qb][ks], sc[qb]);
  }
  copy_part<HG>(nxt, 2, voff);
  copy_part<HG>(nxt, 3, voff);

  // ---- online softmax: lane holds head col r16 of each block, tokens 4*g4 + i
  i16x4 pt[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float sv[4] = {sc[qb][0], sc[qb][1], sc[qb][2], sc[qb][3]};
    if (tok0 + 16 > lr) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok0 + 4 * g4 + i >= lr) sv[i] = -__builtin_inff();
    }
    float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mt = wave_max16(mt);
    const float mnew = fmaxf(m[qb], mt);
    const float alpha = exp2_fast((m[qb] - mnew) * c);  // 0 while m is -inf
    l[qb] *= alpha;
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int cb = 0; cb < VB; ++cb) acc[qb][cb] *= alpha;
    }
    m[qb] = mnew;
    const float mc = mnew * c;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2_fast(fmaf(sv[i], c, -mc));
      ps += p;
      pt[qb][i] = __builtin_bit_cast(short, (__bf16)p);
    }
    l[qb] += ps;
  }
  copy_part<HG>(nxt, 4, voff);
  copy_part<HG>(nxt, 5, voff);

  // ---- values O^T[col][head] += V^T[col][tok] . P^T[tok][head]
  i16x4 vt[VB];
#pragma unroll
  for (int cb = 0; cb < VB; ++cb) vt[cb] = lds_read_tr16(st + HALF + v_read_offset<HG>(sub, g4, r16, hk, cb));
  copy_part<HG>(nxt, 6, voff);
  copy_part<HG>(nxt, 7, voff);
#pragma unroll
  for (int cb = 0; cb < VB; ++cb)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) acc[qb][cb] = mfma_16x16x16(vt[cb], pt[qb], acc[qb][cb]);
}

template <int HG, int NQB>
__device__ __forceinline__ void run_segment(const GqaArgs& a, Smem& sm, int group, int b, int t0, int t1,
                                            int ntiles_b, int g) {
  using G = Geo<HG>;
  const SplitArgs& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int gs = a.hq / a.hkv;               // query heads per KV head (<= 16 NQB)
  const int hk = wave % HG;                   // KV head within the group
  const int sub = wave / HG;                  // 16-token sub-tile of every tile
  const int kvh = group * HG + hk;            // KV head index
  const int g4 = lane >> 4, r16 = lane & 15;
  DCP_LDS char* tiles = (DCP_LDS char*)sm.tiles;
  const int n = t1 - t0;
  const int lr = uni(clamped_local_len(s, b));
  const int32_t* trow = table_row(s, b);

  // lane offsets of the copies from the wave's sub-tile base
  uint32_t voff[CPI];
#pragma unroll
  for (int j = 0; j < CPI; ++j) voff[j] = copy_src_offset<HG>(wave, j, lane, a.hkv);

  bf16x8 qf[NQB][KS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int col = 16 * qb + r16;
    const bool ok = col < gs;
    const bf16x8* qp = (const bf16x8*)(a.q + ((int64_t)b * a.hq + (ok ? kvh * gs + col : 0)) * D + 8 * g4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks] = qp[4 * ks];
      if (!ok) qf[qb][ks] = bf16x8{};
    }
  }
  f32x4 acc[NQB][VB];
  float m[NQB], l[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
    for (int cb = 0; cb < VB; ++cb) acc[qb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[qb] = -__builtin_inff();
    l[qb] = 0.f;
  }

  const int pg_lo = uni((t0 * G::TILE) / s.block_size);
  const int pg_hi = uni(min(s.max_blocks, (min(t1 * G::TILE, lr) - 1) / s.block_size + 1));
  TableWin win{pg_lo, min(pg_hi, pg_lo + TBL)};
  load_window(a, trow, sm, pg_lo, pg_hi);  // in flight together with the q loads
  wait_vmcnt<0>();
  wait_lgkm0();
  barrier();
  // q has arrived (vmcnt 0); tie it here so the compiler places no wait for it
  // inside the tile loop, where it would drain the copy prefetch.
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[qb][ks]));

  copy_all<HG>(plan_copy<HG>(a, trow, sm, win, pg_hi, lr, group, t0, tiles, true), voff);
  if (n > 1) copy_all<HG>(plan_copy<HG>(a, trow, sm, win, pg_hi, lr, group, t0 + 1, tiles + STAGE, true), voff);
  if (n > 2) copy_all<HG>(plan_copy<HG>(a, trow, sm, win, pg_hi, lr, group, t0 + 2, tiles + 2 * STAGE, true), voff);
  for (int i = 0; i < n; ++i) {
    const int k = t0 + i;
    const int rem = n - 1 - i;
    if (rem >= 2) wait_vmcnt<2 * DMA_N>();
    else if (rem == 1) wait_vmcnt<DMA_N>();
    else wait_vmcnt<0>();
    barrier();
    DCP_LDS char* cur = tiles + (i % NST) * STAGE;
    const int valid = lr - k * G::TILE;
    if (valid < G::TILE) {
      zero_tail<HG>(cur, valid);
      wait_lgkm0();
      barrier();
    }
    const TileCopy nxt = plan_copy<HG>(a, trow, sm, win, pg_hi, lr, group, k + 3,
                                       tiles + ((i + 3) % NST) * STAGE, i + 3 < n);
    const int tok0 = k * G::TILE + 16 * sub;
    if (tok0 < lr) {
      compute_tile<HG, NQB>(cur, sub, tok0, lr, hk, qf, acc, m, l, s.c, nxt, voff);
    } else {
      // the wave's sub-tile is past the request's end: only the copies
#pragma unroll
      for (int c = 0; c < DMA_N; ++c) copy_part<HG>(nxt, c, voff);
    }
  }
  barrier();

  float lt[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) lt[qb] = wave_sum16(l[qb]);

  if constexpr (G::SUB > 1) {
    // the waves of sub-tiles 1.. hand their states to sub-tile 0's wave
    MergeSlot* ms = (MergeSlot*)sm.tiles;
    if (sub > 0) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        MergeSlot& d = ms[(hk * (G::SUB - 1) + sub - 1) * NQB + qb];
#pragma unroll
        for (int cb = 0; cb < VB; ++cb) d.acc[cb][lane] = acc[qb][cb];
        if (g4 == 0) {
          d.m[r16] = m[qb];
          d.l[r16] = lt[qb];
        }
      }
    }
    wait_lgkm0();
    barrier();
    if (sub == 0) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        // the owner's own first sub-tile is inside the request, so mx is finite
        float mx = m[qb];
#pragma unroll
        for (int u = 1; u < G::SUB; ++u) mx = fmaxf(mx, ms[(hk * (G::SUB - 1) + u - 1) * NQB + qb].m[r16]);
        const float w0 = exp2_fast((m[qb] - mx) * s.c);
        float L = w0 * lt[qb];
#pragma unroll
        for (int cb = 0; cb < VB; ++cb) acc[qb][cb] *= w0;
#pragma unroll
        for (int u = 1; u < G::SUB; ++u) {
          const MergeSlot& d = ms[(hk * (G::SUB - 1) + u - 1) * NQB + qb];
          const float wu = exp2_fast((d.m[r16] - mx) * s.c);  // 0 for a wave that saw no token
          L += wu * d.l[r16];
#pragma unroll
          for (int cb = 0; cb < VB; ++cb) acc[qb][cb] += wu * d.acc[cb][lane];
        }
        m[qb] = mx;
        lt[qb] = L;
      }
    }
  }

  if (sub == 0) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int col = 16 * qb + r16;
      if (col >= gs) continue;
      const int qh = kvh * gs + col;
      if (t0 == 0 && t1 == ntiles_b) {
        const float inv = 1.f / lt[qb];
        float* dst = s.out + ((size_t)b * a.hq + qh) * D + 4 * g4;
#pragma unroll
        for (int cb = 0; cb < VB; ++cb) *(f32x4*)(dst + 16 * cb) = acc[qb][cb] * inv;
        if (g4 == 0) s.lse[(size_t)b * a.hq + qh] = (m[qb] * s.c + __log2f(lt[qb])) * kLn2;
      } else {
        const int slot = g + b;
        float* dst = (float*)s.ws_o + ((size_t)slot * a.hq + qh) * D + 4 * g4;
#pragma unroll
        for (int cb = 0; cb < VB; ++cb) *(f32x4*)(dst + 16 * cb) = acc[qb][cb];
        if (g4 == 0) {
          float* ml = s.ws_ml + ((size_t)slot * a.hq + qh) * 2;
          ml[0] = m[qb];
          ml[1] = lt[qb];
        }
      }
    }
  }
  if constexpr (G::SUB > 1) barrier();  // the merge slots are read before the ring is refilled
}

template <int HG, int NQB>
__global__ __launch_bounds__(THREADS, 1) void partial_kernel(GqaArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem sm;
  const SplitArgs& s = a.s;
  const int tid = threadIdx.x;
  const int g = blockIdx.x, group = blockIdx.y;
  const int T = plan_tiles<THREADS>(s, Geo<HG>::TILE, sm.pref, sm.wsum);
  const int geff = split_wgs(s, T);
  if (g == 0 && group == 0) {
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
    if (pe > pb && st.t1 > st.t0) run_segment<HG, NQB>(a, sm, group, b, st.t0, st.t1, st.ntiles, g);
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

template <int HG>
void launch_hg(const GqaArgs& a, int nqb, hipStream_t stream) {
  const dim3 grid(a.s.G, a.hkv / HG);
  switch (nqb) {
    case 1: hipLaunchKernelGGL((partial_kernel<HG, 1>), grid, dim3(THREADS), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((partial_kernel<HG, 2>), grid, dim3(THREADS), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((partial_kernel<HG, 3>), grid, dim3(THREADS), 0, stream, a); break;
    default: hipLaunchKernelGGL((partial_kernel<HG, 4>), grid, dim3(THREADS), 0, stream, a); break;
  }
}

}  // namespace gqa

int gqa_heads_per_workgroup(int hkv) { return hkv % 4 == 0 ? 4 : hkv % 2 == 0 ? 2 : 1; }
int gqa_tile_tokens(int hkv) { return 64 / gqa_heads_per_workgroup(hkv); }

hipError_t launch_gqa_partial(const GqaArgs& a, hipStream_t stream) {
  if (a.s.batch == 0) return hipSuccess;
  const int nqb = (a.hq / a.hkv + 15) / 16;
  switch (gqa_heads_per_workgroup(a.hkv)) {
    case 4: gqa::launch_hg<4>(a, nqb, stream); break;
    case 2: gqa::launch_hg<2>(a, nqb, stream); break;
    default: gqa::launch_hg<1>(a, nqb, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const ReducePlan rp = reduce_plan(a.s.batch, a.hq, a.s.G, gqa::RED_COL_PARTS);
  hipLaunchKernelGGL(gqa::reduce_kernel, rp.grid, dim3(REDUCE_THREADS), 0, stream, a, rp.by_segments ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dcp
