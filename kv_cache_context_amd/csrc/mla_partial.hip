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
constexpr int NST = 4;                // tiles resident in LDS
constexpr int CPR = ROW / 16;         // 16-byte chunks per row (72)
constexpr int THREADS = 256;
constexpr int DMA_N = TILE * CPR / THREADS;  // copies per thread per tile (9)
constexpr int KS = DK / 32;           // k-steps of the score contraction (18)
constexpr int VB = R / 16;            // 16-column blocks of the value contraction (32)
static_assert(TILE * CPR % THREADS == 0, "tile copy split");

// Chunk swizzle of LDS row r (depends on r mod 16, value < 8 so a row's 72
// chunks stay inside their aligned groups of 8).  Chosen so that 16
// consecutive rows at one chunk, and 8 rows x 2 adjacent chunks, each fall in
// distinct 16-byte bank groups for 32- and 64-bank LDS.
__host__ __device__ constexpr int swz(int r) {
  r &= 15;
  const int hi = ((r >> 1) & 1) | (((r ^ (r >> 2)) & 1) << 1);
  const int lo = ((r >> 2) ^ (r >> 3)) & 1;
  return 2 * hi + lo;
}

struct Smem {
  char tiles[NST * STAGE];
  int pref[kMaxBatch + 1];
  int wsum[THREADS / 64];
};

__device__ __forceinline__ void issue_tile(const MlaArgs& a, const int32_t* trow, int lr, int k,
                                           DCP_LDS char* stage, const int (&goff)[DMA_N],
                                           const int (&grow)[DMA_N]) {
  const SplitArgs& s = a.s;
  const int B = s.block_size;
  const int tok0 = k * TILE;
  const int pg0 = uni(tok0 / B);
  const int in0 = tok0 - pg0 * B;
  const int split = B - in0;  // tile rows [0, split) are in block pg0, the rest in pg0 + 1
  const int mb1 = s.max_blocks - 1;
  int e0 = ld_uniform(trow, pg0 < mb1 ? pg0 : mb1);
  e0 = uni(min(max(e0, 0), s.num_blocks - 1));
  int e1 = e0;
  if (split < TILE) {
    e1 = ld_uniform(trow, pg0 + 1 < mb1 ? pg0 + 1 : mb1);
    e1 = uni(min(max(e1, 0), s.num_blocks - 1));
  }
  const char* kv = (const char*)a.kv;
  const char* base0 = kv + ((int64_t)e0 * B + in0) * ROW;
  const char* base1 = kv + ((int64_t)e1 * B - split) * ROW;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < DMA_N; ++i) {
    const char* src = (grow[i] < split ? base0 : base1) + goff[i];
    dma16(src, stage + (i * (THREADS / 64) + wave) * 1024);
  }
  (void)lr;
}

// Zero the tile rows at and past `valid` (the unused end of the last block),
// so stale cache contents can never reach the value contraction.
__device__ __forceinline__ void zero_tail(DCP_LDS char* stage, int valid) {
  const int start = valid * CPR;
  for (int c = start + (int)threadIdx.x; c < TILE * CPR; c += THREADS)
    *(DCP_LDS f32x4*)(stage + c * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ void compute_tile(const DCP_LDS char* st, int tok0, int lr,
                                             const bf16x8 (&qf)[KS], f32x4 (&acc)[VB], float& m,
                                             float& l, float c) {
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, r16 = lane & 15;

  // ---- scores S^T[tok][head], two 16-token blocks
  const int fz = swz(r16);
  const int offE = ((g4) ^ fz) * 16;
  const int offO = ((4 | g4) ^ fz) * 16;
  const DCP_LDS char* k0p = st + r16 * ROW;
  const DCP_LDS char* k1p = st + (16 + r16) * ROW;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int off = (ks >> 1) * 128 + ((ks & 1) ? offO : offE);
    const bf16x8 ka = *(const DCP_LDS bf16x8*)(k0p + off);
    const bf16x8 kb = *(const DCP_LDS bf16x8*)(k1p + off);
    s0 = mfma_16x16x32(ka, qf[ks], s0);
    s1 = mfma_16x16x32(kb, qf[ks], s1);
  }

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
  const float mnew = fmaxf(m, mt);
  const float alpha = exp2_fast((m - mnew) * c);
  const float mc = mnew * c;
  float p[8];
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = exp2_fast(fmaf(sv[j], c, -mc));
    ps += p[j];
  }
  l = l * alpha + ps;
  m = mnew;
  if (!__all(alpha == 1.f)) {
#pragma unroll
    for (int cb = 0; cb < VB; ++cb) acc[cb] *= alpha;
  }
  bf16x8 pt;
#pragma unroll
  for (int j = 0; j < 8; ++j) pt[j] = (__bf16)p[j];

  // ---- values O^T[col][head] += V^T[col][tok] . P^T[tok][head]
  const int rowa = 4 * g4 + (r16 >> 2);
  const int fa = swz(rowa);
  const int hb = (r16 & 3) >> 1;
  const int byte = (r16 & 1) * 8;
  const DCP_LDS char* va = st + rowa * ROW + byte;
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) voff[q] = (((2 * q) | hb) ^ fa) * 16;
#pragma unroll
  for (int cb = 0; cb < VB; ++cb) {
    const DCP_LDS char* p0 = va + (cb >> 2) * 128 + voff[cb & 3];
    const i16x4 v0 = lds_read_tr16(p0);
    const i16x4 v1 = lds_read_tr16(p0 + 16 * ROW);
    const i16x8 v8 = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc[cb] = mfma_16x16x32(__builtin_bit_cast(bf16x8, v8), pt, acc[cb]);
  }
}

__global__ __launch_bounds__(THREADS, 1) void partial_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem sm;
  const SplitArgs& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  // per-thread copy pattern of a tile: LDS chunk slot -> source chunk (swizzled)
  int goff[DMA_N], grow[DMA_N];
#pragma unroll
  for (int i = 0; i < DMA_N; ++i) {
    const int slot = (i * (THREADS / 64) + wave) * 64 + lane;
    const int r = slot / CPR, ch = slot % CPR;
    grow[i] = r;
    goff[i] = r * ROW + ((ch ^ swz(r)) * 16);
  }

  DCP_LDS char* tiles = (DCP_LDS char*)sm.tiles;
  const int heads = a.heads;
  const bool active = wave * 16 < heads;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int head = wave * 16 + r16;

  int b = find_request(sm.pref, s.batch, p0);
  for (;;) {
    const int pb = uni(sm.pref[b]), pe = uni(sm.pref[b + 1]);
    if (pe > pb) {
      const int t0 = (p0 > pb ? p0 : pb) - pb;
      const int t1 = (p1 < pe ? p1 : pe) - pb;
      const int n = t1 - t0;
      const int lr = uni(clamped_local_len(s, b));
      const int32_t* trow = s.table + (int64_t)b * s.max_blocks;

      bf16x8 qf[KS];
      if (active) {
        const bf16x8* qp =
            (const bf16x8*)(a.q + ((int64_t)b * heads + head) * DK + 8 * g4);
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

      issue_tile(a, trow, lr, t0, tiles, goff, grow);
      if (n > 1) issue_tile(a, trow, lr, t0 + 1, tiles + STAGE, goff, grow);
      if (n > 2) issue_tile(a, trow, lr, t0 + 2, tiles + 2 * STAGE, goff, grow);
      for (int i = 0; i < n; ++i) {
        const int k = t0 + i;
        const int rem = n - 1 - i;
        if (rem >= 2) wait_vmcnt<2 * DMA_N>();
        else if (rem == 1) wait_vmcnt<DMA_N>();
        else wait_vmcnt<0>();
        barrier();
        DCP_LDS char* cur = tiles + (i % NST) * STAGE;
        const int valid = lr - k * TILE;
        if (valid < TILE) {  // last tile of the request: clear rows past the end
          zero_tail(cur, valid);
          wait_lgkm0();
          barrier();
        }
        if (i + 3 < n) issue_tile(a, trow, lr, k + 3, tiles + ((i + 3) % NST) * STAGE, goff, grow);
        if (active) compute_tile(cur, k * TILE, lr, qf, acc, m, l, s.c);
      }
      barrier();  // every wave is done with the tiles before the next segment refills them

      if (active) {
        const int slot = g + b;
        const float lt = wave_sum16(l);
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
    if (pe >= p1 || b + 1 >= s.batch) break;
    ++b;
  }
}

__global__ __launch_bounds__(256) void reduce_kernel(MlaArgs a) {
  const int b = blockIdx.y;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (h >= a.heads) return;
  reduce_row<R>(a.s, a.heads, b, h);
}

}  // namespace mla

hipError_t launch_mla_partial(const MlaArgs& a, hipStream_t stream) {
  if (a.s.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(mla::partial_kernel, dim3(a.s.G), dim3(mla::THREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla::reduce_kernel, dim3((a.heads + 3) / 4, a.s.batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dcp
