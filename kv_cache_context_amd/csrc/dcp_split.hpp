// Split planning and split reduction shared by the MLA and GQA partial kernels.
//
// A shard's local work is a list of tiles (fixed token count each): request b
// contributes ceil(L_r(b) / tile) tiles, where L_r(b) is its local length on
// this shard.  The G_eff split workgroups take equal contiguous ranges of the
// concatenated tile list ("stream-K"), so ragged batches stay balanced and no
// host read of seq_lens is needed.  Workgroup g owns tiles
// [floor(g*T/G_eff), floor((g+1)*T/G_eff)); a range may span several requests
// and a request may span several workgroups.  Each (workgroup, request) piece
// writes one partial state into slot g + b, which is unique along the
// monotone path the pieces follow.  The reduce kernel merges the slots of each
// request with the same LSE rule the cross-shard combine uses.
#pragma once

#include "dcp_device.hpp"
#include "dcp_internal.hpp"

namespace dcp {

__device__ __forceinline__ int clamp_len(const SplitArgs& s, int L) {
  const int lr = local_len(L, s.nshards, s.rank, s.layout);
  const int cap = s.max_blocks * s.block_size;  // what one table row can address
  return lr < cap ? lr : cap;
}
// Local length of request b (b wave-uniform).
__device__ __forceinline__ int clamped_local_len(const SplitArgs& s, int b) {
  return uni(clamp_len(s, ld_uniform(s.seq_lens, b)));
}

// Fills s_pref[0..batch] with the inclusive prefix sums of tiles per request
// (s_pref[0] = 0) and returns the total T.  All threads of the block call it.
template <int THREADS>
__device__ int plan_tiles(const SplitArgs& s, int tile, int* s_pref, int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = THREADS / 64;
  int carry = 0;
  for (int base = 0; base < s.batch; base += THREADS) {
    const int b = base + tid;
    int n = 0;
    if (b < s.batch) n = (clamp_len(s, s.seq_lens[b]) + tile - 1) / tile;
    int v = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) s_wsum[wave] = v;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int x = s_wsum[w];
      woff += (w < wave) ? x : 0;
      tot += x;
    }
    if (b < s.batch) s_pref[b + 1] = carry + woff + v;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
  return uni(carry);
}

__device__ __forceinline__ int split_wgs(const SplitArgs& s, int T) {
  if (T <= 0) return 0;
  const int want = (T + s.min_tiles - 1) / s.min_tiles;
  return want < s.G ? want : s.G;
}

// Largest b in [0, batch) with s_pref[b] <= p (the request holding tile p,
// skipping requests that have no tiles).
__device__ __forceinline__ int find_request(const int* s_pref, int batch, int p) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uni(s_pref[mid]) <= p) lo = mid; else hi = mid - 1;
  }
  return uni(lo);
}

// Merge the split partials of one (request, head) row.  One wave per row;
// lane i handles dv/64 consecutive outputs.  Writes the normalized output and
// the natural-log LSE; a request with no local tokens gets (0, -inf).
template <int DV>
__device__ __forceinline__ void reduce_row(const SplitArgs& s, int heads, int b, int h) {
  static_assert(DV % 256 == 0 || DV == 128, "dv");
  constexpr int PER = DV / 64;  // floats per lane
  const int lane = threadIdx.x & 63;
  const int geff = s.ws_meta[0];
  const int pb = s.ws_meta[1 + b], pe = s.ws_meta[2 + b];
  const int T = s.ws_meta[1 + s.batch];
  float* orow = s.out + ((size_t)b * heads + h) * DV + lane * PER;
  if (pe <= pb || geff <= 0 || T <= 0) {
#pragma unroll
    for (int i = 0; i < PER; i += 4) *(f32x4*)(orow + i) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane == 0) s.lse[(size_t)b * heads + h] = -__builtin_inff();
    return;
  }
  const int g0 = (int)(((int64_t)(pb + 1) * geff - 1) / T);
  const int g1 = (int)(((int64_t)pe * geff - 1) / T);
  float M = -__builtin_inff();
  for (int g = g0; g <= g1; ++g) M = fmaxf(M, s.ws_ml[((size_t)(g + b) * heads + h) * 2]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float Lsum = 0.f;
  for (int g = g0; g <= g1; ++g) {
    const size_t row = (size_t)(g + b) * heads + h;
    const float mg = s.ws_ml[row * 2];
    const float lg = s.ws_ml[row * 2 + 1];
    const float w = exp2_fast((mg - M) * s.c);
    Lsum += w * lg;
    const float* src = s.ws_o + row * DV + lane * PER;
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const f32x4 x = *(const f32x4*)(src + i);
      acc[i] += w * x[0];
      acc[i + 1] += w * x[1];
      acc[i + 2] += w * x[2];
      acc[i + 3] += w * x[3];
    }
  }
  const float inv = 1.f / Lsum;
#pragma unroll
  for (int i = 0; i < PER; i += 4)
    *(f32x4*)(orow + i) = f32x4{acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
  if (lane == 0) s.lse[(size_t)b * heads + h] = (M * s.c + __log2f(Lsum)) * kLn2;
}

}  // namespace dcp
