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

// Merge the split partials of request b, heads h0, h0 + hstep, ... .  A
// workgroup of DV/2 threads serves one request: it reads the request's split
// metadata once (a request held by one workgroup was written by the partial
// kernel itself and is skipped here), then per head computes the segment
// weights into LDS and streams its two output columns of every segment with
// independent loads.  Writes the normalized output and the natural-log LSE;
// a request with no local tokens gets (0, -inf).
template <int DV>
__device__ __forceinline__ void reduce_request(const SplitArgs& s, int heads, int b, int h0, int hstep,
                                               float* s_w) {
  constexpr int NT = DV / 2;
  const int tid = threadIdx.x;
  const int geff = s.ws_meta[0];
  const int pb = s.ws_meta[1 + b], pe = s.ws_meta[2 + b];
  const int T = s.ws_meta[1 + s.batch];
  if (pe <= pb || geff <= 0 || T <= 0) {
    for (int h = h0; h < heads; h += hstep) {
      *(float2*)(s.out + ((size_t)b * heads + h) * DV + 2 * tid) = make_float2(0.f, 0.f);
      if (tid == 0) s.lse[(size_t)b * heads + h] = -__builtin_inff();
    }
    return;
  }
  const int g0 = (int)(((int64_t)(pb + 1) * geff - 1) / T);
  const int g1 = (int)(((int64_t)pe * geff - 1) / T);
  if (g1 == g0) return;  // one workgroup held the whole request and wrote the result itself
  const int nseg = g1 - g0 + 1;  // <= kMaxSplitWGs
  __shared__ float s_red[NT / 64];
  for (int h = h0; h < heads; h += hstep) {
    float mloc = -__builtin_inff();
    for (int i = tid; i < nseg; i += NT) mloc = fmaxf(mloc, s.ws_ml[((size_t)(g0 + i + b) * heads + h) * 2]);
    mloc = wave_max(mloc);
    if ((tid & 63) == 0) s_red[tid >> 6] = mloc;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) M = fmaxf(M, s_red[i]);
    float lloc = 0.f;
    for (int i = tid; i < nseg; i += NT) {
      const size_t row = (size_t)(g0 + i + b) * heads + h;
      const float wgt = exp2_fast((s.ws_ml[row * 2] - M) * s.c);
      s_w[i] = wgt;
      lloc += wgt * s.ws_ml[row * 2 + 1];
    }
    lloc = wave_sum(lloc);
    __syncthreads();
    if ((tid & 63) == 0) s_red[tid >> 6] = lloc;
    __syncthreads();
    float Lsum = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) Lsum += s_red[i];
    float2 acc = make_float2(0.f, 0.f);
    const float* src = s.ws_o + ((size_t)(g0 + b) * heads + h) * DV + 2 * tid;
    const size_t seg_stride = (size_t)heads * DV;
    int i = 0;
    for (; i + 8 <= nseg; i += 8) {
      float2 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = *(const float2*)(src + (size_t)(i + u) * seg_stride);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc.x += s_w[i + u] * x[u].x;
        acc.y += s_w[i + u] * x[u].y;
      }
    }
    for (; i < nseg; ++i) {
      const float2 x = *(const float2*)(src + (size_t)i * seg_stride);
      acc.x += s_w[i] * x.x;
      acc.y += s_w[i] * x.y;
    }
    const float inv = 1.f / Lsum;
    *(float2*)(s.out + ((size_t)b * heads + h) * DV + 2 * tid) = make_float2(acc.x * inv, acc.y * inv);
    if (tid == 0) s.lse[(size_t)b * heads + h] = (M * s.c + __log2f(Lsum)) * kLn2;
    __syncthreads();  // s_w and s_red are reused by the next head
  }
}

// Grid for the split reduce: blocks.y = requests, blocks.x = head strides
// (enough blocks overall to cover the chip, one metadata read per block).
inline dim3 reduce_grid(int batch, int heads) {
  int per = 1024 / (batch > 0 ? batch : 1);
  if (per < 1) per = 1;
  if (per > heads) per = heads;
  return dim3(per, batch);
}

}  // namespace dcp
