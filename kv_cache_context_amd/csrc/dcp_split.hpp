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

// Local length attended by row set b: request b / q_len, query token j =
// b % q_len, whose causal prefix is the first L - q_len + 1 + j of the
// request's L global positions.  The shard's part of the cache is cut from the
// full length L (for the contiguous layout, runs of ceil(L / N)); the result is
// capped at what one table row can address.
__host__ __device__ __forceinline__ int clamp_len(const SplitArgs& s, int L, int j) {
  int lr;
  if (s.q_len <= 1 || s.layout == 0) {
    lr = local_len(s.q_len <= 1 ? L : L - s.q_len + 1 + j, s.nshards, s.rank, s.layout);
  } else {
    const int lim = L - s.q_len + 1 + j;  // positions below lim are attended
    const int64_t c = ((int64_t)(L > 0 ? L : 0) + s.nshards - 1) / s.nshards;
    const int64_t lo = c * s.rank;
    int64_t hi = lo + c;
    if (hi > L) hi = L;
    if (hi > lim) hi = lim;
    lr = hi > lo ? (int)(hi - lo) : 0;
  }
  const int cap = s.max_blocks * s.block_size;  // what one table row can address
  return lr < cap ? lr : cap;
}
// Local length of row set b (b wave-uniform).
__device__ __forceinline__ int clamped_local_len(const SplitArgs& s, int b) {
  const int req = b / s.q_len;
  return uni(clamp_len(s, ld_uniform(s.seq_lens, req), b - req * s.q_len));
}
// Block-table row of row set b.
__device__ __forceinline__ const int32_t* table_row(const SplitArgs& s, int b) {
  return s.table + (int64_t)(b / s.q_len) * s.max_blocks;
}

// Fills s_pref[0..batch] with the inclusive prefix sums of the requests' work
// (s_pref[0] = 0) and returns the total T.  A request of n > 0 tiles weighs
// n + seg_cost: a segment boundary inside a workgroup's range costs the end of
// one segment (pipeline drain, partial write) and the start of the next
// (block-table window, q, pipeline fill), so the request's positions carry
// seg_head = seg_cost / 2 charge positions before its tiles and the rest after
// them, and the stream-K split hands a workgroup whose range holds a boundary
// that many fewer tiles.  Two workgroups that meet at a request boundary pay
// one segment end and one segment start between them, so the halves keep
// them balanced too.  Request b's tile k sits at position s_pref[b] + seg_head + k.
// All threads of the block call it.
template <int THREADS>
__device__ int plan_tiles(const SplitArgs& s, int tile, int* s_pref, int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = THREADS / 64;
  int carry = 0;
  for (int base = 0; base < s.batch; base += THREADS) {
    const int b = base + tid;
    int n = 0;
    if (b < s.batch) {
      const int req = b / s.q_len;
      n = (clamp_len(s, s.seq_lens[req], b - req * s.q_len) + tile - 1) / tile;
    }
    if (n > 0) n += s.seg_cost;
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

__host__ __device__ __forceinline__ int seg_head(const SplitArgs& s) { return s.seg_cost >> 1; }
__host__ __device__ __forceinline__ int seg_tail(const SplitArgs& s) { return s.seg_cost - (s.seg_cost >> 1); }

// Tiles [t0, t1) of request b (positions [pb, pe)) that fall in the workgroup's
// positions [p0, p1); empty (t1 <= t0) when the range holds only charge
// positions of the request or nothing of it.
struct SegTiles {
  int t0, t1, ntiles;
};
__host__ __device__ __forceinline__ SegTiles seg_tiles(const SplitArgs& s, int pb, int pe, int p0, int p1) {
  const int r0 = pb + seg_head(s);  // position of tile 0
  const int re = pe - seg_tail(s);  // position after the last tile
  SegTiles t;
  t.t0 = (p0 > r0 ? p0 : r0) - r0;
  t.t1 = (p1 < re ? p1 : re) - r0;
  t.ntiles = re - r0;
  return t;
}

__host__ __device__ __forceinline__ int split_wgs(const SplitArgs& s, int T) {
  if (T <= 0) return 0;
  const int want = (T + s.min_tiles - 1) / s.min_tiles;
  return want < s.G ? want : s.G;
}

// Largest b in [0, batch) with s_pref[b] <= p (the request holding position p,
// skipping requests that have no tiles).
__device__ __forceinline__ int find_request(const int* s_pref, int batch, int p) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uni(s_pref[mid]) <= p) lo = mid; else hi = mid - 1;
  }
  return uni(lo);
}

// ---------------------------------------------------------------- split reduce
//
// Request b's tiles [pb + seg_head, pe - seg_tail) of the stream-K partition (T positions
// over geff workgroups) were covered by workgroups g0..g1; workgroup g wrote the
// un-normalized (m, l, o) of request b to slot g + b.  A request held by one
// workgroup was finished by that workgroup and is skipped here; a request with
// no local tokens gets (0, -inf).  The merge of segments i is
//   M = max m_i, w_i = exp2((m_i - M) c), L = sum w_i l_i,
//   o = sum w_i o_i / L, lse = (M c + log2 L) ln 2.
// Two block mappings (blocks of REDUCE_THREADS = 8 waves), chosen by the host
// from the launch shape; both give the same result:
//  * by heads (many requests, few segments each): block (head group of 8,
//    request); wave w merges head w of the group, each lane DV/64 columns,
//    all segments.
//  * by segments (few requests, many segments): block (column part, head,
//    request); the 8 waves take every 8th segment (8 loads in flight per
//    lane) and add their sums in LDS.
constexpr int REDUCE_THREADS = 512;
constexpr int kReduceHeads = 8;  // heads per block in the by-heads mapping
static_assert(kReduceHeads <= REDUCE_THREADS / 64, "one head per wave in the by-heads mapping");

struct SegRange {
  int g0, nseg;  // first segment slot offset and segment count; nseg 0: empty request
};

__host__ __device__ __forceinline__ SegRange seg_range(const SplitArgs& s, int b) {
  const int geff = s.ws_meta[0];
  const int pb = s.ws_meta[1 + b], pe = s.ws_meta[2 + b];
  const int T = s.ws_meta[1 + s.batch];
  if (pe <= pb || geff <= 0 || T <= 0) return {0, 0};
  // workgroups holding the request's first and last tile
  const int g0 = (int)(((int64_t)(pb + seg_head(s) + 1) * geff - 1) / T);
  const int g1 = (int)(((int64_t)(pe - seg_tail(s)) * geff - 1) / T);
  return {g0, g1 - g0 + 1};
}

// Segment weights of heads h0 .. h0 + nh - 1 (nh <= kReduceHeads) into
// s_w[j * kMaxSplitWGs + i], with s_M[j] = max m_i (raw score units) and
// s_L[j] = sum w_i l_i.  Wave w handles head j = w.
__device__ __forceinline__ void seg_weights(const SplitArgs& s, int heads, int b, const SegRange& r, int h0,
                                            int nh, float* s_w, float* s_M, float* s_L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = wave; j < nh; j += REDUCE_THREADS / 64) {
    const int h = h0 + j;
    float mx = -__builtin_inff();
    for (int i = lane; i < r.nseg; i += 64) mx = fmaxf(mx, s.ws_ml[((size_t)(r.g0 + i + b) * heads + h) * 2]);
    mx = wave_max(mx);
    float L = 0.f;
    for (int i = lane; i < r.nseg; i += 64) {
      const size_t row = (size_t)(r.g0 + i + b) * heads + h;
      const float w = exp2_fast((s.ws_ml[row * 2] - mx) * s.c);
      s_w[j * kMaxSplitWGs + i] = w;
      L += w * s.ws_ml[row * 2 + 1];
    }
    L = wave_sum(L);
    if (lane == 0) {
      s_M[j] = mx;
      s_L[j] = L;
    }
  }
  __syncthreads();
}

// Segment weights of one head h, the whole block working: thread t takes
// segment t (nseg <= kMaxSplitWGs = REDUCE_THREADS), so every (m, l) pair is
// read in one round trip.  Same results as seg_weights with nh = 1, into
// s_w[i], s_M[0], s_L[0].
static_assert(kMaxSplitWGs <= REDUCE_THREADS, "one segment per thread");
__device__ __forceinline__ void seg_weights_one(const SplitArgs& s, int heads, int b, const SegRange& r, int h,
                                                float* s_w, float* s_M, float* s_L, float (&red)[2][REDUCE_THREADS / 64]) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  float2 ml = make_float2(-__builtin_inff(), 0.f);
  if (t < r.nseg) ml = *(const float2*)(s.ws_ml + ((size_t)(r.g0 + t + b) * heads + h) * 2);
  const float wm = wave_max(ml.x);
  if (lane == 0) red[0][wave] = wm;
  __syncthreads();
  float mx = red[0][0];
#pragma unroll
  for (int w = 1; w < REDUCE_THREADS / 64; ++w) mx = fmaxf(mx, red[0][w]);
  const float wgt = t < r.nseg ? exp2_fast((ml.x - mx) * s.c) : 0.f;
  if (t < r.nseg) s_w[t] = wgt;
  const float ws = wave_sum(wgt * ml.y);
  if (lane == 0) red[1][wave] = ws;
  __syncthreads();
  if (t == 0) {
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < REDUCE_THREADS / 64; ++w) L += red[1][w];
    s_M[0] = mx;
    s_L[0] = L;
  }
  __syncthreads();
}

template <int N>
struct FVec {
  float v[N];
};
// N consecutive partial columns as fp32, from fp32 or bf16 (uint16_t bits)
// storage.
template <int N, typename T>
__device__ __forceinline__ FVec<N> load_cols(const T* p) {
  FVec<N> r;
  if constexpr (sizeof(T) == 2) {
    static_assert(N == 2 || N == 4 || N % 8 == 0, "bf16 column run");
    uint32_t w[N / 2];
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int k = 0; k < N / 8; ++k) {
        const uint4 x = *(const uint4*)(p + 8 * k);
        w[4 * k] = x.x;
        w[4 * k + 1] = x.y;
        w[4 * k + 2] = x.z;
        w[4 * k + 3] = x.w;
      }
    } else if constexpr (N == 4) {
      const uint2 x = *(const uint2*)p;
      w[0] = x.x;
      w[1] = x.y;
    } else {
      w[0] = *(const uint32_t*)p;
    }
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
      r.v[2 * k] = __uint_as_float(w[k] << 16);
      r.v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const float4 x = *(const float4*)(p + 4 * k);
      r.v[4 * k] = x.x;
      r.v[4 * k + 1] = x.y;
      r.v[4 * k + 2] = x.z;
      r.v[4 * k + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    const float2 x = *(const float2*)p;
    r.v[0] = x.x;
    r.v[1] = x.y;
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) r.v[k] = p[k];
  }
  return r;
}
template <int N>
__device__ __forceinline__ void store_cols(float* p, const FVec<N>& r) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k)
      *(float4*)(p + 4 * k) = make_float4(r.v[4 * k], r.v[4 * k + 1], r.v[4 * k + 2], r.v[4 * k + 3]);
  } else if constexpr (N == 2) {
    *(float2*)p = make_float2(r.v[0], r.v[1]);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) p[k] = r.v[k];
  }
}

struct ReduceSmem {
  float w[kReduceHeads * kMaxSplitWGs];
  float M[kReduceHeads], L[kReduceHeads];
  float red[2][REDUCE_THREADS / 64];  // per-wave maxima and sums of seg_weights_one
  float part[REDUCE_THREADS / 64][512];  // by-segments mapping: per-wave sums of a column part
};

// By heads: block (head group hg, request b).  T: element type of the
// workspace partials (float, or uint16_t holding bf16).
#ifndef DCP_REDUCE_HEADS_UNROLL
#define DCP_REDUCE_HEADS_UNROLL 8
#endif
template <int DV, typename T>
__device__ __forceinline__ void reduce_by_heads(const SplitArgs& s, int heads, int b, int hg, ReduceSmem& sm) {
  // segment loads in flight per lane: 8 measured ~2 us faster per call than 4
  // at C2 (whose long requests split into ~64 segments), 16 slower
  constexpr int HU = DCP_REDUCE_HEADS_UNROLL;
  constexpr int C = DV / 64;  // columns per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h0 = hg * kReduceHeads;
  const int nh = min(kReduceHeads, heads - h0);
  const SegRange r = seg_range(s, b);
  if (r.nseg == 1) return;  // finished by the workgroup that held it
  if (r.nseg == 0) {
    FVec<C> z;
#pragma unroll
    for (int k = 0; k < C; ++k) z.v[k] = 0.f;
    for (int j = wave; j < nh; j += REDUCE_THREADS / 64) {
      store_cols<C>(s.out + ((size_t)b * heads + h0 + j) * DV + lane * C, z);
      if (lane == 0) s.lse[(size_t)b * heads + h0 + j] = -__builtin_inff();
    }
    return;
  }
  const size_t stride = (size_t)heads * DV;
  // the first two segments of this wave's head (a split request has at least
  // two) are requested before the weights, so both round trips overlap; a wave
  // past the group's heads reads a valid row it does not use
  FVec<C> pre[2];
  {
    const int hp = min(h0 + wave, heads - 1);
    const T* src = (const T*)s.ws_o + ((size_t)(r.g0 + b) * heads + hp) * DV + lane * C;
    pre[0] = load_cols<C, T>(src);
    pre[1] = load_cols<C, T>(src + stride);
  }
  seg_weights(s, heads, b, r, h0, nh, sm.w, sm.M, sm.L);
  for (int j = wave; j < nh; j += REDUCE_THREADS / 64) {
    const int h = h0 + j;
    const T* src = (const T*)s.ws_o + ((size_t)(r.g0 + b) * heads + h) * DV + lane * C;
    const float* w = sm.w + j * kMaxSplitWGs;
    FVec<C> acc;
#pragma unroll
    for (int k = 0; k < C; ++k) acc.v[k] = w[0] * pre[0].v[k] + w[1] * pre[1].v[k];
    int i = 2;
    for (; i + HU <= r.nseg; i += HU) {
      FVec<C> x[HU];
#pragma unroll
      for (int u = 0; u < HU; ++u) x[u] = load_cols<C, T>(src + (size_t)(i + u) * stride);
#pragma unroll
      for (int u = 0; u < HU; ++u)
#pragma unroll
        for (int k = 0; k < C; ++k) acc.v[k] += w[i + u] * x[u].v[k];
    }
    for (; i < r.nseg; ++i) {
      const FVec<C> x = load_cols<C, T>(src + (size_t)i * stride);
#pragma unroll
      for (int k = 0; k < C; ++k) acc.v[k] += w[i] * x.v[k];
    }
    const float inv = 1.f / sm.L[j];
#pragma unroll
    for (int k = 0; k < C; ++k) acc.v[k] *= inv;
    store_cols<C>(s.out + ((size_t)b * heads + h) * DV + lane * C, acc);
    if (lane == 0) s.lse[(size_t)b * heads + h] = (sm.M[j] * s.c + __log2f(sm.L[j])) * kLn2;
  }
}

// By segments: block (column part cp of CP, head h, request b).
template <int DV, int CP, typename T>
__device__ __forceinline__ void reduce_by_segments(const SplitArgs& s, int heads, int b, int h, int cp,
                                                   ReduceSmem& sm) {
  constexpr int C = DV / CP / 64;  // columns per lane
  static_assert(C >= 1 && DV / CP <= 512, "column part");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = cp * (DV / CP) + lane * C;
  const SegRange r = seg_range(s, b);
  if (r.nseg == 1) return;
  if (r.nseg == 0) {
    if (wave == 0) {
      FVec<C> z;
#pragma unroll
      for (int k = 0; k < C; ++k) z.v[k] = 0.f;
      store_cols<C>(s.out + ((size_t)b * heads + h) * DV + col, z);
      if (lane == 0 && cp == 0) s.lse[(size_t)b * heads + h] = -__builtin_inff();
    }
    return;
  }
  const size_t stride = (size_t)heads * DV;
  const T* src = (const T*)s.ws_o + ((size_t)(r.g0 + b) * heads + h) * DV + col;
  constexpr int NW = REDUCE_THREADS / 64;
  // this wave's first U segments are requested before the weights (indices
  // clamped into the request: loads past its last segment are not used).
  // Deeper prefetch (U = 32, up to 256 segments in one round trip) measured
  // slower at 256 segments and at 64.
  constexpr int U = 8;
  FVec<C> pre[U];
#pragma unroll
  for (int u = 0; u < U; ++u) pre[u] = load_cols<C, T>(src + (size_t)min(wave + u * NW, r.nseg - 1) * stride);
  seg_weights_one(s, heads, b, r, h, sm.w, sm.M, sm.L, sm.red);
  FVec<C> acc;
#pragma unroll
  for (int k = 0; k < C; ++k) acc.v[k] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (wave + u * NW < r.nseg) {
#pragma unroll
      for (int k = 0; k < C; ++k) acc.v[k] += sm.w[wave + u * NW] * pre[u].v[k];
    }
  int i = wave + U * NW;
  for (; i + (U - 1) * NW < r.nseg; i += U * NW) {
    FVec<C> x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = load_cols<C, T>(src + (size_t)(i + u * NW) * stride);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < C; ++k) acc.v[k] += sm.w[i + u * NW] * x[u].v[k];
  }
  for (; i < r.nseg; i += NW) {
    const FVec<C> x = load_cols<C, T>(src + (size_t)i * stride);
#pragma unroll
    for (int k = 0; k < C; ++k) acc.v[k] += sm.w[i] * x.v[k];
  }
#pragma unroll
  for (int k = 0; k < C; ++k) sm.part[wave][lane * C + k] = acc.v[k];
  __syncthreads();
  if (wave == 0) {
    const float inv = 1.f / sm.L[0];
#pragma unroll
    for (int k = 0; k < C; ++k) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) t += sm.part[q][lane * C + k];
      acc.v[k] = t * inv;
    }
    store_cols<C>(s.out + ((size_t)b * heads + h) * DV + col, acc);
    if (lane == 0 && cp == 0) s.lse[(size_t)b * heads + h] = (sm.M[0] * s.c + __log2f(sm.L[0])) * kLn2;
  }
}

// Launch shape of the split reduce.  The by-segments mapping is used when the
// workgroups outnumber the requests 16 to 1 or more (then a split request has
// many segments); otherwise by heads.
struct ReducePlan {
  bool by_segments;
  dim3 grid;
};
inline ReducePlan reduce_plan(int batch, int heads, int G, int col_parts) {
  ReducePlan p;
  p.by_segments = G >= 16 * batch;
  if (p.by_segments) p.grid = dim3(col_parts, heads, batch);
  else p.grid = dim3((heads + kReduceHeads - 1) / kReduceHeads, batch);
  return p;
}

}  // namespace dcp
