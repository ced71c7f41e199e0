// LSE-weighted merge of N shard partials, fused with the bf16 output cast.
//
// Definition (vLLM blog post on Decode Context Parallelism, section 4.1: the
// ranks' LSE values reweight their partial outputs, whose sum is the exact
// attention output): for each (request, head) row, with M = max_i lse_i,
//   lse = M + ln(sum_i exp(lse_i - M)),   o = sum_i exp(lse_i - lse) * o_i.
// A row whose partials are all empty (lse = -inf) is (0, -inf).
//
// Bandwidth-bound.  Each thread owns 4 consecutive output columns of one
// (request, head) row: it reads the row's N LSEs (cache-resident, shared by the
// row's threads) and its N fp32 partial chunks with independent 16-byte loads,
// forms the weights itself and writes bf16 (and optionally the fp32 result and
// the merged LSE).  A 256-thread block covers 256/(dv/4) rows,
// so even small batches spread over many blocks.
#include "dcp_device.hpp"
#include "dcp_internal.hpp"

namespace dcp {

// Shard counts 2, 4 and 8 have their own instances (NS > 0): every partial
// chunk and LSE of the thread's row is requested at once, before the weights
// are formed, so the loads' latencies overlap.  NS = 0 serves any count.
template <int NS>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int tpr = a.dv >> 2;                 // threads per row (<= 256)
  const int rpb = 256 / tpr;                 // rows per block
  const int row = blockIdx.x * rpb + (int)threadIdx.x / tpr;
  const int c = (int)threadIdx.x % tpr;
  if (row >= a.rows || (int)threadIdx.x >= rpb * tpr) return;
  const int ns = NS > 0 ? NS : a.nshards;
  const float* lse = a.plse + row;
  const size_t off = (size_t)row * a.dv + 4 * c;
  const size_t stride = (size_t)a.rows * a.dv;
  const float* base = a.po + off;
  f32x4 x[NS > 0 ? NS : 1];
  float lv[NS > 0 ? NS : 1];
  float M = -__builtin_inff();
  if constexpr (NS > 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      x[i] = *(const f32x4*)(base + (size_t)i * stride);
      lv[i] = lse[(size_t)i * a.rows];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) M = fmaxf(M, lv[i]);
  } else {
    for (int i = 0; i < ns; ++i) M = fmaxf(M, lse[(size_t)i * a.rows]);
  }
  if (M == -__builtin_inff()) {
    if (a.out_bf16) *(uint2*)(a.out_bf16 + off) = make_uint2(0u, 0u);
    if (a.out_f32) *(f32x4*)(a.out_f32 + off) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c == 0 && a.lse_out) a.lse_out[row] = -__builtin_inff();
    return;
  }
  float S = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (NS > 0) {
    float w[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      w[i] = exp2_fast((lv[i] - M) * kLog2e);
      S += w[i];
    }
    const float inv = 1.f / S;
#pragma unroll
    for (int i = 0; i < NS; ++i) acc += (w[i] * inv) * x[i];
  } else {
    for (int i = 0; i < ns; ++i) S += exp2_fast((lse[(size_t)i * a.rows] - M) * kLog2e);
    const float inv = 1.f / S;
    int i = 0;
    for (; i + 4 <= ns; i += 4) {
      f32x4 y[4];
      float wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        y[u] = *(const f32x4*)(base + (size_t)(i + u) * stride);
        wv[u] = exp2_fast((lse[(size_t)(i + u) * a.rows] - M) * kLog2e) * inv;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += wv[u] * y[u];
    }
    for (; i < ns; ++i)
      acc += exp2_fast((lse[(size_t)i * a.rows] - M) * kLog2e) * inv * *(const f32x4*)(base + (size_t)i * stride);
  }
  if (a.out_bf16)
    *(uint2*)(a.out_bf16 + off) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  if (a.out_f32) *(f32x4*)(a.out_f32 + off) = acc;
  if (c == 0 && a.lse_out) a.lse_out[row] = M + __log2f(S) * kLn2;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int rpb = 256 / (a.dv >> 2);
  const dim3 grid((a.rows + rpb - 1) / rpb);
  switch (a.nshards) {
    case 2: hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(combine_kernel<0>, grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace dcp
