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
// row's threads), forms the weights itself, then streams the N fp32 partial
// chunks with independent 16-byte loads and writes bf16 (and optionally the
// fp32 result and the merged LSE).  A 256-thread block covers 256/(dv/4) rows,
// so even small batches spread over many blocks.
#include "dcp_device.hpp"
#include "dcp_internal.hpp"

namespace dcp {

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int tpr = a.dv >> 2;                 // threads per row (<= 256)
  const int rpb = 256 / tpr;                 // rows per block
  const int row = blockIdx.x * rpb + (int)threadIdx.x / tpr;
  const int c = (int)threadIdx.x % tpr;
  if (row >= a.rows || (int)threadIdx.x >= rpb * tpr) return;
  const float* lse = a.plse + row;
  float M = -__builtin_inff();
  for (int i = 0; i < a.nshards; ++i) M = fmaxf(M, lse[(size_t)i * a.rows]);
  const size_t off = (size_t)row * a.dv + 4 * c;
  if (M == -__builtin_inff()) {
    if (a.out_bf16) *(uint2*)(a.out_bf16 + off) = make_uint2(0u, 0u);
    if (a.out_f32) *(f32x4*)(a.out_f32 + off) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c == 0 && a.lse_out) a.lse_out[row] = -__builtin_inff();
    return;
  }
  float S = 0.f;
  for (int i = 0; i < a.nshards; ++i) S += exp2_fast((lse[(size_t)i * a.rows] - M) * kLog2e);
  const float inv = 1.f / S;
  const size_t stride = (size_t)a.rows * a.dv;
  const float* base = a.po + off;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int i = 0;
  for (; i + 4 <= a.nshards; i += 4) {
    f32x4 x[4];
    float wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u] = *(const f32x4*)(base + (size_t)(i + u) * stride);
      wv[u] = exp2_fast((lse[(size_t)(i + u) * a.rows] - M) * kLog2e) * inv;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += wv[u] * x[u];
  }
  for (; i < a.nshards; ++i)
    acc += exp2_fast((lse[(size_t)i * a.rows] - M) * kLog2e) * inv * *(const f32x4*)(base + (size_t)i * stride);
  if (a.out_bf16)
    *(uint2*)(a.out_bf16 + off) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  if (a.out_f32) *(f32x4*)(a.out_f32 + off) = acc;
  if (c == 0 && a.lse_out) a.lse_out[row] = M + __log2f(S) * kLn2;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int rpb = 256 / (a.dv >> 2);
  hipLaunchKernelGGL(combine_kernel, dim3((a.rows + rpb - 1) / rpb), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dcp
