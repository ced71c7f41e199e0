// LSE-weighted merge of N shard partials, fused with the bf16 output cast.
//
// Definition (vLLM blog post on Decode Context Parallelism, section 4.1: the
// ranks' LSE values reweight their partial outputs, whose sum is the exact
// attention output): for each (request, head) row, with M = max_i lse_i,
//   lse = M + ln(sum_i exp(lse_i - M)),   o = sum_i exp(lse_i - lse) * o_i.
// A row whose partials are all empty (lse = -inf) is (0, -inf).
//
// Bandwidth-bound: one wave per row reads the N LSEs (one per lane), reduces
// them across the wave, then streams the N fp32 rows with 16-byte loads and
// writes bf16 (and optionally the fp32 result and the merged LSE).
#include "dcp_device.hpp"
#include "dcp_internal.hpp"

namespace dcp {

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const float li = lane < a.nshards ? a.plse[(size_t)lane * a.rows + row] : -__builtin_inff();
  const float M = wave_max(li);
  const int nv = a.dv >> 2;
  if (M == -__builtin_inff()) {
    for (int c = lane; c < nv; c += 64) {
      if (a.out_bf16) *(uint2*)(a.out_bf16 + (size_t)row * a.dv + 4 * c) = make_uint2(0u, 0u);
      if (a.out_f32) *(f32x4*)(a.out_f32 + (size_t)row * a.dv + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (lane == 0 && a.lse_out) a.lse_out[row] = -__builtin_inff();
    return;
  }
  const float w = lane < a.nshards ? exp2_fast((li - M) * kLog2e) : 0.f;
  const float S = wave_sum(w);
  const float wn = w / S;
  if (lane == 0 && a.lse_out) a.lse_out[row] = M + __log2f(S) * kLn2;
  const size_t stride = (size_t)a.rows * a.dv;
  const float* base = a.po + (size_t)row * a.dv;
  // The column loop stays converged (uniform trip count) so every lane's weight
  // is live when it is broadcast; lanes past the row end only skip memory.
  for (int c0 = 0; c0 < nv; c0 += 64) {
    const int c = c0 + lane;
    const bool on = c < nv;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < a.nshards; ++i) {
      const float wi = __shfl(wn, i);
      if (on) acc += wi * *(const f32x4*)(base + i * stride + 4 * c);
    }
    if (!on) continue;
    if (a.out_bf16)
      *(uint2*)(a.out_bf16 + (size_t)row * a.dv + 4 * c) =
          make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    if (a.out_f32) *(f32x4*)(a.out_f32 + (size_t)row * a.dv + 4 * c) = acc;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((a.rows + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dcp
