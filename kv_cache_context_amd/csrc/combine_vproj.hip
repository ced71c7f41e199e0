// DCP combine fused with the per-head value up-projection and a sigmoid gate.
//
// The Kimi K3 GB300 decode page describes the DCP step of its decode path as
// one tuned kernel that combines the shards' partial results together with the
// value projection and the gating.  For every (request b, head h):
//   o      = sum_i exp(lse_i - lse*) * o_i,  lse* = M + ln sum_i exp(lse_i - M)
//            (the LSE merge of the N latent partials, vLLM blog post on Decode
//            Context Parallelism, section 4.1)
//   y[n]   = sigmoid(gate[b][h][n]) * sum_k o[k] * w_uv_t[h][n][k]
// with the latent width Dv (512 for MLA) and the projected width Dvo.
//
// One workgroup of 4 waves takes 16 requests of one head:
//  1. the 16 rows' shard weights exp(lse_i - lse*) go to LDS (16 lanes per row);
//  2. the merged latent rows are formed with 16-byte partial loads and stored
//     to LDS as bf16, padded rows so the MFMA operand reads spread over banks;
//  3. out[16 x cols] = O . W_h^T with v_mfma_f32_16x16x32_bf16, O from LDS and
//     W_h (k contiguous) from global, wave w taking output column blocks w,
//     w + 4, ... of the workgroup's columns.  The first KW k-steps of the
//     wave's W operands are requested at kernel start, so their latency hides
//     behind steps 1-2; later ones stream through a KW-deep register window;
//  4. the gate and the casts are applied on the accumulator registers.
// The latent rows are rounded to bf16 only as MFMA operands (the fp32 merge
// itself is exact to fp32 rounding); accumulation is fp32.
#include "dcp_device.hpp"
#include "dcp_internal.hpp"

namespace dcp {
namespace vproj {

constexpr int ROWS = 16;      // requests per workgroup (one MFMA row block)
constexpr int THREADS = 256;  // 4 waves
constexpr int MAXN = 64;      // shards
constexpr int MAXDV = 1024;

// NQ: column blocks per wave (1, 2 or 4); grid (row blocks, heads, column
// groups): workgroup z takes column blocks [z * nbw, (z + 1) * nbw).
template <int NQ>
__global__ __launch_bounds__(THREADS) void kernel(VprojArgs a, int nbw) {
  constexpr int KW = NQ <= 1 ? 8 : 4;  // k-steps of W operands in flight per wave
  __shared__ float s_w[ROWS][MAXN];
  __shared__ __attribute__((aligned(16))) uint16_t s_o[ROWS * (MAXDV + 8)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * ROWS, h = blockIdx.y;
  const int H = a.heads, dv = a.dv, dvo = a.dvo, n = a.nshards;
  const int ostride = dv + 8;  // bf16 elements per LDS row
  const int g4 = lane >> 4, r16 = lane & 15;
  const int nb0 = blockIdx.z * nbw;
  const int ksteps = dv >> 5;
  const uint16_t* wh = a.w + (size_t)h * dvo * dv;

  // W operands of the first KW k-steps, requested before the merge work
  bf16x8 breg[KW][NQ];
  auto wload = [&](int ks, int q) -> bf16x8 {
    const int nb = nb0 + wave + 4 * q;
    return *(const bf16x8*)(wh + (size_t)(nb * 16 + r16) * dv + ks * 32 + 8 * g4);
  };
#pragma unroll
  for (int k = 0; k < KW; ++k)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (wave + 4 * q < nbw && k < ksteps) breg[k][q] = wload(k, q);

  // ---- 1. shard weights of the 16 rows: 16 lanes per row
  {
    const int i = tid >> 4, j = tid & 15;
    const int r = r0 + i;
    float lv[MAXN / 16];
    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < MAXN / 16; ++k) {
      const int s = j + 16 * k;
      lv[k] = (r < a.batch && s < n) ? a.plse[((size_t)s * a.batch + r) * H + h] : -__builtin_inff();
      mx = fmaxf(mx, lv[k]);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
    const bool empty = mx == -__builtin_inff();
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < MAXN / 16; ++k) {
      lv[k] = empty ? 0.f : exp2_fast((lv[k] - mx) * kLog2e);  // 0 for -inf entries
      sum += lv[k];
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
    const float inv = empty ? 0.f : 1.f / sum;
#pragma unroll
    for (int k = 0; k < MAXN / 16; ++k)
      if (j + 16 * k < n) s_w[i][j + 16 * k] = lv[k] * inv;
    if (j == 0 && r < a.batch && a.lse_out)
      a.lse_out[(size_t)r * H + h] = empty ? -__builtin_inff() : mx + __log2f(sum) * kLn2;
  }
  __syncthreads();

  // ---- 2. merged latent rows -> LDS (bf16); rows past the batch are zero
  {
    const int cpr = dv >> 2;  // 4-column chunks per row
    const size_t sstride = (size_t)a.batch * H * dv;
    for (int c = tid; c < ROWS * cpr; c += THREADS) {
      const int ri = c / cpr;
      const int r = r0 + ri;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (r < a.batch) {
        const float* src = a.po + ((size_t)r * H + h) * dv + 4 * (c % cpr);
        for (int s0 = 0; s0 < n; s0 += 8) {
          f32x4 x[8];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            x[k] = (s0 + k < n) ? *(const f32x4*)(src + (size_t)(s0 + k) * sstride) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (s0 + k < n) acc += s_w[ri][s0 + k] * x[k];
        }
      }
      uint16_t* dst = s_o + ri * ostride + 4 * (c % cpr);
      *(uint2*)dst = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
  }
  __syncthreads();

  // ---- 3. out[16 x cols] = O . W_h^T on the matrix cores
  f32x4 acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < ksteps; k0 += KW) {
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      const int ks = k0 + k;
      if (ks < ksteps) {
        const bf16x8 av = *(const bf16x8*)(s_o + r16 * ostride + ks * 32 + 8 * g4);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          if (wave + 4 * q < nbw) {
            acc[q] = mfma_16x16x32(av, breg[k][q], acc[q]);
            if (ks + KW < ksteps) breg[k][q] = wload(ks + KW, q);
          }
      }
    }
  }

  // ---- 4. gate and stores: lane holds column nb*16 + r16 of rows 4*g4 + i
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (wave + 4 * q >= nbw) continue;
    const int col = (nb0 + wave + 4 * q) * 16 + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 4 * g4 + i;
      if (r >= a.batch) continue;
      const size_t idx = ((size_t)r * H + h) * dvo + col;
      float y = acc[q][i];
      if (a.gate) {
        const float gl = __uint_as_float((uint32_t)a.gate[idx] << 16);
        y *= 1.f / (1.f + exp2_fast(-gl * kLog2e));
      }
      if (a.out_f32) a.out_f32[idx] = y;
      if (a.out_bf16) a.out_bf16[idx] = bf16_bits_rne(y);
    }
  }
}

}  // namespace vproj

hipError_t launch_combine_vproj(const VprojArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int rb = (a.batch + vproj::ROWS - 1) / vproj::ROWS;
  const int nblk = a.dvo / 16;
  // a small batch leaves too few workgroups for the projection weights'
  // bandwidth: split the output columns over two workgroups (each repeats the
  // merge of its rows, which is cheap when rows are few)
  const int cs = ((int64_t)rb * a.heads < 256 && nblk % 2 == 0 && nblk >= 2) ? 2 : 1;
  const int nbw = nblk / cs;
  const dim3 grid(rb, a.heads, cs);
  if (nbw <= 4) hipLaunchKernelGGL(vproj::kernel<1>, grid, dim3(vproj::THREADS), 0, stream, a, nbw);
  else if (nbw <= 8) hipLaunchKernelGGL(vproj::kernel<2>, grid, dim3(vproj::THREADS), 0, stream, a, nbw);
  else hipLaunchKernelGGL(vproj::kernel<4>, grid, dim3(vproj::THREADS), 0, stream, a, nbw);
  return hipGetLastError();
}

}  // namespace dcp
