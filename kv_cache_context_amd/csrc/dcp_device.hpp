// Device-side helpers shared by the DCP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dcp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;  // one 16x16x32 MFMA operand
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;

#define DCP_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l holds A row l%16 / B column l%16, k-slots 8*(l/16)..+7; D column l%16,
// rows 4*(l/16)..+3.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16x16] * B[16x16]; lane l holds k-slots 4*(l/16)..+3.
__device__ __forceinline__ f32x4 mfma_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Transposing LDS read: inside each group of 16 lanes, lane i receives element
// (i % 4) of the 4 x 16-bit values loaded by lanes 4*j + i/4, j = 0..3.  With
// lane L of a group pointing at row (L/4), columns 4*(L%4)..+3 of a row-major
// 4 x 16 tile, lane i gets column i of the 4 rows.
__device__ __forceinline__ i16x4 lds_read_tr16(const DCP_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((DCP_LDS i16x4*)p);
}

// Mark a value as uniform across the wave (keeps it, and loads addressed by it, scalar).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read-only load through the scalar cache (index must be wave-uniform).  Used
// for block-table entries and lengths, which the kernels never write.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Copy 16 bytes global -> LDS without passing through registers
// (global_load_lds_dwordx4).  `lds_wave_base` must be the same for all lanes of
// the wave; lane i writes base + 16*i.  Issued from inline assembly on purpose:
// the compiler then does not add its own conservative "wait for every LDS copy"
// before later LDS reads.  The caller owns completion: wait_vmcnt<N>() (vector
// memory operations of a wave complete in issue order) followed by barrier().
__device__ __forceinline__ void dma16(const void* src, DCP_LDS void* lds_wave_base) {
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)lds_wave_base);
  // m0 is reserved: the compiler keeps no value in it across statements here
  // (it sets m0 itself right before each of its own uses).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(m0)
      : "memory", "m0");
#pragma clang diagnostic pop
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset (the saddr form): no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t voff, DCP_LDS void* lds_wave_base) {
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)lds_wave_base);
  // build the 64-bit base from wave-uniform halves so it lands in an SGPR pair
  const uint64_t b64 = (uint64_t)(uintptr_t)base;
  const uint64_t sbase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b64 >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b64);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(m0)
      : "memory", "m0");
#pragma clang diagnostic pop
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0) only

// Workgroup barrier that neither waits on memory counters nor lets the compiler
// move memory accesses across it.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Reductions over the lanes l, l^16, l^32, l^48 (the four 16-lane rows of the
// wave) with the gfx950 row-swap instructions: v_permlane16_swap exchanges odd
// rows of one operand with even rows of the other and v_permlane32_swap the
// upper half of one with the lower half of the other, so with both operands
// holding v, the two results hold v and its partner lane's v in some order and
// a commutative op of the two is the pairwise reduction.  Pure VALU: no LDS
// round trip.
__device__ __forceinline__ float row_swap16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_swap32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_swap16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float row_swap32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max16(float v) { return row_swap32_max(row_swap16_max(v)); }
__device__ __forceinline__ float wave_sum16(float v) { return row_swap32_sum(row_swap16_sum(v)); }
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Number of a request's L global tokens that live on shard r of n.
// Round-robin: positions r, r+n, ...; contiguous: [r*C, min(L,(r+1)*C)), C = ceil(L/n).
__host__ __device__ __forceinline__ int local_len(int L, int n, int r, int layout) {
  if (L <= 0) return 0;
  const int64_t LL = L;
  if (layout == 0) return LL > r ? (int)((LL - r + n - 1) / n) : 0;
  const int64_t c = (LL + n - 1) / n;
  const int64_t lo = c * r;
  const int64_t hi = LL < lo + c ? LL : lo + c;
  return hi > lo ? (int)(hi - lo) : 0;
}

// Eight E4M3 codes (two dwords, code k in byte k % 4 of dword k / 4) widened
// to bf16, in order.  The conversion is exact.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;  // round to nearest even (v_cvt_pk_bf16_f32)
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float a) {
  const __bf16 x = (__bf16)a;  // round to nearest even
  return __builtin_bit_cast(uint16_t, x);
}

}  // namespace dcp
