// Shard-local MLA decode attention (absorbed form) for gfx950, latent dimension
// split across the waves of a workgroup.
//
// What one shard computes (vLLM blog post on Decode Context Parallelism,
// sections 4.1 and 5.3): every query head attends its request's local latent
// rows [c_kv | k_rope] (576 values); the value is c_kv (512).  The output is
// the normalized partial attention and its natural-log LSE, merged across
// shards by dcp_combine.
//
// Work of one split workgroup: 4 waves, one per SIMD (up to 512 registers
// each), 32-token tiles of its range of the shard's tile list.
//  * Latent split: wave w owns latent columns 128w .. 128w + 127 of c_kv and one
//    32-wide step of k_rope (step w & 1 of token half w >> 1).  It loads exactly
//    those bytes of every tile row from HBM straight into registers, already in
//    the MFMA operand layout (16 rows x 64 contiguous bytes per load
//    instruction), so each latent byte crosses HBM once and is read by one wave.
//  * Scores: the wave's partial S^T[32 tok x 64 heads] over its columns, with
//    v_mfma_f32_16x16x32_bf16 (K rows as the A operand, its part of q for all
//    heads held in registers for the segment).  The four partials are summed
//    through LDS; wave h then owns the softmax of head block h (16 heads).
//  * Softmax in base 2 against a fixed per-head reference (the maximum of the
//    segment's first tile), so the accumulators are never rescaled; a tile that
//    passes it by more than the headroom makes the segment run again with the
//    true maxima preset (exact either way).
//  * Values: the wave's own c_kv columns are the value columns it accumulates,
//    O^T[128 cols x 64 heads] += V^T[cols x 32 tok] . P^T[32 tok x 64 heads].
//    V^T needs tokens along the operand's k dimension, so the wave writes its
//    columns of the tile to a private LDS region and reads them back with the
//    transposing ds_read_b64_tr_b16; P^T of all head blocks comes from LDS.
//  * Per tile and CU, LDS carries 32 KiB of V (written once, read once), 32 KiB
//    of partial scores and 4 KiB of probabilities, against the 36 KiB tile.
//  * Software pipeline: the value contraction of tile i - 1 is issued after
//    tile i's scores and partial-score writes, so its matrix work runs while the
//    waves meet at the exchange; the transposing reads and the probability
//    reads of tile i are issued after the exchange and consumed one tile later,
//    off the exchange's path.
//  * Split-K partials go to the workspace (bf16 outputs with fp32 reference and
//    sum) and the split reduce merges them.
//
// fp8 latent cache (OCP E4M3 codes, one dequantization scale s): the same
// split over 576-byte rows; each lane's codes are widened exactly to bf16 in
// registers (v_cvt_scalef32_pk_bf16_fp8) and feed both the score operands and
// the wave's V region, so the tile computation is the bf16 one.  s multiplies
// the softmax scale and the output once.
#include "dcp_device.hpp"
#include "dcp_internal.hpp"
#include "dcp_split.hpp"

namespace dcp {
namespace mlak {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int R = 512, P = 64, DK = R + P;
constexpr int TILE = 32;          // tokens per tile
constexpr int NWAVE = 4;
constexpr int THREADS = 64 * NWAVE;
constexpr int NCB = 8;            // 16-column value blocks per wave (128 columns)
// One row of a wave's V region: 128 bf16 columns (256 bytes) plus 16 bytes of
// padding.  With 272-byte rows the 16-byte unit (row, chunk) sits in bank group
// (17 row + chunk) mod 32 (LDS: 128 banks of 4 bytes), so the 16 rows of one
// transposing read (two chunks each) and the 16 rows of one 16-lane group of
// a row-wise write all fall in distinct bank groups, and every address of a
// lane is its base plus an immediate offset.
constexpr int VROW = 272;
#ifndef DCP_MLAK_NB
#define DCP_MLAK_NB 3
#endif
constexpr int NB = DCP_MLAK_NB;   // tile register buffers: NB - 1 tiles are requested ahead
static_assert(NB >= 2 && NB <= 4, "register buffers");
constexpr float kHeadroomLog2 = 64.f;  // p may reach 2^64 above the fixed reference

// Tile modes: FULL computes scores, softmax and values; MAXIMUM only each
// head's running maximum of the scores (the first pass of a rerun).
enum { FULL = 0, MAXIMUM = 1 };

// Cache row format: bf16 (FP8 = false) or E4M3 codes (FP8 = true).
template <bool FP8>
struct Fmt {
  static constexpr int ROW = DK * (FP8 ? 1 : 2);  // bytes per latent row
};

// One tile's loads of one lane (row 16 tb + (lane & 15) of token half tb).
// bf16: c[4 tb + ks] = latent columns 128 w + 32 ks + 8 (lane >> 4) + 0..7;
//       rope = k_rope k = 32 (w & 1) + 8 (lane >> 4) + 0..7 of row
//       16 (w >> 1) + (lane & 15).
// fp8:  c[2 tb + j] = 16 codes of columns 128 w + 64 j + 16 (lane >> 4) + 0..15;
//       rope = 8 codes, k and row as for bf16.
template <bool FP8>
struct KTile;
template <>
struct KTile<false> {
  u32x4 c[8];
  u32x4 rope;
  int ent0, ent1;  // table entries of the tile this buffer is loaded with next
};
template <>
struct KTile<true> {
  u32x4 c[4];
  u32x2 rope;
  int ent0, ent1;
};

template <int NHB>
struct Smem {
  f32x4 sx[NWAVE][2][NHB][64];  // partial scores: writer wave, token half, head block, lane
  uint4 px[NHB][64];            // P^T operand (8 bf16) per head block and lane
  int flag[4];                  // per owner wave: a tile passed the reference's headroom
  float em[NHB][16], el[NHB][16];  // segment end: reference and softmax sum per head
  char v[NWAVE][TILE * VROW];   // each wave's value columns of the current tile
  int pref[kMaxBatch + 1];
  int wsum[NWAVE];
};
static_assert(sizeof(Smem<4>) <= 160 * 1024, "LDS budget");

// Global-memory pointer (address space 1): loads through it are global loads,
// counted by vmcnt only (a generic pointer would give flat loads, which the
// LDS counter also tracks).
typedef const __attribute__((address_space(1))) char* gptr;

// A global pointer whose value is the same in every lane, built from
// readfirstlane halves so it lives in SGPRs (loads then use the scalar-base
// form with a 32-bit lane offset).
__device__ __forceinline__ gptr uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  return (gptr)u;
}

// Walks a segment's tiles in order and issues each tile's loads.
// Block-table entries are fetched with vector loads (vmcnt, in order with the
// tile loads) rather than scalar loads: a pending scalar load would make every
// wait for an LDS result a wait for all LDS operations.  Each register buffer
// carries the two table entries of the tile it will hold next; issuing tile t
// into buffer k uses k's entries and fetches those of tile t + NB, which are
// waited for only when that tile is issued (after tile t, loaded before them,
// has been consumed).  Past the segment's last tile the tile loads repeat the
// last tile's addresses (cache hits, results unused), so every step issues the
// same loads and the wait counts stay static.
template <bool FP8>
struct Loader {
  const char* kv;
  const int32_t* trow;
  int B, lastb, num_blocks;
  int left;      // tiles still to issue
  int lb, in;    // next tile to issue: local block and row of its token 0
  int flb, fin;  // next tile whose entries are fetched (NB tiles ahead of lb, in)
  gptr base0;    // row 0 of token half 0 / 1 of the last issued tile
  gptr base1;
  uint32_t offc;  // this lane's offset of its first c_kv load in a half
  uint32_t offr;  // and of its k_rope load
  int tbr;        // token half of the wave's k_rope load

  // local blocks of the two token halves of the tile starting at (blk, row)
  __device__ __forceinline__ int second_half(int blk, int row, int* row1) const {
    const int i1 = row + 16;  // B is a multiple of 16: a 16-row half never spans two blocks
    if (i1 < B) {
      *row1 = i1;
      return blk;
    }
    *row1 = i1 - B;
    return blk + 1;
  }
  __device__ __forceinline__ void advance(int& blk, int& row) const {
    row += TILE;
    while (row >= B) {
      row -= B;
      ++blk;
    }
  }
  // the table entries of the tile at the fetch cursor into k, and advance it
  __device__ __forceinline__ void fetch(KTile<FP8>& k) {
    typedef const __attribute__((address_space(1))) int32_t* gint;
    int r1;
    const int lb1 = second_half(flb, fin, &r1);
    k.ent0 = *(gint)(trow + min(flb, lastb));
    k.ent1 = *(gint)(trow + min(lb1, lastb));
    advance(flb, fin);
  }

  __device__ __forceinline__ void issue(KTile<FP8>& k) {
    constexpr int ROW = Fmt<FP8>::ROW;
    if (left > 0) {
      int in1;
      second_half(lb, in, &in1);
      const int c0 = uni(min(max(k.ent0, 0), num_blocks - 1));
      const int c1 = uni(min(max(k.ent1, 0), num_blocks - 1));
      base0 = uniform_ptr(kv + ((int64_t)c0 * B + in) * ROW);
      base1 = uniform_ptr(kv + ((int64_t)c1 * B + in1) * ROW);
      advance(lb, in);
      --left;
    }
    typedef const __attribute__((address_space(1))) u32x4* g16;
    gptr br = tbr ? base1 : base0;
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        k.c[j] = *(g16)(base0 + offc + 64 * j);
        k.c[2 + j] = *(g16)(base1 + offc + 64 * j);
      }
      k.rope = *(const __attribute__((address_space(1))) u32x2*)(br + offr);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        k.c[ks] = *(g16)(base0 + offc + 64 * ks);
        k.c[4 + ks] = *(g16)(base1 + offc + 64 * ks);
      }
      k.rope = *(g16)(br + offr);
    }
    fetch(k);  // entries of the tile this buffer holds next (NB tiles on)
  }
};

// Runs tiles [t0, t1) of row set b.
// FULL: writes the final result (whole request in this workgroup) or the split
//   partial of workspace slot slot_g + b.  The softmax reference of each head is
//   the maximum of the segment's first tile (or `mref`, when preset) and never
//   moves, so the accumulators are never rescaled; if a later tile exceeds it by
//   more than the headroom (p would pass 2^64), nothing is written and the call
//   returns true: the caller then finds each head's true maximum (MAXIMUM) and
//   runs again with it preset, where p <= 1 everywhere.
// MAXIMUM: stores each head's maximum score in `mref` (owner lanes).
// All waves call it with the same arguments (it holds workgroup barriers).
template <bool FP8, int NHB, int MODE>
__device__ __attribute__((always_inline)) inline bool run_segment(const MlaArgs& a, Smem<NHB>& sm, int b, int t0,
                                                                  int t1, int ntiles_b, int slot_g, bool preset,
                                                                  float& mref) {
  constexpr int ROW = Fmt<FP8>::ROW;
  const SplitArgs& s = a.s;
  const int lane = threadIdx.x & 63;
  const int w = uni(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int heads = 16 * NHB;
  const int n = t1 - t0;
  const int lr = uni(clamped_local_len(s, b));
  const float c = s.c;
  const float thr = kHeadroomLog2 / c;  // raw-score headroom above the reference

  // ---- q: this wave's columns of every head, in the score operand layout
  bf16x8 qf[NHB][4], qr[NHB];
  {
    const uint16_t* qrow = a.q + (int64_t)b * heads * DK;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const uint16_t* qh = qrow + (16 * hb + r) * DK;
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          qf[hb][2 * j] = *(const bf16x8*)(qh + 128 * w + 64 * j + 16 * g);
          qf[hb][2 * j + 1] = *(const bf16x8*)(qh + 128 * w + 64 * j + 16 * g + 8);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[hb][ks] = *(const bf16x8*)(qh + 128 * w + 32 * ks + 8 * g);
      }
      qr[hb] = *(const bf16x8*)(qh + R + 32 * (w & 1) + 8 * g);
    }
  }

  // ---- tile loads
  Loader<FP8> ld;
  ld.kv = (const char*)a.kv;
  ld.trow = table_row(s, b);
  ld.B = s.block_size;
  ld.lastb = uni(min(s.max_blocks - 1, (lr - 1) / s.block_size));
  ld.num_blocks = s.num_blocks;
  ld.left = n;
  ld.lb = uni((t0 * TILE) / s.block_size);
  ld.in = uni(t0 * TILE - ld.lb * s.block_size);
  ld.flb = ld.lb;
  ld.fin = ld.in;
  ld.tbr = w >> 1;
  if constexpr (FP8) {
    ld.offc = r * ROW + 128 * w + 16 * g;
    ld.offr = r * ROW + R + 32 * (w & 1) + 8 * g;
  } else {
    ld.offc = r * ROW + 2 * (128 * w + 8 * g);
    ld.offr = r * ROW + 2 * (R + 32 * (w & 1) + 8 * g);
  }
  KTile<FP8> kb[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) ld.fetch(kb[u]);  // entries of tiles 0 .. NB - 1
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) ld.issue(kb[u]);

  f32x4 acc[NCB][NHB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) acc[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // owner wave: reference and softmax sum of its lane's head
  float m = (MODE == FULL && preset) ? mref : -__builtin_inff(), l = 0.f;
  bool ovf = false;

  DCP_LDS char* vw = (DCP_LDS char*)sm.v[w];
  // this lane's row-wise write address (row r of token half 0, chunk g; bf16
  // chunk 4 ks + g, fp8 chunks 8 j + 2 g (+ 1) are immediate offsets from it)
  DCP_LDS char* vwr = vw + r * VROW + (FP8 ? 32 : 16) * g;
  // this lane's V^T read address (column block 0, token rows 4g + 0..3; +16
  // rows for the second half): lane r of a 16-lane group reads 4 columns of row
  // 4g + r/4 so that the transposing read hands it column r of the 4 rows
  const DCP_LDS char* vrd = vw + (4 * g + (r >> 2)) * VROW + 16 * ((r & 3) >> 1) + 8 * (r & 1);

  // operands of the previous tile's value contraction (zero before the first
  // tile: the first step adds nothing)
  i16x4 vlo[NCB], vhi[NCB];
  bf16x8 pt[NHB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) vlo[cb] = vhi[cb] = i16x4{0, 0, 0, 0};
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) pt[hb] = bf16x8{};

  auto values = [&]() {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const bf16x8 v8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[cb], vhi[cb], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) acc[cb][hb] = mfma_16x16x32(v8, pt[hb], acc[cb][hb]);
    }
  };

  auto tile = [&](int i, KTile<FP8>& kc) {
    const int k = t0 + i;
    const int valid = lr - k * TILE;  // rows of this tile inside the request
    const bool tail = valid < TILE;

    // ---- K operands (bf16)
    bf16x8 kop[2][4], kro;
    if constexpr (FP8) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 x = kc.c[2 * tb + j];
          kop[tb][2 * j] = e4m3x8_to_bf16(x[0], x[1]);
          kop[tb][2 * j + 1] = e4m3x8_to_bf16(x[2], x[3]);
        }
      kro = e4m3x8_to_bf16(kc.rope[0], kc.rope[1]);
    } else {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kop[tb][ks] = __builtin_bit_cast(bf16x8, kc.c[4 * tb + ks]);
      kro = __builtin_bit_cast(bf16x8, kc.rope);
    }

    // ---- the wave's V columns to its LDS region (after the previous tile's
    // transposing reads of it: LDS executes a wave's operations in order).
    // bf16: columns 32 ks + 8 g (chunk 4 ks + g); fp8: 16 columns 64 j + 16 g
    // as chunks 8 j + 2 g and 8 j + 2 g + 1, j = ks / 2
    if constexpr (MODE == FULL) {
      auto vstore = [&](int tb, int ks, bf16x8 x) {
        const int off = tb * 16 * VROW + (FP8 ? 128 * (ks >> 1) + 16 * (ks & 1) : 64 * ks);
        *(DCP_LDS bf16x8*)(vwr + off) = x;
      };
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vstore(tb, ks, kop[tb][ks]);
      if (tail) {
        // rows past the request hold value 0 (their probabilities are 0 too,
        // but stale rows could hold any bits); the empty asm keeps this a
        // branch taken on the last tile only, not selects on every tile
        asm volatile("" ::: "memory");
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          if (16 * tb + r >= valid) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) vstore(tb, ks, bf16x8{});
          }
      }
    }

    // ---- partial scores over the wave's columns; its k_rope step goes to
    // token half w >> 1 (the other half gets a zero operand)
    const bf16x8 kr0 = ld.tbr ? bf16x8{} : kro;
    const bf16x8 kr1 = ld.tbr ? kro : bf16x8{};
    f32x4 sacc[2][NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      sacc[0][hb] = mfma_16x16x32(kr0, qr[hb], f32x4{0.f, 0.f, 0.f, 0.f});
      sacc[1][hb] = mfma_16x16x32(kr1, qr[hb], f32x4{0.f, 0.f, 0.f, 0.f});
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) sacc[tb][hb] = mfma_16x16x32(kop[tb][ks], qf[hb][ks], sacc[tb][hb]);
    // every head block's partial to LDS (the owner reads all four back)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) sm.sx[w][tb][hb][lane] = sacc[tb][hb];
    __builtin_amdgcn_sched_barrier(0);
    // the previous tile's value contraction: its matrix work runs while the
    // waves meet at the exchange
    if constexpr (MODE == FULL) values();
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();
    barrier();

    // ---- softmax of the owned head block (wave w < NHB): lane holds head
    // 16 w + r, tokens 16 tb + 4 g + 0..3
    if (w < NHB) {
      f32x4 part[2][NWAVE];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int w2 = 0; w2 < NWAVE; ++w2) part[tb][w2] = sm.sx[w2][tb][w][lane];
      float sv[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const f32x4 st = (part[tb][0] + part[tb][1]) + (part[tb][2] + part[tb][3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * tb + e] = st[e];
      }
      if (tail) {
        asm volatile("" ::: "memory");  // a branch on the last tile, not selects on every tile
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * tb + 4 * g + e >= valid) sv[4 * tb + e] = -__builtin_inff();
      }
      float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mx = wave_max16(mx);
      if constexpr (MODE == MAXIMUM) {
        m = fmaxf(m, mx);
      } else {
        if (preset) {
        } else if (i == 0) {
          m = mx;  // the segment's first tile holds a valid token: finite
        } else {
          ovf = ovf || (mx > m + thr);
        }
        const float mc = m * c;
        float ps = 0.f;
        bf16x8 p8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2_fast(fmaf(sv[e], c, -mc));
          ps += p;
          p8[e] = (__bf16)p;
        }
        l += ps;
        sm.px[w][lane] = __builtin_bit_cast(uint4, p8);
      }
    }
    wait_lgkm0();
    barrier();

    // ---- operands of this tile's value contraction, consumed by the next
    // step (each wave's reads complete before it next passes a barrier: the
    // wait before the exchange barrier covers them)
    if constexpr (MODE == FULL) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) pt[hb] = __builtin_bit_cast(bf16x8, sm.px[hb][lane]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        vlo[cb] = lds_read_tr16(vrd + 32 * cb);
        vhi[cb] = lds_read_tr16(vrd + 32 * cb + 16 * VROW);
      }
    }
  };

  // Every unrolled step issues its loads (tile i + NB - 1, or the last tile's
  // again past the end) whether or not it computes, so the order of the loads
  // is the same on every path and the compiler's wait for tile i's registers
  // leaves the NB - 1 later tiles in flight.
  for (int i0 = 0; i0 < n; i0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      ld.issue(kb[(u + NB - 1) % NB]);
      __builtin_amdgcn_sched_barrier(0);
      if (i0 + u < n) tile(i0 + u, kb[u]);
    }
  }

  if constexpr (MODE == MAXIMUM) {
    mref = m;
    barrier();  // every wave is done with the exchange buffers
    return false;
  }
  values();  // the last tile's value contraction

  if (!preset) {
    // did any owner's head pass the headroom?  (each flag write completes
    // before the barrier that publishes it)
    if (w < NHB) {
      const bool any_ovf = __any(ovf);  // the vote runs on the whole wave
      if (lane == 0) sm.flag[w] = any_ovf ? 1 : 0;
    }
    wait_lgkm0();
    barrier();
    bool redo = false;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) redo = redo || uni(sm.flag[hb]) != 0;
    barrier();  // the flags are read before any wave can write them again
    if (redo) return true;
  }

  // ---- segment end: the owners publish each head's reference and sum
  if (w < NHB) {
    const float lt = wave_sum16(l);
    if (g == 0) {
      sm.em[w][r] = m;
      sm.el[w][r] = lt;
    }
  }
  wait_lgkm0();
  barrier();
  const int col = 128 * w + 4 * g;
  if (t0 == 0 && t1 == ntiles_b) {
    // the whole row set is in this workgroup: write the final result
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int head = 16 * hb + r;
      const float lh = sm.el[hb][r];
      const float inv = (FP8 ? a.vscale : 1.f) / lh;
      float* dst = s.out + ((size_t)b * heads + head) * R + col;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) *(f32x4*)(dst + 16 * cb) = acc[cb][hb] * inv;
      if (w == 0 && g == 0) s.lse[(size_t)b * heads + head] = (sm.em[hb][r] * c + __log2f(lh)) * kLn2;
    }
  } else {
    // split partial, un-normalized, bf16 (rounded to nearest even); the merge
    // divides by the segments' weighted sums, so each element's rounding moves
    // the merged row by at most 2^-9 max|v|
    const int slot = slot_g + b;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int head = 16 * hb + r;
      uint16_t* dst = (uint16_t*)s.ws_o + ((size_t)slot * heads + head) * R + col;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f32x4 v = FP8 ? acc[cb][hb] * a.vscale : acc[cb][hb];
        *(uint2*)(dst + 16 * cb) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
      if (w == 0 && g == 0) {
        float* ml = s.ws_ml + ((size_t)slot * heads + head) * 2;
        ml[0] = sm.em[hb][r];
        ml[1] = sm.el[hb][r];
      }
    }
  }
  barrier();  // the end-of-segment exchange is free again
  return false;
}

template <bool FP8, int NHB>
__global__ __launch_bounds__(THREADS, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void partial_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(1024))) Smem<NHB> sm;
  const SplitArgs& s = a.s;
  const int tid = threadIdx.x;
  const int bid = blockIdx.x;

  const int T = plan_tiles<THREADS>(s, TILE, sm.pref, sm.wsum);
  const int geff = split_wgs(s, T);
  if (bid == 0) {
    for (int i = tid; i <= s.batch; i += THREADS) s.ws_meta[1 + i] = sm.pref[i];
    if (tid == 0) s.ws_meta[0] = geff;
  }
  if (bid >= geff) return;
  // Workgroups go to the 8 XCDs round-robin (block i to XCD i mod 8).  For
  // multi-token steps the split ranges are numbered so that each XCD holds a
  // contiguous run of them: the row sets of one request's tokens sit next to
  // each other in the tile list and read the same cache rows at about the
  // same time, so neighbouring ranges on one XCD share its L2.
  const int g = uni((s.q_len > 1 && geff % 8 == 0) ? (bid % 8) * (geff / 8) + bid / 8 : bid);
  const int p0 = uni((int)((int64_t)g * T / geff));
  const int p1 = uni((int)((int64_t)(g + 1) * T / geff));

  int b = find_request(sm.pref, s.batch, p0);
  for (;;) {
    const int pb = uni(sm.pref[b]), pe = uni(sm.pref[b + 1]);
    const SegTiles st = seg_tiles(s, pb, pe, p0, p1);
    if (pe > pb && st.t1 > st.t0) {
      // fixed-reference pass; on overflow, find the true maxima and run again
      // with them preset (that run cannot overflow)
      float mref = 0.f;
      bool preset = false;
      for (int pass = 0; pass < 2; ++pass) {
        if (!run_segment<FP8, NHB, FULL>(a, sm, b, st.t0, st.t1, st.ntiles, g, preset, mref)) break;
        run_segment<FP8, NHB, MAXIMUM>(a, sm, b, st.t0, st.t1, st.ntiles, g, false, mref);
        preset = true;
      }
    }
    if (pe >= p1 || b + 1 >= s.batch) break;
    ++b;
  }
}

#ifndef DCP_MLAK_RED_COL_PARTS
#define DCP_MLAK_RED_COL_PARTS 2
#endif
constexpr int RED_COL_PARTS = DCP_MLAK_RED_COL_PARTS;  // column parts of the by-segments reduce

__global__ __launch_bounds__(REDUCE_THREADS) void reduce_kernel(MlaArgs a, int by_segments) {
  __shared__ ReduceSmem sm;
  if (by_segments) reduce_by_segments<R, RED_COL_PARTS, uint16_t>(a.s, a.heads, blockIdx.z, blockIdx.y, blockIdx.x, sm);
  else reduce_by_heads<R, uint16_t>(a.s, a.heads, blockIdx.y, blockIdx.x, sm);
}

template <bool FP8>
hipError_t launch(const MlaArgs& a, hipStream_t stream) {
  switch (a.heads / 16) {
    case 1: hipLaunchKernelGGL((partial_kernel<FP8, 1>), dim3(a.s.G), dim3(THREADS), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((partial_kernel<FP8, 2>), dim3(a.s.G), dim3(THREADS), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((partial_kernel<FP8, 3>), dim3(a.s.G), dim3(THREADS), 0, stream, a); break;
    default: hipLaunchKernelGGL((partial_kernel<FP8, 4>), dim3(a.s.G), dim3(THREADS), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace mlak

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream) {
  if (a.s.batch == 0) return hipSuccess;
  hipError_t e = a.fp8 ? mlak::launch<true>(a, stream) : mlak::launch<false>(a, stream);
  if (e != hipSuccess) return e;
  const ReducePlan rp = reduce_plan(a.s.batch, a.heads, a.s.G, mlak::RED_COL_PARTS);
  hipLaunchKernelGGL(mlak::reduce_kernel, rp.grid, dim3(REDUCE_THREADS), 0, stream, a, rp.by_segments ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dcp
