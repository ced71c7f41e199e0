// Tile layout of the GQA partial kernel: which cache bytes each wave's copies
// move to which LDS bytes, and where the score and value operands are read.
// Shared by the kernel and by the host-side check of the layout.
//
// A workgroup streams HG consecutive KV heads (HG = 4, 2 or 1).  One part of a
// stage (K or V) is 16 KiB: TILE = 16 * SUB tokens x HG heads x 256 bytes,
// SUB = 4 / HG 16-token sub-tiles; token t of the tile is LDS row t (TROW
// bytes), head h of it the 256 bytes at h * 256.  Within a head's row the 16
// chunks of 16 bytes are XOR-swizzled by the token: LDS chunk p of token t
// holds cache chunk p ^ swz(t).  Wave w takes KV head w % HG of the group and
// sub-tile w / HG of every tile, and copies (part of) that sub-tile: 4 copies
// of 1 KiB per part, each SUB tokens x HG heads, so every copy stays inside one
// 16-token sub-tile and hence inside one cache block (block sizes are
// multiples of 16).
#pragma once

#include <stdint.h>

namespace dcp {
namespace gqa {

constexpr int D = 128;                 // head dim
constexpr int HROW = D * 2;            // bytes per (token, head) row
constexpr int HALF = 16 * 1024;        // the K (or V) part of a stage
constexpr int CPI = 4;                 // 1 KiB copy instructions per wave per part (16 per part)

template <int HG>
struct Geo {
  static_assert(HG == 1 || HG == 2 || HG == 4, "KV heads per workgroup");
  static constexpr int SUB = 4 / HG;           // 16-token sub-tiles per tile (one per wave of a head)
  static constexpr int TROW = HG * HROW;       // bytes per token in a tile
  static constexpr int TILE = 16 * SUB;        // tokens per tile
  static_assert(TILE * TROW == HALF, "a part is 16 KiB");
};

// Chunk swizzle of token row t inside one head's 16 chunks of 16 bytes.
__host__ __device__ constexpr int swz(int t) { return t & 15; }

// Copy slot of wave w's j-th copy of a part: 1 KiB at LDS offset 1024 * slot,
// holding tile tokens slot * SUB .. + SUB - 1.  With one sub-tile (HG = 4) the
// waves interleave tokens; otherwise wave w takes four consecutive slots, all
// inside its sub-tile w / HG.
template <int HG>
__host__ __device__ constexpr int copy_slot(int wave, int j) {
  return Geo<HG>::SUB == 1 ? 4 * j + wave : 4 * wave + j;
}

// Byte offset of lane `lane`'s 16 bytes of copy j of wave `wave`, from the
// cache address of (token 0 of the wave's sub-tile, head HG * group) in a cache
// whose token rows hold `hkv` heads: token slot * SUB + lane / (16 HG) of the
// tile, head (lane / 16) % HG of the group, swizzled chunk.
template <int HG>
__host__ __device__ inline uint32_t copy_src_offset(int wave, int j, int lane, int hkv) {
  const int tok = copy_slot<HG>(wave, j) * Geo<HG>::SUB + lane / (16 * HG);  // token of the tile
  const int h = (lane >> 4) % HG, ch = lane & 15;
  const int rel = tok - 16 * (wave / HG);  // from the copy sub-tile's token 0
  return (uint32_t)(rel * hkv * HROW + h * HROW + ((ch ^ swz(tok)) * 16));
}

// LDS byte offset (within a part) of lane `lane`'s 16 bytes of copy j of wave
// `wave` (a global->LDS copy puts lane i at its base + 16 i).
template <int HG>
__host__ __device__ constexpr int copy_dst_offset(int wave, int j, int lane) {
  return copy_slot<HG>(wave, j) * 1024 + 16 * lane;
}

// LDS byte offset (within the K part) of the 16 bytes holding cache chunk
// `chunk` (k = 8 chunk .. + 7) of token r16 of sub-tile `sub`, head hk.
template <int HG>
__host__ __device__ constexpr int k_read_offset(int sub, int r16, int hk, int chunk) {
  return (16 * sub + r16) * Geo<HG>::TROW + hk * HROW + ((chunk ^ swz(r16)) * 16);
}

// LDS byte offset (within the V part) of the 8 bytes lane (g4, r16) hands to
// the transposing read of value column block cb: token row 4 g4 + r16 / 4 of
// sub-tile `sub`, head hk, columns 16 cb + 4 (r16 % 4) .. + 3, so that the read
// gives lane r16 of each 16-lane group column 16 cb + r16 of 4 tokens.
template <int HG>
__host__ __device__ constexpr int v_read_offset(int sub, int g4, int r16, int hk, int cb) {
  return (16 * sub + 4 * g4 + (r16 >> 2)) * Geo<HG>::TROW + hk * HROW + (r16 & 1) * 8 +
         (((2 * cb + ((r16 & 3) >> 1)) ^ swz(4 * g4 + (r16 >> 2))) * 16);
}

}  // namespace gqa
}  // namespace dcp
