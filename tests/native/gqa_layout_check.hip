// Host-side check of the GQA partial kernel's tile layout (test
// infrastructure; the product library does not contain it).
//
// It runs the kernel's own layout functions (gqa_layout.hpp) on the host for
// HG = 4, 2 and 1 KV heads per workgroup and a cache of hkv heads per token,
// and checks:
//  - the 16 copies of 1 KiB of a part (4 waves x 4) write every 16-byte LDS
//    chunk of the 16 KiB part exactly once;
//  - each lane's copy reads the cache bytes that belong where it writes:
//    token t of the tile into LDS row t, head h into head slot h, cache chunk
//    p ^ swz(t) into LDS chunk p;
//  - every copy of a wave stays inside the wave's 16-token sub-tile (so one
//    block-table entry gives its base), and the sub-tile a wave copies is the
//    one it computes;
//  - every score-operand read of a wave (token r16 of its sub-tile, its head,
//    k chunk c) lands on the LDS chunk holding cache chunk c of that token and
//    head;
//  - every value-operand read lands on 8 bytes holding columns
//    16 cb + 4 (r16 % 4) .. + 3 of token 4 g4 + r16 / 4 of the sub-tile.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "gqa_layout.hpp"

namespace {

using namespace dcp::gqa;

int fail(char* msg, int len, const char* what, int a, int b, int c) {
  if (msg && len > 0) std::snprintf(msg, (size_t)len, "%s (%d, %d, %d)", what, a, b, c);
  return 1;
}

// LDS position (token row, head slot, chunk, byte in chunk) of a part offset
struct Pos {
  int t, h, p, byte;
};
template <int HG>
Pos decode_lds(int off) {
  return {off / Geo<HG>::TROW, (off % Geo<HG>::TROW) / HROW, (off % HROW) / 16, off % 16};
}

template <int HG>
int check(int hkv, char* msg, int len) {
  using G = Geo<HG>;
  if (hkv % HG != 0) return fail(msg, len, "hkv not a multiple of HG", hkv, HG, 0);
  std::vector<int> seen(HALF / 16, 0);
  for (int wave = 0; wave < 4; ++wave) {
    const int sub = wave / HG;  // the sub-tile the wave computes (KV head wave % HG)
    for (int j = 0; j < CPI; ++j) {
      for (int lane = 0; lane < 64; ++lane) {
        const int dst = copy_dst_offset<HG>(wave, j, lane);
        if (dst < 0 || dst + 16 > HALF || dst % 16) return fail(msg, len, "copy destination out of the part", wave, j, lane);
        ++seen[dst / 16];
        const Pos q = decode_lds<HG>(dst);
        const uint32_t src = copy_src_offset<HG>(wave, j, lane, hkv);
        const int token_bytes = hkv * HROW;
        const int rel = (int)(src / (uint32_t)token_bytes);
        const int h = (int)(src % (uint32_t)token_bytes) / HROW;
        const int ch = (int)(src % HROW) / 16;
        if (src % 16) return fail(msg, len, "copy source not 16-byte aligned", wave, j, lane);
        if (rel < 0 || rel >= 16) return fail(msg, len, "copy leaves the wave's 16-token sub-tile", wave, j, lane);
        if (16 * sub + rel != q.t) return fail(msg, len, "copy token lands in another LDS row", wave, j, lane);
        if (h >= HG || h != q.h) return fail(msg, len, "copy head lands in another head slot", wave, j, lane);
        if ((q.p ^ swz(q.t)) != ch) return fail(msg, len, "copy chunk does not follow the swizzle", wave, j, lane);
      }
    }
  }
  for (int c = 0; c < HALF / 16; ++c)
    if (seen[c] != 1) return fail(msg, len, "LDS chunk written other than once", c, seen[c], HG);

  for (int sub = 0; sub < G::SUB; ++sub)
    for (int hk = 0; hk < HG; ++hk)
      for (int lane = 0; lane < 64; ++lane) {
        const int g4 = lane >> 4, r16 = lane & 15;
        for (int c = 0; c < 16; ++c) {
          const int off = k_read_offset<HG>(sub, r16, hk, c);
          if (off < 0 || off + 16 > HALF) return fail(msg, len, "K read out of the part", sub, hk, c);
          const Pos q = decode_lds<HG>(off);
          if (q.byte || q.t != 16 * sub + r16 || q.h != hk || (q.p ^ swz(q.t)) != c)
            return fail(msg, len, "K read misses its chunk", sub, r16, c);
        }
        for (int cb = 0; cb < D / 16; ++cb) {
          const int off = v_read_offset<HG>(sub, g4, r16, hk, cb);
          if (off < 0 || off + 8 > HALF) return fail(msg, len, "V read out of the part", sub, hk, cb);
          const Pos q = decode_lds<HG>(off);
          const int col = 8 * (q.p ^ swz(q.t)) + q.byte / 2;  // first of the 4 bf16 columns read
          if (q.byte % 8 || q.t != 16 * sub + 4 * g4 + (r16 >> 2) || q.h != hk || col != 16 * cb + 4 * (r16 & 3))
            return fail(msg, len, "V read misses its columns", sub, lane, cb);
        }
      }
  return 0;
}

}  // namespace

extern "C" int dcp_gqa_layout_check(int hg, int hkv, char* msg, int msg_len) {
  switch (hg) {
    case 4: return check<4>(hkv, msg, msg_len);
    case 2: return check<2>(hkv, msg, msg_len);
    case 1: return check<1>(hkv, msg, msg_len);
    default: return fail(msg, msg_len, "bad HG", hg, hkv, 0);
  }
}
