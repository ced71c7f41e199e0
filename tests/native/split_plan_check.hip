// Host-side check of the split plan both partial kernels follow (test
// infrastructure; the product library does not contain it).
//
// It runs the library's own planning functions (clamp_len, split_wgs,
// seg_tiles, seg_range from dcp_split.hpp) on the host for one configuration,
// walks every workgroup's range the way the partial kernels do, and checks:
//  - every tile of every row set is computed by exactly one workgroup;
//  - a row set's segments sit in consecutive workgroups g0 .. g0 + nseg - 1,
//    and seg_range (what the reduce kernel reads) names exactly those;
//  - a row set held by one workgroup is finished there (the reduce skips it),
//    one held by several is finished by none (the reduce merges it), one with
//    no tiles gets nseg = 0 (the reduce writes (0, -inf));
//  - the slot g + b each segment writes is unique and inside the workspace.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "dcp_split.hpp"

namespace {

int fail(char* msg, int len, const char* what, int a, int b, int c) {
  if (msg && len > 0) std::snprintf(msg, (size_t)len, "%s (%d, %d, %d)", what, a, b, c);
  return 1;
}

}  // namespace

extern "C" int dcp_split_plan_check(int nreq, const int32_t* lens, int q_len, int nshards, int rank, int layout,
                                    int block_size, int max_blocks, int G, int min_tiles, int seg_cost, int tile,
                                    char* msg, int msg_len) {
  if (nreq < 1 || q_len < 1 || G < 1 || G > dcp::kMaxSplitWGs || tile < 1 || min_tiles < 1)
    return fail(msg, msg_len, "bad arguments", nreq, q_len, G);
  dcp::SplitArgs s{};
  s.batch = nreq * q_len;
  s.q_len = q_len;
  s.nshards = nshards;
  s.rank = rank;
  s.layout = layout;
  s.block_size = block_size;
  s.max_blocks = max_blocks;
  s.G = G;
  s.min_tiles = min_tiles;
  s.seg_cost = seg_cost;
  const int rows = s.batch;

  // the plan's weights: a row set with n > 0 tiles weighs n + seg_cost
  std::vector<int> pref(rows + 1, 0), ntiles(rows, 0);
  for (int b = 0; b < rows; ++b) {
    const int req = b / q_len;
    const int n = (dcp::clamp_len(s, lens[req], b - req * q_len) + tile - 1) / tile;
    ntiles[b] = n;
    pref[b + 1] = pref[b] + (n > 0 ? n + seg_cost : 0);
  }
  const int T = pref[rows];
  const int geff = dcp::split_wgs(s, T);
  if (T > 0 && (geff < 1 || geff > G)) return fail(msg, msg_len, "split width", T, geff, G);
  if (T == 0 && geff != 0) return fail(msg, msg_len, "split width of an empty plan", T, geff, G);

  // what the partial kernels leave in the workspace metadata
  std::vector<int32_t> meta(rows + 2);
  meta[0] = geff;
  for (int i = 0; i <= rows; ++i) meta[1 + i] = pref[i];
  s.ws_meta = meta.data();

  std::vector<std::vector<uint8_t>> cover(rows);
  for (int b = 0; b < rows; ++b) cover[b].assign(ntiles[b], 0);
  std::vector<int> first_g(rows, -1), last_g(rows, -1), nseg(rows, 0);
  std::vector<uint8_t> finished(rows, 0), slot_used((size_t)dcp::kMaxSplitWGs + rows, 0);

  for (int g = 0; g < geff; ++g) {
    const int p0 = (int)((int64_t)g * T / geff);
    const int p1 = (int)((int64_t)(g + 1) * T / geff);
    int b = 0;  // largest b with pref[b] <= p0
    while (b + 1 < rows && pref[b + 1] <= p0) ++b;
    for (;;) {
      const int pb = pref[b], pe = pref[b + 1];
      const dcp::SegTiles st = dcp::seg_tiles(s, pb, pe, p0, p1);
      if (pe > pb && st.t1 > st.t0) {
        if (st.ntiles != ntiles[b]) return fail(msg, msg_len, "tile count", b, st.ntiles, ntiles[b]);
        if (st.t0 < 0 || st.t1 > ntiles[b]) return fail(msg, msg_len, "segment out of range", b, st.t0, st.t1);
        for (int k = st.t0; k < st.t1; ++k)
          if (cover[b][k]++) return fail(msg, msg_len, "tile computed twice", b, k, g);
        const int slot = g + b;
        if (slot >= dcp::kMaxSplitWGs + rows) return fail(msg, msg_len, "slot outside the workspace", g, b, slot);
        if (slot_used[slot]++) return fail(msg, msg_len, "slot written twice", g, b, slot);
        if (first_g[b] < 0) first_g[b] = g;
        else if (g != last_g[b] + 1) return fail(msg, msg_len, "segments not in consecutive workgroups", b, last_g[b], g);
        last_g[b] = g;
        ++nseg[b];
        if (st.t0 == 0 && st.t1 == ntiles[b]) finished[b] = 1;
      }
      if (pe >= p1 || b + 1 >= rows) break;
      ++b;
    }
  }

  for (int b = 0; b < rows; ++b) {
    for (int k = 0; k < ntiles[b]; ++k)
      if (cover[b][k] != 1) return fail(msg, msg_len, "tile not computed", b, k, ntiles[b]);
    const dcp::SegRange r = dcp::seg_range(s, b);
    if (ntiles[b] == 0) {
      if (r.nseg != 0) return fail(msg, msg_len, "empty row set given segments", b, r.g0, r.nseg);
      continue;
    }
    if (r.g0 != first_g[b] || r.nseg != nseg[b]) return fail(msg, msg_len, "seg_range disagrees", b, r.g0, r.nseg);
    if ((nseg[b] == 1) != (finished[b] != 0)) return fail(msg, msg_len, "finished flag", b, nseg[b], finished[b]);
  }
  return 0;
}
