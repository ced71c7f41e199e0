// Internal (non-ABI) declarations shared by the host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dcp {

// Upper bound on the number of split workgroups one partial call launches.  The
// workspace is sized for it, so its size depends on (batch, heads) only.
constexpr int kMaxSplitWGs = 512;
// Largest batch the in-kernel split planner handles (its prefix sums sit in LDS).
constexpr int kMaxBatch = 2048;

// Workspace layout of a partial call (all offsets 256-byte aligned):
//   meta  int32 [kMaxBatch + 2]: [0] = split WGs used, [1 + b] = tile prefix sum
//   ml    fp32  [slots][heads][2]: running max (raw score units) and softmax sum
//   o     [slots][heads][dv]: unnormalized partial output, fp32 (GQA) or bf16
//         (MLA: one 64-head partial is 64 KiB instead of 128, halving the
//         split traffic; see the partial kernel)
// slots = kMaxSplitWGs + batch.
struct WsLayout {
  size_t meta_off, ml_off, o_off, total;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// Layout for `slots` partial slots (a call whose split uses G workgroups
// needs G + batch slots; ws_layout reserves the most any call uses).
inline WsLayout ws_layout_slots(size_t slots, int heads, int dv, size_t o_bytes) {
  WsLayout w;
  w.meta_off = 0;
  w.ml_off = align256(sizeof(int32_t) * (kMaxBatch + 2));
  w.o_off = w.ml_off + align256(sizeof(float) * slots * heads * 2);
  w.total = w.o_off + align256(o_bytes * slots * heads * dv);
  return w;
}
inline WsLayout ws_layout(int batch, int heads, int dv, size_t o_bytes) {
  return ws_layout_slots((size_t)kMaxSplitWGs + (size_t)batch, heads, dv, o_bytes);
}

struct SplitArgs {
  const int32_t* table;
  const int32_t* seq_lens;
  int32_t* ws_meta;
  float* ws_ml;
  void* ws_o;  // element type per kernel (fp32 or bf16)
  float* out;
  float* lse;
  int batch, block_size, max_blocks, num_blocks, rank, nshards, layout;
  int G;          // split workgroups launched
  int min_tiles;  // fewest tiles a split workgroup is given
  int seg_cost;   // tiles' worth of work charged per request for its segment boundaries (half before its tiles, half after)
  int q_len;      // query tokens per request: row set b is request b / q_len, token b % q_len
  float scale;    // softmax scale
  float c;        // softmax scale * log2(e)
};

struct MlaArgs {
  SplitArgs s;
  const uint16_t* q;
  const void* kv;  // bf16 or E4M3 rows of 576
  int heads;
  bool fp8;        // E4M3 cache (s.c then includes the dequantization scale)
  float vscale;    // multiplier of the output: the dequantization scale (fp8), else 1
};

struct GqaArgs {
  SplitArgs s;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int hq, hkv;
};

struct CombineArgs {
  const float* po;
  const float* plse;
  uint16_t* out_bf16;
  float* out_f32;
  float* lse_out;
  int nshards, rows, dv;
  float pad;
};

struct VprojArgs {
  const float* po;
  const float* plse;
  const uint16_t* w;     // bf16 [heads][dvo][dv]
  const uint16_t* gate;  // bf16 [batch][heads][dvo] or null
  uint16_t* out_bf16;
  float* out_f32;
  float* lse_out;
  int nshards, batch, heads, dv, dvo;
};

hipError_t launch_mla_partial(const MlaArgs& a, hipStream_t stream);
hipError_t launch_gqa_partial(const GqaArgs& a, hipStream_t stream);
// KV heads one GQA workgroup streams together (4, 2 or 1: the largest dividing Hkv).
int gqa_heads_per_workgroup(int hkv);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_combine_vproj(const VprojArgs& a, hipStream_t stream);

}  // namespace dcp
