// Host side of the C ABI: argument validation, launch planning, status codes.
// Nothing here reads device memory or synchronizes; every launch goes to the
// caller's stream.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "dcp.h"
#include "dcp_internal.hpp"

// Split workspace of the no-allocation entry point: one array per GPU, held
// for the life of the process.  Host code never uses the name `scratch` as an
// address (on the host it is only a stand-in for the device symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current (scratch_addr below).
static __device__ __align__(256) char scratch[DCP_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

dcp_status hip_status(hipError_t e) {
  if (e == hipSuccess) return DCP_OK;
  g_last_hip_error = (int)e;
  return DCP_ERR_HIP;
}

int env_int(const char* name, int dflt, int lo, int hi) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  long x = std::strtol(v, nullptr, 10);
  if (x < lo) x = lo;
  if (x > hi) x = hi;
  return (int)x;
}

// Compute units of the current device, cached per device.
int device_cus(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { *err = e; return 0; }
  static std::atomic<int> cache[64];
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0) { *err = e != hipSuccess ? e : hipErrorInvalidDevice; return 0; }
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Checks shared by both partial entry points.
dcp_status check_split(int batch, int block_size, int max_blocks, int num_blocks, int rank,
                       int nshards, dcp_layout layout, int hint, float scale) {
  if (batch < 0 || nshards < 1 || rank < 0 || rank >= nshards) return DCP_ERR_INVALID_ARGUMENT;
  if (layout != DCP_LAYOUT_ROUND_ROBIN && layout != DCP_LAYOUT_CONTIGUOUS) return DCP_ERR_INVALID_ARGUMENT;
  if (block_size < 1 || max_blocks < 1 || num_blocks < 1 || hint < 1) return DCP_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || !std::isfinite(scale)) return DCP_ERR_INVALID_ARGUMENT;
  if (block_size % 16 != 0 || block_size > 1024) return DCP_ERR_UNSUPPORTED;
  const int64_t cap = (int64_t)max_blocks * block_size;
  if (cap > INT32_MAX) return DCP_ERR_UNSUPPORTED;
  // the longest local slice of a request of length `hint` must fit one table row
  const int64_t local_max = ((int64_t)hint + nshards - 1) / nshards;
  if (local_max > cap) return DCP_ERR_INVALID_ARGUMENT;
  if (batch > dcp::kMaxBatch) return DCP_ERR_UNSUPPORTED;
  return DCP_OK;
}

dcp::SplitArgs split_args(int batch, int block_size, int max_blocks, int num_blocks, int rank,
                          int nshards, dcp_layout layout, float scale, const int32_t* table,
                          const int32_t* seq_lens, float* out, float* lse, void* ws,
                          const dcp::WsLayout& wl) {
  dcp::SplitArgs s;
  s.table = table;
  s.seq_lens = seq_lens;
  s.ws_meta = (int32_t*)((char*)ws + wl.meta_off);
  s.ws_ml = (float*)((char*)ws + wl.ml_off);
  s.ws_o = (char*)ws + wl.o_off;
  s.out = out;
  s.lse = lse;
  s.batch = batch;
  s.block_size = block_size;
  s.max_blocks = max_blocks;
  s.num_blocks = num_blocks;
  s.rank = rank;
  s.nshards = nshards;
  s.layout = (int)layout;
  s.G = 0;
  s.min_tiles = 1;
  s.seg_cost = 0;
  s.q_len = 1;
  s.scale = scale;
  s.c = scale * 1.4426950408889634f;
  return s;
}

// Query tokens per request (0 means 1) and the row sets of the split.
int qlen_of(int32_t q_len) { return q_len <= 0 ? 1 : q_len; }
int rows_of(int32_t batch, int32_t q_len) {
  const int64_t r = (int64_t)batch * qlen_of(q_len);
  return r > INT32_MAX ? INT32_MAX : (int)r;
}
dcp_status check_qlen(int32_t q_len) {
  if (q_len < 0) return DCP_ERR_INVALID_ARGUMENT;
  if (q_len > 16) return DCP_ERR_UNSUPPORTED;
  return DCP_OK;
}

dcp_status mla_check(const dcp_mla_params* p) {
  if (!p) return DCP_ERR_INVALID_ARGUMENT;
  if (check_qlen(p->q_len) != DCP_OK) return check_qlen(p->q_len);
  if (p->num_heads < 1 || p->kv_lora_rank < 1 || p->rope_dim < 1) return DCP_ERR_INVALID_ARGUMENT;
  dcp_status st = check_split(p->batch < 0 ? -1 : rows_of(p->batch, p->q_len), p->block_size,
                              p->max_blocks_per_seq, p->num_blocks, p->shard_rank, p->num_shards, p->layout,
                              p->max_seq_len_hint, p->softmax_scale);
  if (st != DCP_OK) return st;
  if (p->kv_lora_rank != 512 || p->rope_dim != 64) return DCP_ERR_UNSUPPORTED;
  if (p->num_heads % 16 != 0 || p->num_heads > 64) return DCP_ERR_UNSUPPORTED;
  return DCP_OK;
}

dcp_status gqa_check(const dcp_gqa_params* p) {
  if (!p) return DCP_ERR_INVALID_ARGUMENT;
  if (check_qlen(p->q_len) != DCP_OK) return check_qlen(p->q_len);
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1) return DCP_ERR_INVALID_ARGUMENT;
  if (p->num_q_heads % p->num_kv_heads != 0) return DCP_ERR_INVALID_ARGUMENT;
  dcp_status st = check_split(p->batch < 0 ? -1 : rows_of(p->batch, p->q_len), p->block_size,
                              p->max_blocks_per_seq, p->num_blocks, p->shard_rank, p->num_shards, p->layout,
                              p->max_seq_len_hint, p->softmax_scale);
  if (st != DCP_OK) return st;
  if (p->head_dim != 128) return DCP_ERR_UNSUPPORTED;
  if (p->num_kv_heads > 64) return DCP_ERR_UNSUPPORTED;
  if (p->num_q_heads / p->num_kv_heads > 64) return DCP_ERR_UNSUPPORTED;
  return DCP_OK;
}

std::mutex g_scratch_mu;
void* g_scratch_addr[64];

// The current device's scratch address (looked up on first use).
hipError_t scratch_addr(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = a;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

// Both MLA entry points: bf16 cache, or E4M3 cache with dequantization scale kv_scale.
// noalloc: the workspace arguments are ignored and the split workspace is the
// device scratch, laid out for this call's split width.
dcp_status mla_partial(const dcp_mla_params* p, const void* q, const void* kv_cache, bool fp8, float kv_scale,
                       const int32_t* block_table, const int32_t* seq_lens, float* out, float* lse,
                       void* workspace, size_t workspace_bytes, hipStream_t stream, bool noalloc = false) {
  dcp_status st = mla_check(p);
  if (st != DCP_OK) return st;
  if (fp8) {
    // the scaled softmax scale must stay a finite, normal fp32 number
    const double c = (double)p->softmax_scale * (double)kv_scale;
    if (!(kv_scale > 0.f) || !std::isfinite(kv_scale) || !(c >= 1e-30 && c <= 1e30))
      return DCP_ERR_INVALID_ARGUMENT;
  }
  if (p->batch == 0) return DCP_OK;
  if (!q || !kv_cache || !block_table || !seq_lens || !out || !lse) return DCP_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(lse, 4))
    return DCP_ERR_INVALID_ARGUMENT;
  const int rows = rows_of(p->batch, p->q_len);
  dcp::WsLayout wl;
  if (!noalloc) {
    wl = dcp::ws_layout(rows, p->num_heads, 512, 2);
    if (!workspace || workspace_bytes < wl.total || !aligned(workspace, 256)) return DCP_ERR_WORKSPACE;
  }
  hipError_t herr = hipSuccess;
  const int cus = device_cus(&herr);
  if (cus <= 0) return hip_status(herr);
  const int G = env_int("DCP_SPLIT_WGS", cus < dcp::kMaxSplitWGs ? cus : dcp::kMaxSplitWGs, 1, dcp::kMaxSplitWGs);
  if (noalloc) {
    // slots g + b of a split over G workgroups: G + rows of them
    wl = dcp::ws_layout_slots((size_t)G + (size_t)rows, p->num_heads, 512, 2);
    if (wl.total > DCP_NOALLOC_SCRATCH_BYTES) return DCP_ERR_SCRATCH;
    herr = scratch_addr(&workspace);
    if (herr != hipSuccess) return hip_status(herr);
  }

  dcp::MlaArgs a;
  a.s = split_args(rows, p->block_size, p->max_blocks_per_seq, p->num_blocks, p->shard_rank,
                   p->num_shards, p->layout, fp8 ? p->softmax_scale * kv_scale : p->softmax_scale, block_table,
                   seq_lens, out, lse, workspace, wl);
  a.s.q_len = qlen_of(p->q_len);
  a.s.G = G;
  a.s.min_tiles = env_int(fp8 ? "DCP_MLA8_MIN_TILES" : "DCP_MLA_MIN_TILES", 4, 1, 1 << 20);
  a.s.seg_cost = env_int(fp8 ? "DCP_MLA8_SEG_COST" : "DCP_MLA_SEG_COST", 6, 0, 64);
  a.q = (const uint16_t*)q;
  a.kv = kv_cache;
  a.heads = p->num_heads;
  a.fp8 = fp8;
  a.vscale = fp8 ? kv_scale : 1.0f;
  return hip_status(dcp::launch_mla_partial(a, stream));
}

}  // namespace

extern "C" {

int dcp_abi_version(void) { return DCP_ABI_VERSION; }

int dcp_last_hip_error(void) { return g_last_hip_error; }

const char* dcp_status_string(dcp_status s) {
  switch (s) {
    case DCP_OK: return "ok";
    case DCP_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DCP_ERR_UNSUPPORTED: return "unsupported configuration";
    case DCP_ERR_WORKSPACE: return "workspace missing or too small";
    case DCP_ERR_HIP: return "HIP error";
    case DCP_ERR_SCRATCH: return "call needs more than the fixed device scratch of the no-allocation entry point";
  }
  return "unknown status";
}

size_t dcp_mla_workspace_bytes(const dcp_mla_params* p) {
  if (mla_check(p) != DCP_OK) return 0;
  return dcp::ws_layout(rows_of(p->batch, p->q_len), p->num_heads, 512, 2).total;
}

dcp_status dcp_mla_decode_partial(const dcp_mla_params* p, const void* q, const void* kv_cache,
                                  const int32_t* block_table, const int32_t* seq_lens, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  return mla_partial(p, q, kv_cache, false, 1.0f, block_table, seq_lens, out, lse, workspace, workspace_bytes,
                     stream);
}

dcp_status dcp_mla_decode_partial_fp8(const dcp_mla_params* p, const void* q, const void* kv_cache,
                                      float kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                                      float* out, float* lse, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  return mla_partial(p, q, kv_cache, true, kv_scale, block_table, seq_lens, out, lse, workspace, workspace_bytes,
                     stream);
}

dcp_status dcp_mla_decode_partial_noalloc(const dcp_mla_params* p, const void* q, const void* kv_cache,
                                          const int32_t* block_table, const int32_t* seq_lens, float* out,
                                          float* lse, hipStream_t stream) {
  return mla_partial(p, q, kv_cache, false, 1.0f, block_table, seq_lens, out, lse, nullptr, 0, stream, true);
}

size_t dcp_gqa_workspace_bytes(const dcp_gqa_params* p) {
  if (gqa_check(p) != DCP_OK) return 0;
  return dcp::ws_layout(rows_of(p->batch, p->q_len), p->num_q_heads, 128, 4).total;
}

dcp_status dcp_gqa_decode_partial(const dcp_gqa_params* p, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, float* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  dcp_status st = gqa_check(p);
  if (st != DCP_OK) return st;
  if (p->batch == 0) return DCP_OK;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out || !lse)
    return DCP_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(lse, 4))
    return DCP_ERR_INVALID_ARGUMENT;
  const int rows = rows_of(p->batch, p->q_len);
  const dcp::WsLayout wl = dcp::ws_layout(rows, p->num_q_heads, 128, 4);
  if (!workspace || workspace_bytes < wl.total || !aligned(workspace, 256)) return DCP_ERR_WORKSPACE;
  hipError_t herr = hipSuccess;
  const int cus = device_cus(&herr);
  if (cus <= 0) return hip_status(herr);

  dcp::GqaArgs a;
  a.s = split_args(rows, p->block_size, p->max_blocks_per_seq, p->num_blocks, p->shard_rank,
                   p->num_shards, p->layout, p->softmax_scale, block_table, seq_lens, out, lse,
                   workspace, wl);
  a.s.q_len = qlen_of(p->q_len);
  // one workgroup column per group of KV heads streamed together; together
  // they fill the chip once
  const int groups = p->num_kv_heads / dcp::gqa_heads_per_workgroup(p->num_kv_heads);
  int g = (cus + groups - 1) / groups;
  if (g > dcp::kMaxSplitWGs) g = dcp::kMaxSplitWGs;
  a.s.G = env_int("DCP_SPLIT_WGS", g, 1, dcp::kMaxSplitWGs);
  a.s.min_tiles = env_int("DCP_GQA_MIN_TILES", 16, 1, 1 << 20);
  a.s.seg_cost = env_int("DCP_GQA_SEG_COST", 0, 0, 64);
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  return hip_status(dcp::launch_gqa_partial(a, stream));
}

dcp_status dcp_combine(int32_t num_shards, int32_t batch, int32_t num_heads, int32_t head_dim_v,
                       const float* partial_out, const float* partial_lse, void* out_bf16,
                       float* out_f32, float* lse_out, hipStream_t stream) {
  if (num_shards < 1 || batch < 0 || num_heads < 1 || head_dim_v < 1) return DCP_ERR_INVALID_ARGUMENT;
  if (num_shards > 64 || head_dim_v % 4 != 0 || head_dim_v > 1024) return DCP_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)batch * num_heads;
  if (rows > INT32_MAX / 4) return DCP_ERR_UNSUPPORTED;
  if (rows == 0) return DCP_OK;
  if (!partial_out || !partial_lse || (!out_bf16 && !out_f32)) return DCP_ERR_INVALID_ARGUMENT;
  if (!aligned(partial_out, 16) || !aligned(partial_lse, 4) || !aligned(out_bf16, 8) ||
      !aligned(out_f32, 16) || !aligned(lse_out, 4))
    return DCP_ERR_INVALID_ARGUMENT;
  dcp::CombineArgs a;
  a.po = partial_out;
  a.plse = partial_lse;
  a.out_bf16 = (uint16_t*)out_bf16;
  a.out_f32 = out_f32;
  a.lse_out = lse_out;
  a.nshards = num_shards;
  a.rows = (int)rows;
  a.dv = head_dim_v;
  a.pad = 0.f;
  return hip_status(dcp::launch_combine(a, stream));
}

dcp_status dcp_combine_vproj_gate(int32_t num_shards, int32_t batch, int32_t num_heads, int32_t head_dim_v,
                                  int32_t out_dim, const float* partial_out, const float* partial_lse,
                                  const void* w_uv_t, const void* gate, void* out_bf16, float* out_f32,
                                  float* lse_out, hipStream_t stream) {
  if (num_shards < 1 || batch < 0 || num_heads < 1 || head_dim_v < 1 || out_dim < 1) return DCP_ERR_INVALID_ARGUMENT;
  if (num_shards > 64 || head_dim_v % 32 != 0 || head_dim_v > 1024 || out_dim % 16 != 0 || out_dim > 256)
    return DCP_ERR_UNSUPPORTED;
  if ((int64_t)batch * num_heads > INT32_MAX / 4 || num_heads > 65535) return DCP_ERR_UNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!partial_out || !partial_lse || !w_uv_t || (!out_bf16 && !out_f32)) return DCP_ERR_INVALID_ARGUMENT;
  if (!aligned(partial_out, 16) || !aligned(partial_lse, 4) || !aligned(w_uv_t, 16) || !aligned(gate, 2) ||
      !aligned(out_bf16, 2) || !aligned(out_f32, 4) || !aligned(lse_out, 4))
    return DCP_ERR_INVALID_ARGUMENT;
  dcp::VprojArgs a;
  a.po = partial_out;
  a.plse = partial_lse;
  a.w = (const uint16_t*)w_uv_t;
  a.gate = (const uint16_t*)gate;
  a.out_bf16 = (uint16_t*)out_bf16;
  a.out_f32 = out_f32;
  a.lse_out = lse_out;
  a.nshards = num_shards;
  a.batch = batch;
  a.heads = num_heads;
  a.dv = head_dim_v;
  a.dvo = out_dim;
  return hip_status(dcp::launch_combine_vproj(a, stream));
}

}  // extern "C"
