/*
 * dcp.h — C ABI for the hot path of Decode Context Parallelism (DCP) on one
 * AMD Instinct MI355X (gfx950).
 *
 * DCP splits every request's KV cache along the sequence: each of N ranks
 * holds a distinct subset of the token positions (vLLM blog post on Decode
 * Context Parallelism, section 4 "What is DCP?").  At decode time each rank
 * attends the full query against its local slice only and produces a partial
 * output together with the log-sum-exp (LSE) of its scores; the N partials
 * are then reweighted by their LSEs and summed, which reproduces exact
 * attention (section 4.1, the "Compute" and "AllGather + ReduceScatter"
 * steps).  This library provides those two device steps:
 *
 *   dcp_mla_decode_partial  one rank's partial for MLA (one latent row per
 *                           token shared by all query heads; section 5.3)
 *   dcp_mla_decode_partial_fp8
 *                           the same over an fp8 (OCP E4M3) latent cache with
 *                           one dequantization scale
 *   dcp_gqa_decode_partial  one rank's partial for GQA (KV heads shared by
 *                           consecutive groups of query heads; section 5.4)
 *   dcp_combine             the LSE-weighted merge of N partials, fused with
 *                           the cast of the result to bf16
 *   dcp_combine_vproj_gate  the same merge fused with each head's value
 *                           up-projection and a sigmoid output gate
 *
 * On one GPU the N ranks are simulated as N disjoint slices resident in the
 * same HBM; the cross-GPU exchange is not part of this library.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is DEVICE memory owned by the caller, except the
 *   parameter structs, which are host memory read during the call only.  The
 *   library never allocates, frees or keeps a pointer after returning.
 * - Calls are asynchronous: they validate on the host, enqueue kernels on
 *   `stream` (0 = the null stream of the current device) and return.  There
 *   is no device-to-host read and no synchronization.  Inputs must stay valid
 *   and unmodified until the enqueued work completes.
 * - A call sizes its launch for the current device (hipGetDevice): make the
 *   device that holds the buffers current, and pass a stream of that device.
 * - Argument errors are detected on the host before anything is enqueued; the
 *   call then returns a non-zero status and launches nothing.  A failed launch
 *   returns DCP_ERR_HIP; dcp_last_hip_error() gives the hipError_t value.
 * - Values read from device memory (seq_lens, block ids) cannot be validated
 *   without a sync.  The kernels clamp them so that no access leaves the
 *   buffers described by the parameters: a local length is clamped to the
 *   table capacity max_blocks_per_seq * block_size, a block id to
 *   [0, num_blocks), and seq_lens[b] <= 0 means the request has no tokens.
 *   Results for such inputs are unspecified but never fault.
 * - bf16 is the IEEE-754 binary32 upper half (1-8-7), stored as uint16.
 * - All entry points are thread-safe and reentrant; the library holds no
 *   per-call state.
 */
#ifndef DCP_H_
#define DCP_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCP_ABI_VERSION 3

typedef enum {
  DCP_OK = 0,
  DCP_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, rank out of range ... */
  DCP_ERR_UNSUPPORTED = 2,      /* valid but not implemented (dims, head counts, block size) */
  DCP_ERR_WORKSPACE = 3,        /* workspace missing or smaller than *_workspace_bytes() */
  DCP_ERR_HIP = 4,              /* a HIP call failed; see dcp_last_hip_error() */
  DCP_ERR_SCRATCH = 5           /* the call needs more than the fixed device scratch of
                                   dcp_mla_decode_partial_noalloc (DCP_NOALLOC_SCRATCH_BYTES) */
} dcp_status;

/* How a request's token positions are spread over the N shards
 * (section 4 of the DCP post gives the contiguous example).
 *  ROUND_ROBIN: global position t lives on shard t mod N at local index t div N.
 *  CONTIGUOUS : shard r holds positions [r*C, min(L, (r+1)*C)), C = ceil(L/N),
 *               at local index t - r*C.
 * The local slice of shard r is therefore a contiguous run of local indices
 * 0 .. L_r-1; the kernels only need L_r, which they derive from the global
 * length L, N, r and the layout. */
typedef enum { DCP_LAYOUT_ROUND_ROBIN = 0, DCP_LAYOUT_CONTIGUOUS = 1 } dcp_layout;

/* Multi-token steps (q_len = Q > 1), for verifying Q speculative tokens in one
 * decode step (DCP post, section 6 "Future Work", names MTP / speculative
 * decoding with DCP): the cache already holds the step's Q tokens as its last
 * Q positions, seq_lens[b] = L counts them, and query token j (0-based) of
 * request b attends the causal prefix of global positions t <= L - Q + j.
 * The shard layout is that of the cache of length L (for CONTIGUOUS,
 * C = ceil(L/N)); each shard attends the part of every query's prefix it
 * holds.  q, out and lse gain a token index after the request index:
 *     q [batch][Q][heads][dk], out [batch][Q][heads][dv], lse [batch][Q][heads]
 * block_table and seq_lens stay per request.  batch * Q <= 2048.  Each (request,
 * token) pair is its own row set in the split (the KV slice is read once per
 * query token). */

/* ------------------------------------------------------------------ MLA */

typedef struct {
  int32_t batch;              /* requests in the decode step, >= 0 (0 = no-op)             */
  int32_t num_heads;          /* query heads H; 16, 32, 48 or 64                            */
  int32_t kv_lora_rank;       /* latent width R (c_kv); must be 512                         */
  int32_t rope_dim;           /* rotary key width P (k_rope); must be 64                    */
  int32_t block_size;         /* tokens per cache block; a multiple of 16, 16..1024         */
  int32_t max_blocks_per_seq; /* columns of block_table, >= 1                               */
  int32_t num_blocks;         /* blocks in this shard's pool, >= 1                          */
  int32_t shard_rank;         /* r, 0 <= r < num_shards                                     */
  int32_t num_shards;         /* N >= 1                                                     */
  dcp_layout layout;
  int32_t max_seq_len_hint;   /* host-known upper bound on seq_lens[]; >= 1; the shard's
                                 local slice of such a request must fit in one table row     */
  float softmax_scale;        /* multiplies <q, k> before the softmax (> 0, finite)         */
  int32_t q_len;              /* query tokens per request in this step, 0..16 (0 means 1);
                                 see "Multi-token steps" below                               */
} dcp_mla_params;

/* Bytes of device workspace dcp_mla_decode_partial needs for `p`
 * (0 if p is invalid).  Depends only on batch and num_heads. */
size_t dcp_mla_workspace_bytes(const dcp_mla_params* p);

/* One shard's partial MLA decode attention (sections 4.1 and 5.3 of the DCP
 * post: the rank attends the gathered query against its local latent slice).
 * Absorbed form: for each request b and head h, over the shard's local
 * tokens t,
 *     z_t   = softmax_scale * <q[b][h][0:R+P], kv[t][0:R+P]>
 *     lse   = log(sum_t exp(z_t))                       (natural log)
 *     out   = sum_t exp(z_t - lse) * kv[t][0:R]
 * A request whose local slice is empty gets out = 0 and lse = -inf, which the
 * combine treats as "no contribution".
 *
 *  q           bf16 [batch][num_heads][R+P], row-major
 *  kv_cache    bf16 [num_blocks][block_size][R+P]: this shard's pool
 *  block_table int32 [batch][max_blocks_per_seq]: physical block of local block j
 *  seq_lens    int32 [batch]: GLOBAL context length of each request
 *  out         fp32 [batch][num_heads][R] (written)
 *  lse         fp32 [batch][num_heads]    (written)
 *  workspace   device scratch of >= dcp_mla_workspace_bytes(p) bytes, 256-byte
 *              aligned; contents need no initialization and are clobbered.
 * Calls that share a workspace must be ordered on one stream. */
dcp_status dcp_mla_decode_partial(const dcp_mla_params* p, const void* q, const void* kv_cache,
                                  const int32_t* block_table, const int32_t* seq_lens, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* dcp_mla_decode_partial for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops that forbid hipMalloc): the
 * same computation and kernels, with the split workspace taken from a fixed
 * array in device memory that the library holds for the life of the process,
 * one per GPU (DCP_NOALLOC_SCRATCH_BYTES = 32 MiB each).  The call itself
 * allocates nothing; on its first use on a device it looks up that device's
 * array address (hipGetSymbolAddress) with the device current.
 *
 * The scratch needed is 256-byte-aligned metadata, (m, l) pairs and bf16
 * split partials for (split workgroups + batch * q_len) slots of num_heads
 * rows of 512, where the split uses one workgroup per compute unit: at 64
 * heads and 256 compute units, batch * q_len up to 244 fits.  A larger call
 * returns DCP_ERR_SCRATCH and launches nothing.
 *
 * Every call on a GPU shares that GPU's array (the scratch needs no
 * clearing; the kernels write what they read).  Calls that overlap on one
 * GPU race: order them on one stream.  Arguments, results and every other
 * error are those of dcp_mla_decode_partial. */
#define DCP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dcp_status dcp_mla_decode_partial_noalloc(const dcp_mla_params* p, const void* q, const void* kv_cache,
                                          const int32_t* block_table, const int32_t* seq_lens, float* out,
                                          float* lse, hipStream_t stream);

/* dcp_mla_decode_partial over an fp8 latent cache.  The Kimi K3 optimizations
 * page ("Kimi K3 Performance Optimizations in vLLM", decode context
 * parallelism and its serving recipe) runs the KV cache in fp8; the pages fix
 * no encoding, so this library reads the OCP 8-bit float E4M3 format (1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 =
 * NaN, largest magnitude 448) with one scale for the whole cache: stored code
 * x stands for kv_scale * x.  The result is dcp_mla_decode_partial's over the
 * dequantized rows:
 *     z_t   = softmax_scale * <q[b][h], kv_scale * kv[t]>
 *     out   = sum_t exp(z_t - lse) * kv_scale * kv[t][0:R]
 *
 *  kv_cache    E4M3 codes, uint8 [num_blocks][block_size][R+P] (576 bytes per
 *              row), 16-byte aligned
 *  kv_scale    > 0 and finite; softmax_scale * kv_scale must lie in
 *              [1e-30, 1e30]; otherwise DCP_ERR_INVALID_ARGUMENT
 * Every other argument, the workspace size (dcp_mla_workspace_bytes) and the
 * error behaviour are those of dcp_mla_decode_partial.  NaN codes in the
 * cache give unspecified results (never a fault). */
dcp_status dcp_mla_decode_partial_fp8(const dcp_mla_params* p, const void* q, const void* kv_cache,
                                      float kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                                      float* out, float* lse, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* ------------------------------------------------------------------ GQA */

typedef struct {
  int32_t batch;              /* >= 0                                                       */
  int32_t num_q_heads;        /* Hq                                                         */
  int32_t num_kv_heads;       /* Hkv: 1..64; Hq a multiple of Hkv, Hq/Hkv <= 64            */
  int32_t head_dim;           /* D; must be 128                                             */
  int32_t block_size;         /* tokens per cache block; a multiple of 16, 16..1024         */
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t shard_rank;
  int32_t num_shards;
  dcp_layout layout;
  int32_t max_seq_len_hint;
  float softmax_scale;
  int32_t q_len;              /* as in dcp_mla_params                                       */
} dcp_gqa_params;

size_t dcp_gqa_workspace_bytes(const dcp_gqa_params* p);

/* One shard's partial GQA decode attention (sections 4.1 and 5.4 of the DCP
 * post: each KV head is shared by its group of query heads).  Query head h
 * reads KV head g = floor(h * Hkv / Hq); over the shard's local tokens t,
 *     z_t = softmax_scale * <q[b][h], k[t][g]>,  lse = log(sum_t exp(z_t)),
 *     out = sum_t exp(z_t - lse) * v[t][g].
 *  q        bf16 [batch][Hq][D]
 *  k_cache  bf16 [num_blocks][block_size][Hkv][D]
 *  v_cache  bf16 [num_blocks][block_size][Hkv][D]
 *  out      fp32 [batch][Hq][D],  lse fp32 [batch][Hq]
 * Other arguments as for dcp_mla_decode_partial. */
dcp_status dcp_gqa_decode_partial(const dcp_gqa_params* p, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, float* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* -------------------------------------------------------------- combine */

/* LSE-weighted merge of N shard partials into the exact output (section 4.1
 * of the DCP post: the LSE values reweight the partial outputs, which are
 * then summed).  For every (b, h), with M = max_i lse_i:
 *     lse* = M + log(sum_i exp(lse_i - M))
 *     o    = sum_i exp(lse_i - lse*) * o_i
 * If every lse_i is -inf the row is (0, -inf).  The fp32 result is rounded to
 * bf16 (nearest, ties to even) into out_bf16.
 *
 *  partial_out  fp32 [num_shards][batch][num_heads][head_dim_v]
 *  partial_lse  fp32 [num_shards][batch][num_heads]
 *  out_bf16     bf16 [batch][num_heads][head_dim_v] or NULL
 *  out_f32      fp32 [batch][num_heads][head_dim_v] or NULL (result before the cast)
 *  lse_out      fp32 [batch][num_heads] or NULL (merged LSE)
 * At least one of out_bf16 / out_f32 must be non-NULL.  num_shards 1..64,
 * head_dim_v a positive multiple of 4 up to 1024; partial_out and the outputs
 * 16-byte aligned. */
dcp_status dcp_combine(int32_t num_shards, int32_t batch, int32_t num_heads, int32_t head_dim_v,
                       const float* partial_out, const float* partial_lse, void* out_bf16,
                       float* out_f32, float* lse_out, hipStream_t stream);

/* The merge of dcp_combine fused with the epilogue that follows it in an MLA
 * decode layer: each head's value up-projection (latent width head_dim_v to
 * out_dim) and a sigmoid output gate.  The Kimi K3 GB300 decode page describes
 * its DCP step as one kernel that combines the partial results together with
 * the value projection and the gating.  For every (b, h), with o the merged
 * latent row and lse* the merged LSE of dcp_combine:
 *     y[n] = sigmoid(gate[b][h][n]) * sum_k o[k] * w_uv_t[h][n][k]
 * (sigmoid factor 1 when gate is NULL).  o enters the product rounded to bf16;
 * the product accumulates in fp32.
 *
 *  partial_out  fp32 [num_shards][batch][num_heads][head_dim_v]
 *  partial_lse  fp32 [num_shards][batch][num_heads]
 *  w_uv_t       bf16 [num_heads][out_dim][head_dim_v]  (latent index contiguous)
 *  gate         bf16 [batch][num_heads][out_dim] gate logits, or NULL
 *  out_bf16     bf16 [batch][num_heads][out_dim] or NULL
 *  out_f32      fp32 [batch][num_heads][out_dim] or NULL (before the cast)
 *  lse_out      fp32 [batch][num_heads] or NULL (merged LSE)
 * At least one of out_bf16 / out_f32 must be non-NULL.  num_shards 1..64;
 * head_dim_v a positive multiple of 32 up to 1024; out_dim a positive multiple
 * of 16 up to 256; num_heads up to 65535.  partial_out and w_uv_t 16-byte
 * aligned, the rest aligned to their element size.  A row whose partials are
 * all empty gives y = 0 and lse* = -inf. */
dcp_status dcp_combine_vproj_gate(int32_t num_shards, int32_t batch, int32_t num_heads, int32_t head_dim_v,
                                  int32_t out_dim, const float* partial_out, const float* partial_lse,
                                  const void* w_uv_t, const void* gate, void* out_bf16, float* out_f32,
                                  float* lse_out, hipStream_t stream);

/* ------------------------------------------------------------- helpers */

const char* dcp_status_string(dcp_status s);
/* hipError_t of the last DCP_ERR_HIP returned on the calling thread (0 if none). */
int dcp_last_hip_error(void);
int dcp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DCP_H_ */
