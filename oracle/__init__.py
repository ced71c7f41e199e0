"""fp64 CPU oracle for decode-context-parallel (DCP) attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``kv_cache_context_amd``) never imports it, and it never imports the
product path.  It shares no code with the HIP kernels; the only thing both
sides read is the seeded input generator in ``workloads``.

Every function follows a stated definition:

* ``softmax_attention`` — plain softmax attention of one decode query per head
  against a set of keys/values, returning the normalized output and the
  natural-log log-sum-exp of the scaled scores.  This is what each rank
  computes over its local slice in the "Compute" step of the DCP process
  (vLLM blog post on Decode Context Parallelism, section 4.1).
* ``mla_attention`` — the MLA form in absorbed latent space: keys are the
  full latent row [c_kv | k_rope] (576 wide), values are c_kv (512 wide); one
  latent row serves every query head (same post, section 5.3 "MLA Backend").
* ``gqa_attention`` — each KV head serves a consecutive group of query heads
  (section 5.4 "GQA Backend").
* ``decode_e4m3fn`` / ``mla_attention_fp8`` — the fp8 KV cache (the Kimi K3
  optimizations page serves with an fp8 cache): OCP E4M3 codes decoded exactly,
  times one per-cache dequantization scale, then ``mla_attention``.
* ``shard_positions`` — which global token positions a shard holds
  (section 4; round-robin and contiguous layouts).
* ``query_limit`` / ``query_positions`` — the causal prefix of each query
  token of a multi-token decode step (speculative verification, section 6) and
  the part of it a shard holds.
* ``merge`` — the LSE-weighted merge of N partial results into the exact
  output (section 4.1, the AllGather + ReduceScatter step, which reweights
  partial outputs by their LSE values).
* ``combine_vproj_gate`` — the merge followed by each head's value
  up-projection and a sigmoid output gate, the epilogue fused into the DCP
  combine on the Kimi K3 GB300 decode page.
* ``bf16_rne`` — round-to-nearest-even cast of fp32 to bf16 (the output cast).

Parity of every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` against closed forms, library routines and
invariants; see the notes there.
"""
from .attention import (  # noqa: F401
    widen_bf16,
    softmax_attention,
    mla_attention,
    gqa_attention,
    decode_e4m3fn,
    mla_attention_fp8,
    shard_positions,
    query_limit,
    query_positions,
    mla_shard_partial,
    gqa_shard_partial,
    merge,
    combine_vproj_gate,
    bf16_rne,
    bf16_rne_bits,
)
