"""Benchmark of the DCP decode hot path on one MI355X.

A step is one decode step of one attention layer on the timed shard(s): the
shard-local partial attention (MLA or GQA) over the shard's paged KV slice,
then the LSE-weighted combine of all N shards' partials into the bf16 output.
The other shards' partials are computed once before timing and stay resident
in HBM, as they would after the exchange.  Inputs are synthetic (seeded normal
bf16, shapes of the named workload) and resident in HBM before timing.

Cold cache: the timed shards' KV pools are replicated until the copies exceed
twice the 256 MB Infinity Cache, and step i reads copy i mod n, so each step
streams its KV from HBM as a real decode step does (other layers evict it).

Output: one JSON line (rank 0).  `value` is microseconds per decode step.
The roofline object describes the dominant launch (the shard partial call),
timed live with HIP events on the stream the library launches on.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MALL_BYTES = 256 << 20


CAL_COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def stored_traffic(kind, workload):
    """HBM bytes per partial launch from rocprofv3 FETCH_SIZE + WRITE_SIZE runs
    (profiles/traffic.json), or None if absent or measured on other kernel sources."""
    try:
        from kv_cache_context_amd.rocprof_summary import source_hash
        entry = json.load(open(TRAFFIC_FILE)).get(f"{kind}:{workload}")
    except (OSError, ValueError):
        return None
    if not entry or entry.get("source_hash") != source_hash(kind):
        return None
    return entry.get("bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(case, r, q_len=1):
    """Bytes the method must move for shard r's partial: the shard's KV once
    (a q_len-token step's tokens share it), q, outputs and tables."""
    w = case.w
    ll = case.local_lens(r)
    nblk = -(-ll // w.block_size)
    if w.kind == "mla":
        kv = int(ll.sum()) * w.dk * (1 if case.kv_fp8_scale is not None else 2)
    else:
        kv = int(ll.sum()) * w.kv_heads * w.head_dim * 2 * 2
    q = w.batch * q_len * w.heads * w.dk * 2
    out = w.batch * q_len * w.heads * (w.dv + 1) * 4
    meta = int(nblk.sum()) * 4 + w.batch * 4
    return kv + q + out + meta, kv


def _shard_positions_below(L, lim, n, r, layout):
    """How many of shard r's positions (of a cache of length L split over n
    shards, in the input layout) lie below `lim`."""
    import workloads as W
    pos = W.local_positions(L, n, r, layout)  # a range
    return len(range(pos.start, max(pos.start, min(pos.stop, lim)), pos.step))


def attended(case, r, q_len):
    """(request, token) pairs' attended positions on shard r, summed: token j of
    a q_len-token step attends the positions below L - q_len + 1 + j."""
    w = case.w
    if q_len == 1:
        return int(case.local_lens(r).sum())
    return sum(_shard_positions_below(int(L), int(L) - q_len + 1 + j, w.num_shards, r, w.layout)
               for L in case.seq_lens for j in range(q_len))


def algorithmic_flops(case, r, q_len=1):
    w = case.w
    ll = attended(case, r, q_len)
    if w.kind == "mla":
        return ll * w.heads * 2 * (w.dk + w.dv)
    return ll * w.heads * 4 * w.head_dim


def combine_bytes(w, q_len=1):
    return (w.num_shards * w.batch * w.heads * (w.dv + 1) * 4 + w.batch * w.heads * w.dv * 2) * q_len


VPROJ_DVO = 128  # projected head width of the fused epilogue


def vproj_bytes(w, q_len=1):
    """Fused combine epilogue: partials + LSEs in, projection weights, gate logits, bf16 out."""
    return (q_len * w.num_shards * w.batch * w.heads * (w.dv + 1) * 4 + w.heads * VPROJ_DVO * w.dv * 2
            + 2 * q_len * w.batch * w.heads * VPROJ_DVO * 2)


def cpu_baseline(case, budget_s=10.0, q_len=1, budget_1core_s=5.0):
    """The fp64 oracle on the host cores, on a bounded sample of the same step:
    once with every BLAS thread (`value`, `cores`) and once on one thread
    (`value_1core`), with the host CPU model.  See _oracle_step_us."""
    from threadpoolctl import threadpool_info, threadpool_limits
    us, sample = _oracle_step_us(case, budget_s, q_len)
    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    with threadpool_limits(limits=1):
        us1, sample1 = _oracle_step_us(case, budget_1core_s, q_len)
    return {"value": round(us, 1), "unit": "us/step", "cores": threads, "kind": "oracle", "sample": sample,
            "value_1core": round(us1, 1), "sample_1core": sample1, "cpu": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_step_us(case, budget_s, q_len):
    """The oracle computes the timed shards' partials request by request (its
    own fp64 softmax attention over each shard slice, widened from the same
    bf16 inputs) and the LSE merge of the N partials; requests are taken in
    order, cycling, until about `budget_s` seconds of oracle time are spent,
    and the time is scaled by the fraction of the step's local tokens covered.
    Input widening is not timed.  Returns (us per step, sample description)."""
    import oracle
    w = case.w
    ranks = list(w.ranks)
    total_tokens = sum(attended(case, r, q_len) for r in ranks)
    qs = case.queries(q_len) if q_len > 1 else case.q[:, None]
    done_tokens = 0
    t_spent = 0.0
    reqs = 0
    cache = {}
    b = 0
    while t_spent < budget_s:
        if b not in cache:
            if len(cache) > 4:
                cache.pop(next(iter(cache)))
            L = int(case.seq_lens[b])
            shard_in = []
            for r in range(w.num_shards):
                pos = oracle.shard_positions(L, w.num_shards, r, w.layout)
                if r in ranks:
                    rows = case.rows_at(b, pos)
                    if case.kv_fp8_scale is None:
                        rows = [oracle.widen_bf16(x) for x in rows]
                    shard_in.append((r, pos, rows))
                else:
                    shard_in.append((r, pos, None))
            cache[b] = ([oracle.widen_bf16(qs[b, j]) for j in range(q_len)], shard_in)
        qj, shard_in = cache[b]
        L = int(case.seq_lens[b])
        t0 = time.perf_counter()
        for j in range(q_len):
            lim = oracle.query_limit(L, q_len, j)
            parts = []
            for r, pos, rows in shard_in:
                m = int(np.searchsorted(pos, lim))  # shard positions below token j's limit
                if rows is None:
                    parts.append((np.zeros((w.heads, w.dv)), np.full(w.heads, -np.inf)))
                elif w.kind == "mla" and case.kv_fp8_scale is not None:
                    parts.append(oracle.mla_attention_fp8(qj[j], rows[0][:m], case.kv_fp8_scale, w.scale,
                                                          w.kv_lora_rank))
                elif w.kind == "mla":
                    parts.append(oracle.mla_attention(qj[j], rows[0][:m], w.scale, w.kv_lora_rank))
                else:
                    parts.append(oracle.gqa_attention(qj[j], rows[0][:m], rows[1][:m], w.scale))
                if rows is not None:
                    done_tokens += m
            oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        t_spent += time.perf_counter() - t0
        reqs += 1
        b = (b + 1) % w.batch
    frac = done_tokens / max(total_tokens, 1)
    us_per_step = t_spent / max(frac, 1e-12) * 1e6
    return us_per_step, (f"{reqs} request-steps ({q_len} query token(s) each) of the {w.batch}-request step "
                         f"({frac:.2f} steps' worth of local tokens), fp64 numpy, {t_spent:.1f} s of oracle time, "
                         f"scaled to one step")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c1", help="c0 c1 c2 c3 c4a c4b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--epilogue", choices=("combine", "vproj"), default="combine",
                    help="step epilogue: LSE combine + bf16 cast, or the combine fused with the per-head value "
                         "up-projection (128 wide) and sigmoid gate (MLA workloads)")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default="bf16",
                    help="latent cache format of the MLA workloads: bf16, or fp8 E4M3 with one dequantization "
                         "scale")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per request (multi-token decode step, causal within the step)")
    ap.add_argument("--warm-cache", action="store_true", help="no KV rotation (reported as such)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "one GPU only: the N shards are simulated as slices on one device. "
                                   "Run with --gpus 1."}))
        sys.exit(2)

    import torch
    import workloads as W
    from workloads.device import bf16_tensor, fp8_tensor, int32_tensor
    from kv_cache_context_amd import ops

    w = W.WORKLOADS[args.workload]
    ql = args.q_len
    if not 1 <= ql <= 16:
        print(json.dumps({"error": "--q-len must be in 1..16"}))
        sys.exit(2)
    rows = w.batch * ql
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    fp8 = args.kv_dtype == "fp8"
    if fp8 and w.kind != "mla":
        print(json.dumps({"error": "--kv-dtype fp8 applies to the MLA workloads"}))
        sys.exit(2)
    case = W.Case(w, seed=args.seed, kv_fp8_scale=W.FP8_SCALE if fp8 else None)
    n = w.num_shards
    mb = case.max_blocks_per_seq()
    hint = max(1, case.max_seq_len)
    log(f"[bench] workload {w.name}: {w.description}; seq_lens total {int(case.seq_lens.sum())}")

    po = torch.empty((n, rows, w.heads, w.dv), dtype=torch.float32, device=dev)
    pl = torch.empty((n, rows, w.heads), dtype=torch.float32, device=dev)
    q_d = bf16_tensor(case.queries(ql).reshape(rows, w.heads, w.dk) if ql > 1 else case.q, dev)
    lens_d = int32_tensor(case.seq_lens, dev)
    shards = {}
    t0 = time.time()
    caches = case.shards(range(n), max_blocks=mb)
    for r in range(n):
        sc = caches[r]
        caches[r] = None
        common = dict(block_size=w.block_size, max_blocks_per_seq=mb, num_blocks=sc.num_blocks, shard_rank=r,
                      num_shards=n, layout=w.layout, max_seq_len_hint=hint, softmax_scale=w.scale, q_len=ql)
        ent = {"table": int32_tensor(sc.block_table, dev)}
        if w.kind == "mla":
            ent["p"] = ops.mla_params(batch=w.batch, num_heads=w.heads, **common)
            ent["pools"] = [fp8_tensor(sc.pools[0], dev) if fp8 else bf16_tensor(sc.pools[0], dev)]
            ent["ws"] = ops.mla_workspace(ent["p"], dev)
        else:
            ent["p"] = ops.gqa_params(batch=w.batch, num_q_heads=w.heads, num_kv_heads=w.kv_heads, **common)
            ent["pools"] = [(bf16_tensor(sc.pools[0], dev), bf16_tensor(sc.pools[1], dev))]
            ent["ws"] = ops.gqa_workspace(ent["p"], dev)
        del sc
        shards[r] = ent

    def partial(r, copy):
        e = shards[r]
        pool = e["pools"][copy]
        st = torch.cuda.current_stream()
        if fp8:
            ops.dcp_mla_decode_partial_fp8(e["p"], q_d, pool, case.kv_fp8_scale, e["table"], lens_d, po[r], pl[r],
                                           e["ws"], st)
        elif w.kind == "mla":
            ops.dcp_mla_decode_partial(e["p"], q_d, pool, e["table"], lens_d, po[r], pl[r], e["ws"], st)
        else:
            ops.dcp_gqa_decode_partial(e["p"], q_d, pool[0], pool[1], e["table"], lens_d, po[r], pl[r], e["ws"],
                                       st)

    for r in range(n):  # every shard's partial once: the resident inputs of the combine
        partial(r, 0)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in {time.time() - t0:.1f} s")

    timed = list(w.ranks)
    kv_bytes_timed = sum(algorithmic_bytes(case, r)[1] for r in timed)
    copies = 1
    if not args.warm_cache and kv_bytes_timed > 0:
        copies = min(64, max(1, math.ceil(2 * MALL_BYTES / kv_bytes_timed)))
    for r in timed:
        base = shards[r]["pools"][0]
        for _ in range(copies - 1):
            if w.kind == "mla":
                shards[r]["pools"].append(base.clone())
            else:
                shards[r]["pools"].append((base[0].clone(), base[1].clone()))
    torch.cuda.synchronize()
    log(f"[bench] {copies} rotating copies of the timed KV ({kv_bytes_timed / 1e6:.1f} MB each)")

    out_bf = torch.empty((rows, w.heads, w.dv), dtype=torch.bfloat16, device=dev)

    def do_partials(i):
        for r in timed:
            partial(r, i % copies)

    if args.epilogue == "vproj":
        if w.kind != "mla":
            print(json.dumps({"error": "--epilogue vproj applies to the MLA workloads"}))
            sys.exit(2)
        w_bits, g_bits = W.random_vproj(rows, w.heads, VPROJ_DVO, w.dv, seed=args.seed)
        w_uv_d, gate_d = bf16_tensor(w_bits, dev), bf16_tensor(g_bits, dev)
        out_bf = torch.empty((rows, w.heads, VPROJ_DVO), dtype=torch.bfloat16, device=dev)

    def do_combine(i):
        if args.epilogue == "vproj":
            ops.dcp_combine_vproj_gate(po, pl, w_uv_d, gate_d, out_bf, None, None, torch.cuda.current_stream())
        else:
            ops.dcp_combine(po, pl, out_bf, None, None, torch.cuda.current_stream())

    def step(i):
        do_partials(i)
        do_combine(i)

    # Each timed region is K steps captured in one HIP graph and replayed once, so
    # the device timeline has no host launch gaps; HIP events bracket the replay
    # on the stream the kernels run on.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(args.steps):
                fn(i)
        return g

    replay_ms = {}

    def timed_replay(g, reps=5, name=None):
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(side):
                e0.record(side)
                g.replay()
                e1.record(side)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        if name:
            replay_ms[name] = sorted(times)
        return sorted(times)[len(times) // 2]  # median replay

    g_step = capture(step)
    g_part = capture(do_partials)
    g_comb = capture(do_combine)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g_step.replay()  # warm the graph once
    torch.cuda.synchronize()
    total_ms = timed_replay(g_step, name="step")
    ms_per_step = total_ms / args.steps
    part_ms = timed_replay(g_part)
    comb_ms = timed_replay(g_comb)
    part_mean = part_ms / args.steps * 1e3
    comb_mean = comb_ms / args.steps * 1e3

    alg_partial = sum(algorithmic_bytes(case, r, ql)[0] for r in timed)
    alg_comb = vproj_bytes(w, ql) if args.epilogue == "vproj" else combine_bytes(w, ql)
    flops = sum(algorithmic_flops(case, r, ql) for r in timed)
    achieved = alg_partial / (part_mean * 1e-6) / 1e9
    step_gbs = (alg_partial + alg_comb) / (ms_per_step * 1e-3) / 1e9

    res = {
        "metric": "\u00b5s/decode step + achieved HBM GB/s (% peak), shard-local MLA attn + combine",
        "value": round(ms_per_step * 1e3, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "kind": w.kind, "batch": w.batch,
                   "heads": w.heads, "q_len": ql, "kv_dtype": args.kv_dtype, "num_shards": n, "timed_shards": timed, "block_size": w.block_size,
                   "local_tokens": int(sum(case.local_lens(r).sum() for r in timed)),
                   "kv_copies_rotated": copies},
        "step_hbm_gbps": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "partial_us": round(part_mean, 3),
        "combine_us": round(comb_mean, 3),
        "epilogue": "dcp_combine_vproj_gate" if args.epilogue == "vproj" else "dcp_combine",
        "epilogue_gbps": round(alg_comb / (comb_mean * 1e-6) / 1e9, 1),
        "timing": "K steps captured in one HIP graph; HIP events around each of 5 replays, median replay",
        "step_us_replays": [round(t / args.steps * 1e3, 3) for t in replay_ms["step"]],
        "mfma_tflops": round(flops / (part_mean * 1e-6) / 1e12, 2),
        "mfma_frac": round(flops / (part_mean * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "hbm", "kernel": f"dcp_{w.kind}_decode_partial" + ("_fp8" if fp8 else ""),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": alg_partial},
    }
    if args.calibration_copy:
        a = torch.empty(CAL_COPY_BYTES, dtype=torch.uint8, device=dev)
        b2 = torch.empty_like(a)
        b2.copy_(a)
        torch.cuda.synchronize()
        del a, b2
    kind = ("mla8" if fp8 else "mla") if w.kind == "mla" else "gqa"
    res["roofline"]["traffic"] = stored_traffic(kind, w.name) if ql == 1 else None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        res["cpu_baseline"] = cpu_baseline(case, q_len=ql)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
