"""Benchmark of the DCP decode hot path on one MI355X.

A step is one decode step of one attention layer on the timed shard(s): the
shard-local partial attention (MLA or GQA) over the shard's paged KV slice,
then the LSE-weighted combine of all N shards' partials into the bf16 output.
The other shards' partials are computed once before timing and stay resident
in HBM, as they would after the exchange.  Inputs are synthetic (seeded normal
bf16, shapes of the named workload) and resident in HBM before timing.

The default workload is c4, the long-context configuration: one step is the
1M-token request with all 8 shards processed (8 partial calls + the combine,
part c4a) followed by the 128-request batch at 64K context on shard 1 of 8
(one partial call + the combine, part c4b).  Each single configuration
(c0 .. c4b, and c3kv1: the GQA example with one KV head per rank) can be
selected with --workload.

Cold cache: before every timed graph replay an untimed pass reads and writes
a buffer of twice the 256 MB Infinity Cache, so nothing a replay reads is
left in the caches by the previous one; inside a replay, step i reads KV copy
i mod n, with n copies of the timed pools replicated until they exceed twice
the Infinity Cache.  So every step streams its KV from HBM, whatever the step
count, as a real decode step does (other layers evict it).

Output: one JSON line (rank 0).  `value` is microseconds per decode step.
The roofline object describes the dominant entry point (the shard partial
call), timed live with HIP events on the stream the library launches on.
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
METRIC = "µs/decode step + achieved HBM GB/s (% peak), shard-local MLA attn + combine"

# workloads whose step is several configurations run back to back
COMPOSITE = {
    "c4": ("c4a", "c4b"),
}
COMPOSITE_DESCRIPTION = {
    "c4": "MLA long context: b=1 at L=1M with all 8 shards (8 partial calls + combine over 8), then b=128 at "
          "L=64K on shard 1 of 8 (one partial call + combine over 8); 64 heads, latent 512+64 bf16, B=64",
}

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


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_inputs(case, q_len, max_requests=4):
    """The widened inputs of the first few requests of the step (at most
    `max_requests`), for the oracle: per request its query tokens and, per
    shard, the shard's positions and (for the timed shards) its rows.  Not
    timed."""
    import oracle
    w = case.w
    ranks = list(w.ranks)
    qs = case.queries(q_len) if q_len > 1 else case.q[:, None]
    fp8 = case.kv_fp8_scale is not None
    reqs = []
    for b in range(min(w.batch, max_requests)):
        L = int(case.seq_lens[b])
        log(f"[bench] {w.name}: oracle inputs of request {b} (L={L})")
        if len(ranks) * 2 >= w.num_shards:
            # most of the request is needed: generate it once, in global order
            full = case.kv_logical(b)
            take = (lambda pos, full=full: [full[pos]]) if w.kind == "mla" else \
                (lambda pos, full=full: [x[pos] for x in full])
        else:
            take = lambda pos, b=b: case.rows_at(b, pos)  # noqa: E731
        shard_in = []
        for r in range(w.num_shards):
            pos = oracle.shard_positions(L, w.num_shards, r, w.layout)
            rows = None
            if r in ranks:
                rows = take(pos)
                if not fp8:
                    rows = [oracle.widen_bf16(x) for x in rows]
            shard_in.append((r, pos, rows))
        reqs.append((b, L, [oracle.widen_bf16(qs[b, j]) for j in range(q_len)], shard_in))
    return reqs


def _oracle_step_us(case, reqs, budget_s, q_len):
    """The oracle computes the timed shards' partials request by request (its
    own fp64 softmax attention over each shard slice, widened from the same
    bf16 inputs) and the LSE merge of the N partials, cycling over the
    prepared requests (`_oracle_inputs`) until about `budget_s` seconds of
    oracle time are spent (at least one request); the time is scaled by the
    fraction of the step's attended local tokens covered.  Returns (us per
    step, sample description)."""
    import oracle
    w = case.w
    total_tokens = sum(attended(case, r, q_len) for r in w.ranks)
    fp8 = case.kv_fp8_scale is not None
    done_tokens = 0
    t_spent = 0.0
    n = 0
    while t_spent < budget_s or n == 0:
        b, L, qj, shard_in = reqs[n % len(reqs)]
        t0 = time.perf_counter()
        for j in range(q_len):
            lim = oracle.query_limit(L, q_len, j)
            parts = []
            for r, pos, rows in shard_in:
                m = int(np.searchsorted(pos, lim))  # shard positions below token j's limit
                if rows is None:
                    parts.append((np.zeros((w.heads, w.dv)), np.full(w.heads, -np.inf)))
                elif w.kind == "mla" and fp8:
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
        n += 1
    frac = done_tokens / max(total_tokens, 1)
    us_per_step = t_spent / max(frac, 1e-12) * 1e6
    return us_per_step, (f"{w.name}: {n} request-steps ({q_len} query token(s) each) cycling over requests "
                         f"0..{len(reqs) - 1} of the {w.batch}-request step ({frac:.3f} steps' worth of attended "
                         f"local tokens), fp64 numpy, {t_spent:.1f} s of oracle time, scaled to one step")


def cpu_baseline(cases, budget_s=10.0, q_len=1, budget_1core_s=5.0):
    """The fp64 oracle on the host cores, on a bounded sample of the same step
    (for a composite step, the sum of its parts' estimates, the budget split
    evenly between them): once with every BLAS thread (`value`, `cores`) and
    once on one thread (`value_1core`), with the host CPU model.  See
    _oracle_step_us."""
    from threadpoolctl import threadpool_info, threadpool_limits
    n = len(cases)
    prepared = [_oracle_inputs(c, q_len) for c in cases]
    us, samples = 0.0, []
    for c, reqs in zip(cases, prepared):
        u, s = _oracle_step_us(c, reqs, budget_s / n, q_len)
        log(f"[bench] oracle {c.w.name}: {u:.0f} us/step on all cores")
        us += u
        samples.append(s)
    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    us1, samples1 = 0.0, []
    with threadpool_limits(limits=1):
        for c, reqs in zip(cases, prepared):
            u, s = _oracle_step_us(c, reqs, budget_1core_s / n, q_len)
            log(f"[bench] oracle {c.w.name}: {u:.0f} us/step on one core")
            us1 += u
            samples1.append(s)
    return {"value": round(us, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": "; ".join(samples), "value_1core": round(us1, 1), "sample_1core": "; ".join(samples1),
            "cpu": _cpu_model()}


class Part:
    """One configuration of a step: its inputs resident on the device, the
    timed shards' partial calls and the epilogue over all N partials."""

    def __init__(self, name, args, dev):
        import torch
        import workloads as W
        from workloads.device import bf16_tensor, fp8_tensor, int32_tensor
        from kv_cache_context_amd import ops

        self.ops = ops
        w = W.WORKLOADS[name]
        self.w = w
        self.fp8 = args.kv_dtype == "fp8"
        if self.fp8 and w.kind != "mla":
            raise SystemExit(json.dumps({"error": "--kv-dtype fp8 applies to the MLA workloads"}))
        if args.epilogue == "vproj" and w.kind != "mla":
            raise SystemExit(json.dumps({"error": "--epilogue vproj applies to the MLA workloads"}))
        self.ql = ql = args.q_len
        self.vproj = args.epilogue == "vproj"
        case = W.Case(w, seed=args.seed, kv_fp8_scale=W.FP8_SCALE if self.fp8 else None)
        self.case = case
        n = w.num_shards
        rows = w.batch * ql
        mb = case.max_blocks_per_seq()
        hint = max(1, case.max_seq_len)
        log(f"[bench] workload {w.name}: {w.description}; seq_lens total {int(case.seq_lens.sum())}")
        t0 = time.time()
        self.po = torch.empty((n, rows, w.heads, w.dv), dtype=torch.float32, device=dev)
        self.pl = torch.empty((n, rows, w.heads), dtype=torch.float32, device=dev)
        self.q_d = bf16_tensor(case.queries(ql).reshape(rows, w.heads, w.dk) if ql > 1 else case.q, dev)
        self.lens_d = int32_tensor(case.seq_lens, dev)
        self.shards = {}
        caches = case.shards(range(n), max_blocks=mb)
        log(f"[bench] {w.name}: inputs generated in {time.time() - t0:.1f} s")
        for r in range(n):
            sc = caches[r]
            caches[r] = None
            common = dict(block_size=w.block_size, max_blocks_per_seq=mb, num_blocks=sc.num_blocks, shard_rank=r,
                          num_shards=n, layout=w.layout, max_seq_len_hint=hint, softmax_scale=w.scale, q_len=ql)
            ent = {"table": int32_tensor(sc.block_table, dev)}
            if w.kind == "mla":
                ent["p"] = ops.mla_params(batch=w.batch, num_heads=w.heads, **common)
                ent["pools"] = [fp8_tensor(sc.pools[0], dev) if self.fp8 else bf16_tensor(sc.pools[0], dev)]
                ent["ws"] = ops.mla_workspace(ent["p"], dev)
            else:
                ent["p"] = ops.gqa_params(batch=w.batch, num_q_heads=w.heads, num_kv_heads=w.kv_heads, **common)
                ent["pools"] = [(bf16_tensor(sc.pools[0], dev), bf16_tensor(sc.pools[1], dev))]
                ent["ws"] = ops.gqa_workspace(ent["p"], dev)
            del sc
            self.shards[r] = ent
        for r in range(n):  # every shard's partial once: the resident inputs of the combine
            self.partial(r, 0)
        torch.cuda.synchronize()
        log(f"[bench] {w.name}: inputs resident in {time.time() - t0:.1f} s")

        self.timed = list(w.ranks)
        self.kv_bytes_timed = sum(algorithmic_bytes(case, r)[1] for r in self.timed)
        self.copies = 1
        if not args.warm_cache and self.kv_bytes_timed > 0:
            self.copies = min(64, max(1, math.ceil(2 * MALL_BYTES / self.kv_bytes_timed)))
        for r in self.timed:
            base = self.shards[r]["pools"][0]
            for _ in range(self.copies - 1):
                if w.kind == "mla":
                    self.shards[r]["pools"].append(base.clone())
                else:
                    self.shards[r]["pools"].append((base[0].clone(), base[1].clone()))
        torch.cuda.synchronize()
        log(f"[bench] {w.name}: {self.copies} rotating copies of the timed KV ({self.kv_bytes_timed / 1e6:.1f} MB "
            f"each)")

        if self.vproj:
            w_bits, g_bits = W.random_vproj(rows, w.heads, VPROJ_DVO, w.dv, seed=args.seed)
            self.w_uv_d, self.gate_d = bf16_tensor(w_bits, dev), bf16_tensor(g_bits, dev)
            self.out_bf = torch.empty((rows, w.heads, VPROJ_DVO), dtype=torch.bfloat16, device=dev)
        else:
            self.out_bf = torch.empty((rows, w.heads, w.dv), dtype=torch.bfloat16, device=dev)

        self.alg_partial = sum(algorithmic_bytes(case, r, ql)[0] for r in self.timed)
        self.alg_comb = vproj_bytes(w, ql) if self.vproj else combine_bytes(w, ql)
        self.flops = sum(algorithmic_flops(case, r, ql) for r in self.timed)
        self.local_tokens = int(sum(case.local_lens(r).sum() for r in self.timed))

    def partial(self, r, copy):
        import torch
        ops = self.ops
        e = self.shards[r]
        pool = e["pools"][copy]
        st = torch.cuda.current_stream()
        if self.fp8:
            ops.dcp_mla_decode_partial_fp8(e["p"], self.q_d, pool, self.case.kv_fp8_scale, e["table"], self.lens_d,
                                           self.po[r], self.pl[r], e["ws"], st)
        elif self.w.kind == "mla":
            ops.dcp_mla_decode_partial(e["p"], self.q_d, pool, e["table"], self.lens_d, self.po[r], self.pl[r],
                                       e["ws"], st)
        else:
            ops.dcp_gqa_decode_partial(e["p"], self.q_d, pool[0], pool[1], e["table"], self.lens_d, self.po[r],
                                       self.pl[r], e["ws"], st)

    def partials(self, i):
        for r in self.timed:
            self.partial(r, i % self.copies)

    def combine(self, i=0):
        import torch
        st = torch.cuda.current_stream()
        if self.vproj:
            self.ops.dcp_combine_vproj_gate(self.po, self.pl, self.w_uv_d, self.gate_d, self.out_bf, None, None,
                                            st)
        else:
            self.ops.dcp_combine(self.po, self.pl, self.out_bf, None, None, st)

    def step(self, i):
        self.partials(i)
        self.combine(i)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4",
                    help="c4 (default: c4a then c4b in one step), or one of c0 c1 c2 c3 c4a c4b")
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
    ap.add_argument("--warm-cache", action="store_true", help="no KV rotation or eviction (reported as such)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "one GPU only: the N shards are simulated as slices on one device. "
                                   "Run with --gpus 1."}))
        sys.exit(2)
    if not 1 <= args.q_len <= 16:
        print(json.dumps({"error": "--q-len must be in 1..16"}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print(json.dumps({"error": "--steps must be >= 1 and --warmup >= 0"}))
        sys.exit(2)

    import torch
    import workloads as W

    names = COMPOSITE.get(args.workload, (args.workload,))
    for nm in names:
        if nm not in W.WORKLOADS:
            print(json.dumps({"error": f"unknown workload {nm}"}))
            sys.exit(2)
    dev = torch.device("cuda:0")
    parts = [Part(nm, args, dev) for nm in names]

    def step(i):
        for p in parts:
            p.step(i)

    # Eviction between timed replays: read and write twice the Infinity Cache.
    evict = torch.zeros((2 * MALL_BYTES) // 4, dtype=torch.int32, device=dev)

    # Each timed region is K steps captured in one HIP graph and replayed once, so
    # the device timeline has no host launch gaps; HIP events bracket the replay
    # on the stream the kernels run on.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    log("[bench] warmup done")

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(args.steps):
                fn(i)
        return g

    def timed_replay(g, reps=5):
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(side):
                if not args.warm_cache:
                    evict.add_(1)  # untimed: before e0 on the same stream
                e0.record(side)
                g.replay()
                e1.record(side)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)

    g_step = capture(step)
    g_parts = [(capture(p.partials), capture(p.combine)) for p in parts]
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g_step.replay()  # warm the graph once
    torch.cuda.synchronize()
    step_times = timed_replay(g_step)
    ms_per_step = step_times[len(step_times) // 2] / args.steps  # median replay
    part_res = []
    for p, (gp, gc) in zip(parts, g_parts):
        tp = timed_replay(gp)
        tc = timed_replay(gc)
        part_res.append((tp[len(tp) // 2] / args.steps * 1e3, tc[len(tc) // 2] / args.steps * 1e3))
    log("[bench] timing done")

    ql = args.q_len
    fp8 = args.kv_dtype == "fp8"
    alg_partial = sum(p.alg_partial for p in parts)
    alg_comb = sum(p.alg_comb for p in parts)
    flops = sum(p.flops for p in parts)
    part_us = sum(pu for pu, _ in part_res)
    comb_us = sum(cu for _, cu in part_res)
    launches = sum(len(p.timed) for p in parts)
    achieved = alg_partial / (part_us * 1e-6) / 1e9
    step_gbs = (alg_partial + alg_comb) / (ms_per_step * 1e-3) / 1e9
    kinds = {p.w.kind for p in parts}
    kind = kinds.pop() if len(kinds) == 1 else "mixed"
    tkind = ("mla8" if fp8 else "mla") if kind == "mla" else "gqa"

    traffic = None
    if ql == 1:
        tr = [stored_traffic(tkind, p.w.name) for p in parts]
        if all(t is not None for t in tr):
            traffic = int(sum(t * len(p.timed) for t, p in zip(tr, parts)) / launches)

    parts_out = []
    for p, (pu, cu) in zip(parts, part_res):
        a = p.alg_partial / (pu * 1e-6) / 1e9
        parts_out.append({
            "workload": p.w.name, "description": p.w.description, "timed_shards": p.timed,
            "partial_launches": len(p.timed), "local_tokens": p.local_tokens, "kv_copies_rotated": p.copies,
            "partial_us": round(pu, 3), "combine_us": round(cu, 3),
            "partial_bytes": p.alg_partial, "partial_gbps": round(a, 1), "partial_frac": round(a / HBM_PEAK_GBS, 4),
            "epilogue_bytes": p.alg_comb, "epilogue_gbps": round(p.alg_comb / (cu * 1e-6) / 1e9, 1),
            "mfma_tflops": round(p.flops / (pu * 1e-6) / 1e12, 2)})

    w0 = parts[0].w
    desc = COMPOSITE_DESCRIPTION.get(args.workload, w0.description)
    res = {
        "metric": METRIC,
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
        "config": {"workload": args.workload, "description": desc, "kind": kind,
                   "parts": [p.w.name for p in parts], "batch": [p.w.batch for p in parts],
                   "heads": w0.heads, "q_len": ql, "kv_dtype": args.kv_dtype,
                   "num_shards": [p.w.num_shards for p in parts],
                   "timed_shards": [p.timed for p in parts], "block_size": [p.w.block_size for p in parts],
                   "local_tokens": sum(p.local_tokens for p in parts),
                   "kv_copies_rotated": [p.copies for p in parts],
                   "cache": "warm" if args.warm_cache else "cold (2x Infinity Cache evicted before each replay)"},
        "step_hbm_gbps": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "partial_us": round(part_us, 3),
        "combine_us": round(comb_us, 3),
        "epilogue": "dcp_combine_vproj_gate" if args.epilogue == "vproj" else "dcp_combine",
        "epilogue_gbps": round(alg_comb / (comb_us * 1e-6) / 1e9, 1),
        "timing": "K steps captured in one HIP graph; HIP events around each of 5 replays, median replay",
        "step_us_replays": [round(t / args.steps * 1e3, 3) for t in step_times],
        "mfma_tflops": round(flops / (part_us * 1e-6) / 1e12, 2),
        "mfma_frac": round(flops / (part_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "hbm", "kernel": f"dcp_{kind}_decode_partial" + ("_fp8" if fp8 else ""),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "launches_per_step": launches, "bytes_per_launch": int(alg_partial / launches),
                     "note": "achieved = algorithmic bytes of the step's partial calls / their summed duration; "
                             "bytes_per_launch and traffic are averages over those calls"},
        "parts": parts_out,
    }
    if args.calibration_copy:
        a = torch.empty(CAL_COPY_BYTES, dtype=torch.uint8, device=dev)
        b2 = torch.empty_like(a)
        b2.copy_(a)
        torch.cuda.synchronize()
        del a, b2
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        res["cpu_baseline"] = cpu_baseline([p.case for p in parts], q_len=ql)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
