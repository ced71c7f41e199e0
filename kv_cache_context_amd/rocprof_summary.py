"""Summaries of rocprofv3 output for the DCP kernels.

    python -m kv_cache_context_amd.rocprof_summary stats <kernel_stats.csv>
    python -m kv_cache_context_amd.rocprof_summary traffic <fetch counter_collection.csv> \
        <write counter_collection.csv> <kernel name substring> <calibration copy bytes>
    python -m kv_cache_context_amd.rocprof_summary report <prof dir> <name> <mla|gqa> \
        [<bench arguments> <summary file stem>]

`report` writes the markdown summary of one workload's profiling runs (kernel
trace statistics, the bench line of the traced run, and the counter traffic
when the FETCH_SIZE / WRITE_SIZE runs exist) and prints the traffic entry for
profiles/traffic.json.  The directory layout is the one of the commands quoted
in the summary: <dir>/<name>/kt_kernel_stats.csv, <dir>/<name>_kt.log,
<dir>/<name>_FETCH_SIZE/p_counter_collection.csv, <dir>/<name>_WRITE_SIZE/....
<name> is the workload unless bench arguments other than --workload <name>
were used; the summary goes to profiles/<kind>_partial_<name>.md unless a
file stem is given.

`traffic` converts FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into bytes per
launch of the named kernel, each scaled by the ratio between the known size of
a plain device-to-device copy run in the same process (bench.py
--calibration-copy) and what the same counter reports for that copy kernel.
`source_hash()` fingerprints the kernel sources so a stored traffic figure is
only used while the kernel it was measured on is unchanged.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {
    "mla": ["csrc/mla_partial.hip", "csrc/dcp_device.hpp", "csrc/dcp_split.hpp", "csrc/dcp_internal.hpp", "build.py"],
    "mla8": ["csrc/mla_partial.hip", "csrc/dcp_device.hpp", "csrc/dcp_split.hpp", "csrc/dcp_internal.hpp", "build.py"],
    "gqa": ["csrc/gqa_partial.hip", "csrc/gqa_layout.hpp", "csrc/dcp_device.hpp", "csrc/dcp_split.hpp",
            "csrc/dcp_internal.hpp", "build.py"],
    "combine": ["csrc/combine.hip", "csrc/dcp_device.hpp", "csrc/dcp_internal.hpp", "build.py"],
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
# kernel-name substring of each kind's partial kernel in traces
PARTIAL_KERNEL = {"mla": "mla::partial_kernel<false>", "mla8": "mla::partial_kernel<true>",
                  "gqa": "gqa::partial_kernel"}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['Name'][:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(out)


def _per_dispatch(path: str, counter: str):
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int) -> dict:
    res = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = _per_dispatch(path, name)
        copy = [v for k, vs in vals.items() if k.startswith(COPY_KERNEL) for v in vs]
        kern = [v for k, vs in vals.items() if kernel in k for v in vs]
        if not copy or not kern:
            raise SystemExit(f"missing dispatches for {name}: copy {len(copy)} kernel {len(kern)}")
        copy_kib = max(copy)  # the calibration copy is the largest copy in the run
        scale = copy_bytes / (copy_kib * 1024.0)
        avg_kib = sum(kern) / len(kern)
        res[name] = {"kib_per_dispatch": round(avg_kib, 1), "copy_kib": copy_kib, "scale": round(scale, 4),
                     "bytes_per_launch": int(avg_kib * 1024 * scale), "dispatches": len(kern)}
    res["bytes_per_launch"] = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    return res


CAL_COPY_BYTES = 1 << 30


def report(prof: str, wl: str, kind: str, bench_args: str | None = None) -> tuple[str, dict | None]:
    """bench_args: the bench arguments of the runs (default --workload <wl>); the kernel-trace run adds
    --no-cpu-baseline except for c1, the counter runs their own short-run flags."""
    base = bench_args if bench_args is not None else f"--workload {wl}"
    # the default workload's trace is of the default command itself (CPU
    # baseline leg included); c1 keeps its CPU baseline too
    if base == "--workload c4":
        kt_args = ""
    else:
        kt_args = base + ("" if base == "--workload c1" else " --no-cpu-baseline")
    kt_cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {prof}/{wl} -o kt -- "
              f"python -u bench.py {kt_args}").rstrip()
    pmc_cmd = (f"rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d {prof}/{wl}_<counter> -o p -- "
               f"python -u bench.py {base} --steps 5 --warmup 1 --no-cpu-baseline --calibration-copy")
    bench = None
    logp = os.path.join(prof, f"{wl}_kt.log")
    if os.path.exists(logp):
        for line in open(logp):
            if line.startswith("{"):
                bench = json.loads(line)
    lines = [f"# {kind} partial + epilogue, {wl}", ""]
    if bench:
        lines += [f"Workload: {bench['config'].get('description', '')}", ""]
    lines += ["Kernel trace (each step: the timed shards' partial calls, i.e. partial_kernel then its split",
              "reduce, then one combine; warmup, capture and replay dispatches included):", "",
              "```", kt_cmd, "```", "", stats(os.path.join(prof, wl, "kt_kernel_stats.csv")), ""]
    if bench:
        keep = {k: bench[k] for k in ("value", "unit", "partial_us", "combine_us", "step_hbm_gbps", "mfma_tflops")}
        keep["roofline"] = {k: bench["roofline"][k] for k in ("achieved", "peak", "frac", "bytes_per_launch")}
        keep["config"] = {k: bench["config"][k] for k in ("workload", "q_len", "kv_dtype") if k in bench["config"]}
        if "parts" in bench and len(bench["parts"]) > 1:
            keep["parts"] = [{k: p[k] for k in ("workload", "partial_launches", "partial_us", "partial_frac")}
                             for p in bench["parts"]]
        if "cpu_baseline" in bench:
            keep["cpu_baseline"] = bench["cpu_baseline"]
        keep["epilogue"] = bench.get("epilogue")
        lines += ["bench line of the traced run (HIP-event timing of graph replays; `partial_us` is one",
                  "partial call = partial_kernel + reduce_kernel).  Kernel tracing adds a few us to every",
                  "dispatch, so the untraced bench is the timing reference; the kernel averages above are",
                  "the device durations:", "", "```", json.dumps(keep), "```", ""]
    entry = None
    fetch = os.path.join(prof, f"{wl}_FETCH_SIZE", "p_counter_collection.csv")
    write = os.path.join(prof, f"{wl}_WRITE_SIZE", "p_counter_collection.csv")
    if os.path.exists(fetch) and os.path.exists(write):
        t = traffic(fetch, write, PARTIAL_KERNEL[kind], CAL_COPY_BYTES)
        lines += ["HBM traffic of partial_kernel from two counter runs (KiB per dispatch, scaled by the",
                  "counter's reading for a 1 GiB device copy in the same process):", "", "```", pmc_cmd, "```", "",
                  "| counter | KiB/dispatch | copy reads KiB | scale | bytes/launch |", "|---|---|---|---|---|"]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            r = t[c]
            lines.append(f"| {c} | {r['kib_per_dispatch']} | {r['copy_kib']} | {r['scale']} | {r['bytes_per_launch']} |")
        lines += ["", f"Total: {t['bytes_per_launch']} bytes per launch."]
        entry = {"bytes_per_launch": t["bytes_per_launch"], "fetch": t["FETCH_SIZE"]["bytes_per_launch"],
                 "write": t["WRITE_SIZE"]["bytes_per_launch"], "source_hash": source_hash(kind)}
    return "\n".join(lines) + "\n", entry


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5])), indent=1))
    elif sys.argv[1] == "hash":
        print(source_hash(sys.argv[2]))
    elif sys.argv[1] == "report":
        text, entry = report(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5] if len(sys.argv) > 5 else None)
        stem = sys.argv[6] if len(sys.argv) > 6 else f"{sys.argv[4]}_partial_{sys.argv[3]}"
        out = os.path.join(os.path.dirname(PKG), "profiles", f"{stem}.md")
        with open(out, "w") as f:
            f.write(text)
        print(json.dumps({f"{sys.argv[4]}:{sys.argv[3]}": entry}))
