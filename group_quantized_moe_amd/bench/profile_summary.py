"""Summaries of rocprofv3 runs of bench.py for profiles/ (decode workloads).

  trace: a `rocprofv3 --kernel-trace` database of one decode workload ->
         profiles/<workload>_kernels.json and _kernel_trace.md (per-kernel
         median / p10 / p90 / mean durations, achieved rate on the kernel's
         algorithmic bytes, the GPU span of one call);
  pmc:   the counter_collection.csv files of two `rocprofv3 --pmc` passes
         (FETCH_SIZE, then WRITE_SIZE) over the workload and over
         `bench.py --workload copy` (a 256 MiB device copy) ->
         profiles/<workload>_pmc.json: each counter scaled by what it reads
         for the copy of known size, HBM bytes per call against the
         algorithmic bytes.

Both record the hash of the kernel sources (bench.kernel_source_hash), so
that bench.py reports the figures only while the kernels are the ones that
were profiled.  Run from the repository root:

  python -m group_quantized_moe_amd.bench.profile_summary trace decode_q4 <run_results.db>
  python -m group_quantized_moe_amd.bench.profile_summary pmc decode_q4 <fetch.csv> <write.csv> \\
      <copy_fetch.csv> <copy_write.csv>
  python -m group_quantized_moe_amd.bench.profile_summary render decode_q4
"""
import csv
import json
import os
import re
import sqlite3
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import bench       # noqa: E402
import workloads   # noqa: E402

PEAK = bench.PEAK_HBM_GBS
COPY_BYTES = 256 << 20

# workload -> (spec, experts used, title)
DECODE = {
    "decode_q4": (workloads.Q4_GROUP8, 8, "Q4 8-expert decode group (d_model 4096, d_ff 1536, group 64, f32 scales)"),
    "decode_q2": (workloads.Q2_GROUP8, 8, "Q2 8-expert decode group (d_model 4096, d_ff 1536, group 64, f32 scales)"),
    "decode_q4_s16": (workloads.Q4_GROUP8_S16, 8,
                      "Q4 8-expert decode group with 2-byte scales (d_model 4096, d_ff 1536, group 64)"),
    "decode_q2_s16": (workloads.Q2_GROUP8_S16, 8,
                      "Q2 8-expert decode group with 2-byte scales (d_model 4096, d_ff 1536, group 64)"),
    "decode_q4_e1": (workloads.Q4_GROUP8, 1, "one expert of the Q4 group (d_model 4096, d_ff 1536, group 64)"),
    "tiny": (workloads.TINY, 1, "tiny Q4 expert 256 / 512 (latency-bound; 16 replicas, cache-hot)"),
}


def trace_command(workload):
    return (f"rocprofv3 --kernel-trace --stats -d <out> -o run -- python3 bench.py --workload {workload} "
            f"--steps 200 --warmup 20 --cpu-budget 0")


def pmc_commands(workload):
    run = f"python3 bench.py --workload {workload} --steps 20 --warmup 5 --cpu-budget 0"
    return [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o run -- {run}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out> -o run -- {run}",
            "calibration: the same two passes over python3 bench.py --workload copy --steps 20 --warmup 5 "
            "--cpu-budget 0 (a 256 MiB device copy)"]


def kernel_bytes(workload):
    """Algorithmic bytes of one k_gate_up and one k_down launch: each moves
    its experts' codes and scales once; gate_up also reads x, down writes out
    and reads the router weights (the hidden vector between them is not
    counted)."""
    spec, E, _ = DECODE[workload]
    bits, dm, dff = spec["bits"], spec["d_model"], spec["d_ff"]
    sb = 2 if spec.get("scale_f16") else 4
    mat = lambda rows, cols: rows * cols * bits // 8 + rows * (cols // 64) * sb
    return {"k_gate_up": E * 2 * mat(dff, dm) + 4 * dm, "k_down": E * mat(dm, dff) + 4 * dm + 4 * E}


def short_name(name, grid_blocks):
    """Template name without namespaces or arguments; read kernels keyed by grid."""
    if name.startswith("_Z"):
        m = re.search(r"_GLOBAL__N_1(\d+)", name)
        if m:
            n = int(m.group(1))
            name = name[m.end():m.end() + n]
    else:
        name = re.sub(r"^void ", "", name)
        name = re.sub(r"\([^()]*\)$", "", name)   # the argument list
        name = name.split("::")[-1] if "<" not in name else re.sub(r"^.*::(?=k_)", "", name)
    if name.startswith("k_stream_read"):
        name = f"k_stream_read (grid {grid_blocks} blocks)"
    return name


def pct(v, p):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(p * (len(v) - 1)))))]


def cmd_trace(workload, db):
    c = sqlite3.connect(db)
    rows = c.execute("select name, start, end, grid_x, workgroup_x from kernels order by start").fetchall()
    kb = kernel_bytes(workload)
    per = {}
    seq = []
    for name, s, e, gx, wx in rows:
        n = short_name(name, gx // max(1, wx))
        if not n.startswith("k_"):
            continue
        per.setdefault(n, []).append((e - s) / 1000.0)
        seq.append((n, s, e))
    kernels = {}
    for n, d in per.items():
        k = {"dispatches": len(d), "median_us": round(statistics.median(d), 3), "p10_us": round(pct(d, 0.1), 3),
             "p90_us": round(pct(d, 0.9), 3), "mean_us": round(statistics.fmean(d), 3)}
        base = n.split("<")[0]
        if base in kb:
            k["algorithmic_bytes"] = kb[base]
            k["achieved_gbs"] = round(kb[base] / (k["median_us"] * 1e-6) / 1e9, 1)
            k["frac_hbm"] = round(k["achieved_gbs"] / PEAK, 4)
        else:
            k["not_part_of_call"] = True
        kernels[n] = k
    # One call: a k_gate_up and the k_down after it.
    spans, start = [], None
    for n, s, e in seq:
        if n.startswith("k_gate_up"):
            start = s
        elif n.startswith("k_down") and start is not None:
            spans.append((e - start) / 1000.0)
            start = None
    call_kernels = [k for k in kernels.values() if "algorithmic_bytes" in k]
    out = {"workload": workload, "kernel_source_hash": bench.kernel_source_hash("decode"),
           "command": trace_command(workload), "kernels": kernels,
           "call": {"sum_of_kernel_medians_us": round(sum(k["median_us"] for k in call_kernels), 3),
                    "algorithmic_bytes": sum(kb.values()),
                    "span_median_us": round(statistics.median(spans), 3) if spans else None,
                    "span_p10_us": round(pct(spans, 0.1), 3) if spans else None,
                    "span_p90_us": round(pct(spans, 0.9), 3) if spans else None,
                    "calls": len(spans)}}
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernels.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def counter_medians(path):
    """Median counter value (KiB) per kernel over its dispatches."""
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            gx = int(r.get("Grid_Size", r.get("Grid_Size_X", "0")) or 0)
            wx = int(r.get("Workgroup_Size", r.get("Workgroup_Size_X", "1")) or 1)
            vals.setdefault(short_name(r["Kernel_Name"], gx // max(1, wx)), []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def copy_scale(path):
    m = counter_medians(path)
    name = max(m, key=m.get)   # the copy kernel moves by far the most bytes
    return COPY_BYTES / (m[name] * 1024.0)


def cmd_pmc(workload, fetch, write, copy_fetch, copy_write):
    fs, ws = copy_scale(copy_fetch), copy_scale(copy_write)
    fm, wm = counter_medians(fetch), counter_medians(write)
    kb = kernel_bytes(workload)
    per, traffic = {}, 0.0
    for n in sorted(fm):
        if n.split("<")[0] not in kb:
            continue
        per[n] = {"FETCH_SIZE_KiB": round(fm[n], 4), "WRITE_SIZE_KiB": round(wm.get(n, 0.0), 4)}
        traffic += fm[n] * 1024.0 * fs + wm.get(n, 0.0) * 1024.0 * ws
    out = {"workload": workload, "kernel_source_hash": bench.kernel_source_hash("decode"),
           "commands": pmc_commands(workload),
           "calibration": {"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
           "per_kernel_median_KiB_per_dispatch": per, "traffic_bytes_per_step": int(round(traffic)),
           "algorithmic_bytes_per_step": sum(kb.values()),
           "traffic_over_algorithmic": round(traffic / sum(kb.values()), 4)}
    with open(os.path.join(ROOT, "profiles", f"{workload}_pmc.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def render_text(workload):
    """The markdown summary of a workload from its committed JSON files."""
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernels.json")) as f:
        d = json.load(f)
    title = DECODE[workload][2]
    L = [f"# rocprofv3 kernel trace: {title}", "", "Command (from the repository root on one MI355X):", "",
         "```", d["command"], "```", "",
         "Durations of this library's kernels over every dispatch of the run (warmup, timed steps and the "
         "per-call event samples), in microseconds; achieved = algorithmic bytes per launch / median duration; "
         "frac = achieved / 8 TB/s. Summarised by `python -m group_quantized_moe_amd.bench.profile_summary "
         f"trace {workload} <out>/run_results.db`.", "",
         "| kernel | dispatches | median us | p10 us | p90 us | mean us | algorithmic bytes / launch | "
         "achieved GB/s | frac of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for n, k in d["kernels"].items():
        L.append(f"| `{n}` | {k['dispatches']} | {k['median_us']:.2f} | {k['p10_us']:.2f} | {k['p90_us']:.2f} | "
                 f"{k['mean_us']:.2f} | {k.get('algorithmic_bytes', '-')} | {k.get('achieved_gbs', '-')} | "
                 f"{k.get('frac_hbm', '-')} |")
    c = d["call"]
    if any(n.startswith("k_stream_read") for n in d["kernels"]):
        L += ["", "k_stream_read is the same run's read ceiling, not part of the call: a plain streaming read of "
              "the group's bytes (rotated over >= 1 GiB of buffers) as one launch, and of gate_up's bytes then "
              "down's as two, each with a one-pass grid and with 4 blocks per CU. Its rows are keyed by grid "
              "size, so the 4-blocks-per-CU launches of all three reads share one row."]
    gbs = c["algorithmic_bytes"] / (c["sum_of_kernel_medians_us"] * 1e-6) / 1e9
    L += ["", f"Sum of the per-launch medians of one call: {c['sum_of_kernel_medians_us']:.2f} us "
              f"({c['algorithmic_bytes']} algorithmic bytes per call; {gbs:.0f} GB/s = {gbs / PEAK:.3f} of 8 TB/s)."]
    if c.get("span_median_us"):
        L.append(f"GPU span of one call (first kernel's start to its last kernel's end, {c['calls']} calls): median "
                 f"{c['span_median_us']:.2f} us, p10 {c['span_p10_us']:.2f}, p90 {c['span_p90_us']:.2f}; the gaps "
                 "between the launches of one call are the difference to the sum above.")
    pmc = os.path.join(ROOT, "profiles", f"{workload}_pmc.json")
    if os.path.exists(pmc):
        with open(pmc) as f:
            p = json.load(f)
        if p.get("kernel_source_hash") == d["kernel_source_hash"]:
            cal = p["calibration"]
            L += ["", f"HBM traffic from rocprofv3 counters (median per dispatch; FETCH_SIZE x "
                      f"{cal['fetch_scale']:.3f} and WRITE_SIZE x {cal['write_scale']:.3f}, the factors a 256 MiB "
                      "device copy needs to read back its known size):", "",
                  "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic bytes |", "|---|---|---|---|"]
            for n, k in p["per_kernel_median_KiB_per_dispatch"].items():
                t = k["FETCH_SIZE_KiB"] * 1024 * cal["fetch_scale"] + k["WRITE_SIZE_KiB"] * 1024 * cal["write_scale"]
                L.append(f"| `{n}` | {k['FETCH_SIZE_KiB']:.0f} | {k['WRITE_SIZE_KiB']:.0f} | {t:.0f} |")
            L += ["", f"Traffic per call {p['traffic_bytes_per_step']} bytes = {p['traffic_over_algorithmic']:.3f} x "
                      f"the algorithmic bytes (`profiles/{workload}_pmc.json`)."]
    L += ["", f"Machine-readable: `profiles/{workload}_kernels.json` (kernel source hash {d['kernel_source_hash']}; "
              "bench.py reports these figures only while the kernel sources hash the same)."]
    return "\n".join(L) + "\n"


def cmd_render(workload):
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernel_trace.md"), "w") as f:
        f.write(render_text(workload))


def main(argv):
    cmd, workload = argv[0], argv[1]
    if workload not in DECODE:
        raise SystemExit(f"unknown decode workload {workload!r}")
    if cmd == "trace":
        cmd_trace(workload, argv[2])
        cmd_render(workload)
    elif cmd == "pmc":
        cmd_pmc(workload, *argv[2:6])
        cmd_render(workload)
    elif cmd == "render":
        cmd_render(workload)
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
