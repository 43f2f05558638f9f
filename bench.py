"""Benchmark: effective HBM bandwidth and microseconds per Q4 8-expert FFN
decode group on one MI355X.

One step = one smoe_expert_ffn call with T = 1: the fused gate+up+SiLU pass
and the down pass with the router-weighted sum over 8 experts at d_model 4096,
d_ff 1536, 4-bit codes, group 64, f32 scales.  Inputs are seeded synthetic
weights with the shapes and distributions of the Metal Compute Kernels page
(S-MoE docs) workload; they stand in for trained vault blobs.  Weights sit in
HBM before the timed region; to keep the 256 MB Infinity Cache from serving
them, the step cycles through >= 1 GiB of byte-identical replicas.

Prints one JSON line (see the keys below).  `python bench.py --steps K --warmup W`.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak, GB/s
KERNEL_SOURCES = ["group_quantized_moe_amd/csrc/q_decode.hip", "group_quantized_moe_amd/csrc/common.h",
                  "group_quantized_moe_amd/csrc/launch.h", "group_quantized_moe_amd/csrc/smoe_api.cpp"]


def algorithmic_bytes(g, n_experts):
    """Codes + scales of every matrix, x, out and the router weights, each once."""
    weights = g.byte_count()
    return weights + 4 * g.d_model + 4 * g.d_model + 4 * n_experts


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """Measured HBM bytes per step from the committed rocprofv3 counter runs,
    if they were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "decode_q4_8expert_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_step")


def cpu_baseline(g, x, r, budget_s):
    """The f64 oracle on the host: whole 8-expert groups, repeated until the
    time budget is used (at least one group)."""
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.expert_ffn(g.experts, g.bits, g.group, g.d_model, g.d_ff, x, r[None])
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return n, dt, oracle.threads()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 to skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import group_quantized_moe_amd as gq

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    L = gq.lib()
    spec = workloads.Q4_GROUP8
    g, x, r = workloads.make_decode_inputs(spec)
    E = spec["n_experts"]
    nbytes = algorithmic_bytes(g, E)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    base = [to_dev(t) for e in g.experts for m in (e.gate, e.up, e.down) for t in (m.codes, m.scales)]
    replicas = max(2, -(-(1 << 30) // g.byte_count()))
    reps = [base] + [[t.clone() for t in base] for _ in range(replicas - 1)]
    arrays = []
    for rep in reps:
        arr = (gq.Expert * E)()
        for k in range(E):
            gc, gs, uc, us, dc, ds = rep[6 * k:6 * k + 6]
            arr[k] = gq.Expert(gq.QMat(gc.data_ptr(), gs.data_ptr()), gq.QMat(uc.data_ptr(), us.data_ptr()),
                               gq.QMat(dc.data_ptr(), ds.data_ptr()))
        arrays.append(arr)
    xd, rd = to_dev(x), to_dev(r)
    out = torch.empty(g.d_model, dtype=torch.float32, device="cuda")
    ws = torch.zeros(gq.smoe_expert_ffn_workspace(E, g.d_model, g.d_ff, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        rc = L.smoe_expert_ffn(arrays[i % replicas], E, rd.data_ptr(), g.bits, g.group, g.d_model, g.d_ff, 1,
                               xd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_expert_ffn", rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K back-to-back steps between two events on the launch stream.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = e0.elapsed_time(e1)
    us_step = gpu_ms * 1e3 / args.steps
    gbs = nbytes / (us_step * 1e-6) / 1e9

    # Per-launch duration of the step's kernels, measured with an event pair
    # around each step (sampled separately so the timed region has no extra
    # events in it).
    nsamp = min(100, args.steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsamp)]
    for i in range(nsamp):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per_launch_us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))

    cpu = None
    if args.cpu_budget > 0:
        n, dt, cores = cpu_baseline(g, x, r, args.cpu_budget)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole Q4 8-expert groups (f64 oracle, {dt:.1f} s)",
               "us_per_group": round(dt / n * 1e6, 1)}

    achieved = nbytes / (us_step * 1e-6) / 1e9
    line = {
        "metric": "effective HBM GB/s per Q4 8-expert FFN group (decode, T=1)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6),
        "us_per_group": round(us_step, 3),
        "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes x int4 digit planes -> int32, f32 epilogue",
        "data": "synthetic (seeded; stands in for trained expert weights)",
        "config": {"workload": spec["name"], "d_model": g.d_model, "d_ff": g.d_ff, "n_experts": E,
                   "bits": g.bits, "group": g.group, "scales": "f32", "tokens": 1,
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": replicas,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "kernel": "smoe_expert_ffn T=1 (k_gate_up + k_down)",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(),
            "per_launch_us_events": round(per_launch_us, 3),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
