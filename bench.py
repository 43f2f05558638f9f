"""Benchmark of the group-quantised routed-expert FFN path on one MI355X.

Default workload (the headline): one Q4 8-expert FFN decode group, i.e. one
smoe_expert_ffn call with T = 1 -- the fused gate+up+SiLU pass and the down
pass with the router-weighted sum over 8 experts at d_model 4096, d_ff 1536,
4-bit codes, group 64, f32 scales.  Reported as effective HBM GB/s (algorithmic
bytes / time), microseconds per group and fraction of the 8 TB/s HBM peak.

Other rows of the path, one JSON line each with --workload:
  decode_q2           the same group with 2-bit codes
  decode_q4_s16, decode_q2_s16
                      the groups with 2-byte (binary16) scales
  prefill             --tokens T (16, 64 or 256): every token through all 8
                      experts on the matrix cores (bound by HBM at T = 16, by
                      the f16 MFMA rate above)
  bf16                --shape q_proj|o_proj|kv_proj|lm_head dense matvec
  routed              --tokens T --topk K: routed prefill, each token through its
                      top-K of the 8 experts (top-K of N(0,1) logits)
  bf16_batch          q, k and v projections (8192x4096, 2 x 512x4096) over
                      one x as one batched launch, with the three separate
                      launches timed beside it
  attn                one token's decode attention block (64 query and 4 KV
                      heads of 128, d_model 4096, f32 KV cache of 4096
                      positions, the token at the last one): projections,
                      QK norm, RoPE, KV append, GQA attention, o_proj

Inputs are seeded synthetic weights with the shapes and distributions of the
Metal Compute Kernels page (S-MoE docs) workloads; they stand in for trained
weights.  Weights sit in HBM before the timed region; so that the 256 MB
Infinity Cache cannot serve them, each step cycles through >= 1 GiB of
byte-identical replicas.

`python bench.py [--workload W] --steps K --warmup W` prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, GB/s
PEAK_F16_TFLOPS = 2500.0       # MI355X dense f16 matrix peak, TFLOP/s
CSRC = "group_quantized_moe_amd/csrc/"
# The kernel sources (device code, tiling and launch plan) behind each workload:
# the counter-based traffic figures are only used while these are unchanged.
KERNEL_SOURCES = {
    "decode": [CSRC + "q_decode.hip", CSRC + "common.h"],
    "prefill": [CSRC + "q_batch.hip", CSRC + "common.h"],
    "bf16": [CSRC + "bf16_matvec.hip", CSRC + "common.h"],
    "attn": [CSRC + "attn.hip", CSRC + "bf16_matvec.hip", CSRC + "common.h"],
}


def kernel_source_hash(kind):
    """Hash of the code (comments and whitespace removed) of the sources behind
    a workload's kernels: a comment edit keeps the counter figures valid, any
    code change voids them."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, p)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(name, kind):
    """Measured HBM bytes per step from the committed rocprofv3 counter runs
    (profiles/<name>_pmc.json), if they were taken on the current kernel
    sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return d.get("traffic_bytes_per_step")


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def replica_count(nbytes):
    return max(2, -(-(1 << 30) // nbytes))


def expert_arrays(gq, g, E, replicas):
    """ctypes smoe_expert arrays for `replicas` device copies of the group."""
    base = [to_dev(t) for e in g.experts for m in (e.gate, e.up, e.down) for t in (m.codes, m.scales)]
    reps = [base] + [[t.clone() for t in base] for _ in range(replicas - 1)]
    arrays = []
    for rep in reps:
        arr = (gq.Expert * E)()
        for k in range(E):
            gc, gs, uc, us, dc, ds = rep[6 * k:6 * k + 6]
            arr[k] = gq.Expert(gq.QMat(gc.data_ptr(), gs.data_ptr()), gq.QMat(uc.data_ptr(), us.data_ptr()),
                               gq.QMat(dc.data_ptr(), ds.data_ptr()))
        arrays.append(arr)
    return arrays, reps


def time_steps(step, steps, warmup, stream):
    """Warmup, then `steps` back-to-back steps between two events on the
    launch stream; then a median per-call duration from an event pair around
    each of up to 100 further calls (sampled apart from the timed region)."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    us_step = e0.elapsed_time(e1) * 1e3 / steps
    nsamp = min(100, steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsamp)]
    for i in range(nsamp):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per_call = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))
    return us_step, per_call, wall * 1e6 / steps


def cpu_oracle(fn, budget_s, units_per_call):
    """Run the f64 oracle repeatedly until budget_s has passed (at least once);
    returns (calls, seconds, threads)."""
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return n, time.perf_counter() - t0, oracle.threads()


def decode_bench(args, spec, profile):
    import torch
    import workloads
    import group_quantized_moe_amd as gq
    L = gq.lib()
    g, x, r = workloads.make_decode_inputs(spec)
    E = spec["n_experts"]
    # Algorithmic bytes: codes + scales of every matrix, x, out and the router weights, each once.
    nbytes = g.byte_count() + 4 * g.d_model + 4 * g.d_model + 4 * E
    replicas = replica_count(g.byte_count())
    arrays, _keep = expert_arrays(gq, g, E, replicas)
    xd, rd = to_dev(x), to_dev(r)
    out = torch.empty(g.d_model, dtype=torch.float32, device="cuda")
    ws = torch.zeros(gq.smoe_expert_ffn_workspace(E, g.d_model, g.d_ff, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    fmt = g.bits | (gq.SMOE_SCALE_F16 if g.scale_f16 else 0)

    def step(i):
        rc = L.smoe_expert_ffn(arrays[i % replicas], E, rd.data_ptr(), fmt, g.group, g.d_model, g.d_ff, 1,
                               xd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_expert_ffn", rc)

    us_step, per_call, wall_us = time_steps(step, args.steps, args.warmup, stream)
    gbs = nbytes / (us_step * 1e-6) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        n, dt, cores = cpu_oracle(lambda: oracle.expert_ffn(g.experts, g.bits, g.group, g.d_model, g.d_ff,
                                                            x, r[None]), args.cpu_budget, 1)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole {E}-expert Q{g.bits} groups (f64 oracle, {dt:.1f} s)",
               "us_per_group": round(dt / n * 1e6, 1)}
    return {
        "metric": f"effective HBM GB/s per Q{g.bits} {E}-expert FFN group (decode, T=1"
                  + (", f16 scales)" if g.scale_f16 else ")"),
        "value": round(gbs, 1),
        "unit": "GB/s",
        "ms_per_step": round(us_step / 1e3, 6),
        "us_per_group": round(us_step, 3),
        "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "wall_us_per_step": round(wall_us, 3),
        "dtype": f"u{g.bits} codes x i4 digit planes -> i32, f32 epilogue",
        "config": {"workload": spec["name"], "d_model": g.d_model, "d_ff": g.d_ff, "n_experts": E,
                   "bits": g.bits, "group": g.group, "scales": "f16" if g.scale_f16 else "f32", "tokens": 1,
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": replicas,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "kernel": "one smoe_expert_ffn call = k_gate_up + k_down on one stream",
            "achieved": round(nbytes / (per_call * 1e-6) / 1e9, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / (per_call * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(profile, "decode"),
            "per_call_us_events": round(per_call, 3),
        },
        "cpu_baseline": cpu,
    }


def prefill_bench(args):
    import torch
    import workloads
    import group_quantized_moe_amd as gq
    L = gq.lib()
    T = args.tokens
    spec = workloads.Q4_GROUP8
    g = workloads.make_group(spec)
    X, R = workloads.make_batch_inputs(T)
    E = spec["n_experts"]
    flops = 2 * T * E * 3 * g.d_model * g.d_ff
    nbytes = g.byte_count() + T * g.d_model * 4 * 2 + T * E * 4
    replicas = replica_count(g.byte_count())
    arrays, _keep = expert_arrays(gq, g, E, replicas)
    xd, rd = to_dev(X), to_dev(R)
    out = torch.empty(T * g.d_model, dtype=torch.float32, device="cuda")
    ws = torch.zeros(gq.smoe_expert_ffn_workspace(E, g.d_model, g.d_ff, T), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        rc = L.smoe_expert_ffn(arrays[i % replicas], E, rd.data_ptr(), 4, 64, g.d_model, g.d_ff, T,
                               xd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_expert_ffn", rc)

    us_step, per_call, wall_us = time_steps(step, args.steps, args.warmup, stream)
    tflops = flops / (per_call * 1e-6) / 1e12
    gbs = nbytes / (per_call * 1e-6) / 1e9
    hbm_bound = T <= 16
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        ns = 4
        n, dt, cores = cpu_oracle(lambda: oracle.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X[:ns], R[:ns]),
                                  args.cpu_budget, ns)
        cpu = {"value": round(n * ns * 2 * E * 3 * g.d_model * g.d_ff / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": cores, "kind": "oracle",
               "sample": f"{n} calls of {ns} tokens x {E} experts (f64 oracle, {dt:.1f} s)",
               "us_per_token": round(dt / (n * ns) * 1e6, 1)}
    return {
        "metric": f"prefill tokens/s through 8 Q4 experts (T={T}), with TFLOP/s and HBM GB/s",
        "value": round(T / (us_step * 1e-6), 1),
        "unit": "tokens/s",
        "ms_per_step": round(us_step / 1e3, 6),
        "us_per_call": round(us_step, 3),
        "tflops": round(flops / (us_step * 1e-6) / 1e12, 2),
        "hbm_gbs": round(nbytes / (us_step * 1e-6) / 1e9, 1),
        "wall_us_per_step": round(wall_us, 3),
        "dtype": "f16 exact codes x f16 hi/lo activations -> f32",
        "config": {"workload": f"prefill_q4_8expert_4096x1536_T{T}", "tokens": T, "d_model": g.d_model,
                   "d_ff": g.d_ff, "n_experts": E, "bits": 4, "group": 64, "algorithmic_flops": flops,
                   "algorithmic_bytes": nbytes, "replicas_rotated": replicas, "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "kernel": "one smoe_expert_ffn call = k_tb_prep + k_tb_gate_up + k_tb_down",
            "achieved": round(gbs if hbm_bound else tflops, 2),
            "peak": PEAK_HBM_GBS if hbm_bound else PEAK_F16_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round((gbs / PEAK_HBM_GBS) if hbm_bound else (tflops / PEAK_F16_TFLOPS), 4),
            "traffic": load_traffic(f"prefill_t{T}", "prefill"),
            "per_call_us_events": round(per_call, 3),
        },
        "cpu_baseline": cpu,
    }


def routed_bench(args):
    """Routed prefill: T tokens, each through its top_k of the 8 Q4 experts."""
    import torch
    import workloads
    import group_quantized_moe_amd as gq
    L = gq.lib()
    T, k = args.tokens, args.topk
    spec = workloads.Q4_GROUP8
    g = workloads.make_group(spec)
    X, ids, w = workloads.make_routed_inputs(T, k, workloads.ROUTED["seed"])
    E = spec["n_experts"]
    used = sorted(set(int(e) for e in ids.ravel()))
    flops = 2 * T * k * 3 * g.d_model * g.d_ff
    per_expert = g.byte_count() // E
    nbytes = per_expert * len(used) + T * g.d_model * 4 * 2 + T * k * 8
    replicas = replica_count(g.byte_count())
    arrays, _keep = expert_arrays(gq, g, E, replicas)
    xd, idd, wd = to_dev(X), to_dev(ids), to_dev(w)
    out = torch.empty(T * g.d_model, dtype=torch.float32, device="cuda")
    ws = torch.zeros(gq.smoe_routed_ffn_workspace(E, g.d_model, g.d_ff, T, k), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        rc = L.smoe_routed_ffn(arrays[i % replicas], E, 4, 64, g.d_model, g.d_ff, T, k, idd.data_ptr(),
                               wd.data_ptr(), xd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_routed_ffn", rc)

    us_step, per_call, wall_us = time_steps(step, args.steps, args.warmup, stream)
    tflops = flops / (per_call * 1e-6) / 1e12
    gbs = nbytes / (per_call * 1e-6) / 1e9
    hbm_bound = T * k <= 16 * E
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        ns = 4
        n, dt, cores = cpu_oracle(lambda: oracle.routed_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X[:ns], ids[:ns],
                                                            w[:ns]), args.cpu_budget, ns)
        cpu = {"value": round(n * ns * 2 * k * 3 * g.d_model * g.d_ff / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": cores, "kind": "oracle",
               "sample": f"{n} calls of {ns} tokens x top-{k} (f64 oracle, {dt:.1f} s)"}
    return {
        "metric": f"routed prefill tokens/s, {T} tokens x top-{k} of 8 Q4 experts",
        "value": round(T / (us_step * 1e-6), 1),
        "unit": "tokens/s",
        "ms_per_step": round(us_step / 1e3, 6),
        "us_per_call": round(us_step, 3),
        "tflops": round(flops / (us_step * 1e-6) / 1e12, 2),
        "hbm_gbs": round(nbytes / (us_step * 1e-6) / 1e9, 1),
        "wall_us_per_step": round(wall_us, 3),
        "dtype": "f16 exact codes x f16 hi/lo activations -> f32",
        "config": {"workload": f"routed_prefill_q4_8expert_4096x1536_T{T}_top{k}", "tokens": T, "top_k": k,
                   "experts_used": len(used), "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                   "replicas_rotated": replicas, "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "kernel": "one smoe_routed_ffn call (slot lists with token prep, gate_up [+ finish], down, combine)",
            "achieved": round(gbs if hbm_bound else tflops, 2),
            "peak": PEAK_HBM_GBS if hbm_bound else PEAK_F16_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round((gbs / PEAK_HBM_GBS) if hbm_bound else (tflops / PEAK_F16_TFLOPS), 4),
            "traffic": load_traffic(f"routed_t{T}_k{k}", "prefill"),
            "per_call_us_events": round(per_call, 3),
        },
        "cpu_baseline": cpu,
    }


def bf16_bench(args):
    import torch
    import workloads
    import group_quantized_moe_amd as gq
    L = gq.lib()
    shape = {s[2]: s for s in workloads.BF16_SHAPES}[args.shape]
    rows, cols, role, seed = shape
    W, x = workloads.make_bf16(rows, cols, seed)
    nbytes = rows * cols * 2 + cols * 4 + rows * 4
    replicas = replica_count(rows * cols * 2)
    Wd = to_dev(W)
    reps = [Wd] + [Wd.clone() for _ in range(replicas - 1)]
    xd = to_dev(x)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        rc = L.matvec_bf16(reps[i % replicas].data_ptr(), rows, cols, xd.data_ptr(), y.data_ptr(), None, 0, sp)
        if rc != 0:
            raise gq.SmoeError("matvec_bf16", rc)

    us_step, per_call, wall_us = time_steps(step, args.steps, args.warmup, stream)
    gbs = nbytes / (us_step * 1e-6) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        n, dt, cores = cpu_oracle(lambda: oracle.matvec_bf16(W, x), args.cpu_budget, 1)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole {rows}x{cols} matvecs (f64 oracle, {dt:.1f} s)"}
    return {
        "metric": f"effective HBM GB/s of the bf16 matvec {rows}x{cols} ({role})",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "ms_per_step": round(us_step / 1e3, 6),
        "us_per_call": round(us_step, 3),
        "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "wall_us_per_step": round(wall_us, 3),
        "dtype": "bf16 x f32 -> f32",
        "config": {"workload": f"bf16_{role}_{rows}x{cols}", "rows": rows, "cols": cols,
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": replicas,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "kernel": "k_matvec_bf16 (one launch per call)",
            "achieved": round(nbytes / (per_call * 1e-6) / 1e9, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / (per_call * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(f"bf16_{role}", "bf16"),
            "per_call_us_events": round(per_call, 3),
        },
        "cpu_baseline": cpu,
    }


def bf16_batch_bench(args):
    """The batched bf16 matvec: a token's q, k and v projections over one x in
    one launch, against the same three matvecs launched one by one."""
    import torch
    import workloads
    import group_quantized_moe_amd as gq
    L = gq.lib()
    jobs = workloads.BF16_BATCH
    Ws, x = workloads.make_bf16_batch(jobs)
    cols = jobs[0][1]
    wbytes = sum(r * c * 2 for r, c, _, _ in jobs)
    nbytes = wbytes + cols * 4 + sum(r * 4 for r, _, _, _ in jobs)
    replicas = replica_count(wbytes)
    dWs = [to_dev(W) for W in Ws]
    reps = [dWs] + [[w.clone() for w in dWs] for _ in range(replicas - 1)]
    xd = to_dev(x)
    ys = [torch.empty(r, dtype=torch.float32, device="cuda") for r, _, _, _ in jobs]
    arrays = [gq.bf16_job_array([(w, xd, y) for w, y in zip(rep, ys)]) for rep in reps]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        rc = L.matvec_bf16_batch(arrays[i % replicas], len(jobs), sp)
        if rc != 0:
            raise gq.SmoeError("matvec_bf16_batch", rc)

    def step_separate(i):
        for w, y, (r, c, _, _) in zip(reps[i % replicas], ys, jobs):
            rc = L.matvec_bf16(w.data_ptr(), r, c, xd.data_ptr(), y.data_ptr(), None, 0, sp)
            if rc != 0:
                raise gq.SmoeError("matvec_bf16", rc)

    us_step, per_call, wall_us = time_steps(step, args.steps, args.warmup, stream)
    us_sep, per_sep, _ = time_steps(step_separate, args.steps, args.warmup, stream)
    gbs = nbytes / (us_step * 1e-6) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        n, dt, cores = cpu_oracle(lambda: [oracle.matvec_bf16(W, x) for W in Ws], args.cpu_budget, 1)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole q/k/v batches (f64 oracle, {dt:.1f} s)"}
    shapes = "+".join(f"{r}x{c}" for r, c, _, _ in jobs)
    return {
        "metric": f"effective HBM GB/s of one batched bf16 matvec launch ({shapes}, shared x)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "ms_per_step": round(us_step / 1e3, 6),
        "us_per_call": round(us_step, 3),
        "us_per_call_separate_launches": round(us_sep, 3),
        "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "wall_us_per_step": round(wall_us, 3),
        "dtype": "bf16 x f32 -> f32",
        "config": {"workload": f"bf16_batch_qkv_{shapes}", "jobs": [list(j[:3]) for j in jobs],
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": replicas,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "kernel": "k_matvec_bf16_batch (one launch per call)",
            "achieved": round(nbytes / (per_call * 1e-6) / 1e9, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / (per_call * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": load_traffic("bf16_batch_qkv", "bf16"),
            "per_call_us_events": round(per_call, 3),
            "per_call_us_events_separate_launches": round(per_sep, 3),
        },
        "cpu_baseline": cpu,
    }


def attn_bench(args):
    """One token's decode attention block (smoe_attn_decode) over a full
    4096-position cache, with every weight and cache replica rotated."""
    import torch
    import workloads
    import group_quantized_moe_amd as gq
    L = gq.lib()
    spec = workloads.ATTN
    w, x, K, V = workloads.make_attn_inputs(spec)
    dm, H, KV, hd, ctx, pos = (spec[k] for k in ("d_model", "n_head", "n_kv", "head_dim", "max_ctx", "pos"))
    nq, nk = H * hd, KV * hd
    wbytes = 2 * (nq * dm + 2 * nk * dm + dm * nq) + 4 * 2 * hd
    kv_read = 2 * KV * pos * hd * 4            # cached rows 0..pos-1 of K and V
    # Algorithmic bytes: every weight once, the cached rows once, x and out, the appended rows.
    nbytes = wbytes + kv_read + 4 * dm * 2 + 2 * nk * 4
    replicas = replica_count(wbytes + 2 * KV * ctx * hd * 4)
    base = [to_dev(a) for a in (w.wq, w.wk, w.wv, w.wo, w.q_norm, w.k_norm, K, V)]
    reps = [base] + [[t.clone() for t in base] for _ in range(replicas - 1)]
    structs = [gq.AttnWeights(*(t.data_ptr() for t in rep[:6])) for rep in reps]
    xd = to_dev(x)
    out = torch.empty(dm, dtype=torch.float32, device="cuda")
    ws = torch.empty(gq.smoe_attn_decode_workspace(dm, H, KV, hd, ctx), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        r = i % replicas
        rc = L.smoe_attn_decode(ctypes.byref(structs[r]), dm, H, KV, hd, xd.data_ptr(), pos, spec["rope_base"],
                                reps[r][6].data_ptr(), reps[r][7].data_ptr(), ctx, out.data_ptr(), ws.data_ptr(),
                                ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_attn_decode", rc)

    us_step, per_call, wall_us = time_steps(step, args.steps, args.warmup, stream)
    gbs = nbytes / (us_step * 1e-6) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        n, dt, cores = cpu_oracle(lambda: oracle.attn_decode(w, x, pos, spec["rope_base"], K, V),
                                  args.cpu_budget, 1)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole attention blocks at position {pos} (f64 oracle, {dt:.1f} s)",
               "us_per_block": round(dt / n * 1e6, 1)}
    return {
        "metric": "effective HBM GB/s per decode attention block (64/4 heads x 128, 4096-position f32 KV cache)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "ms_per_step": round(us_step / 1e3, 6),
        "us_per_block": round(us_step, 3),
        "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "wall_us_per_step": round(wall_us, 3),
        "dtype": "bf16 x f32 -> f32 projections, f32 attention",
        "config": {"workload": spec["name"], "d_model": dm, "n_head": H, "n_kv": KV, "head_dim": hd,
                   "max_ctx": ctx, "pos": pos, "rope_base": spec["rope_base"],
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": replicas,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "kernel": "one smoe_attn_decode call = qkv batch + partial (norm, rotation, append, chunk attention) + combine + o_proj on one stream",
            "achieved": round(nbytes / (per_call * 1e-6) / 1e9, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / (per_call * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": load_traffic("attn_decode", "attn"),
            "per_call_us_events": round(per_call, 3),
        },
        "cpu_baseline": cpu,
    }


def copy_calibration(args):
    """A plain device-to-device copy of 256 MiB (torch's copy kernel): the
    counter runs divide FETCH_SIZE / WRITE_SIZE of a kernel by what the same
    counters read for this copy of known size."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    us_step, per_call, wall_us = time_steps(lambda i: dst.copy_(src), args.steps, args.warmup, stream)
    return {"metric": "device-to-device copy of 256 MiB (counter calibration)",
            "value": round(2 * n / (us_step * 1e-6) / 1e9, 1), "unit": "GB/s (read + write)",
            "ms_per_step": round(us_step / 1e3, 6), "bytes_read": n, "bytes_written": n,
            "dtype": "u8", "config": {"workload": "copy_256MiB"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_q4", choices=["decode_q4", "decode_q2", "decode_q4_s16", "decode_q2_s16", "prefill", "bf16",
                             "bf16_batch", "routed", "attn", "copy"])
    ap.add_argument("--tokens", type=int, default=16, help="prefill / routed: tokens per call")
    ap.add_argument("--topk", type=int, default=2, help="routed: experts per token")
    ap.add_argument("--shape", default="q_proj", help="bf16: q_proj, o_proj, kv_proj or lm_head")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 to skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU code: it runs on one device)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.workload == "decode_q4":
        line = decode_bench(args, workloads.Q4_GROUP8, "decode_q4")
    elif args.workload == "decode_q2":
        line = decode_bench(args, workloads.Q2_GROUP8, "decode_q2")
    elif args.workload == "decode_q4_s16":
        line = decode_bench(args, workloads.Q4_GROUP8_S16, "decode_q4_s16")
    elif args.workload == "decode_q2_s16":
        line = decode_bench(args, workloads.Q2_GROUP8_S16, "decode_q2_s16")
    elif args.workload == "prefill":
        line = prefill_bench(args)
    elif args.workload == "copy":
        line = copy_calibration(args)
    elif args.workload == "routed":
        line = routed_bench(args)
    elif args.workload == "bf16_batch":
        line = bf16_batch_bench(args)
    elif args.workload == "attn":
        line = attn_bench(args)
    else:
        line = bf16_bench(args)
    head = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded; stands in for trained weights)"}
    print(json.dumps({**{k: line[k] for k in ("metric", "value", "unit")}, **head,
                      **{k: v for k, v in line.items() if k not in ("metric", "value", "unit")}}), flush=True)


if __name__ == "__main__":
    main()
