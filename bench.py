"""Benchmark of the group-quantised routed-expert FFN path on one MI355X.

Default run (the headline): one Q4 8-expert FFN decode group, i.e. one
smoe_expert_ffn call with T = 1 -- the fused gate+up+SiLU pass and the down
pass with the router-weighted sum over 8 experts at d_model 4096, d_ff 1536,
4-bit codes, group 64, f32 scales.  Reported as effective HBM GB/s (algorithmic
bytes / time), microseconds per group and per expert, and fraction of the
8 TB/s HBM peak.  The same JSON line carries:

  roofline       the call's achieved rate from the same timing as `value`, the
                 per-kernel figures of the committed rocprofv3 trace and the
                 counter-based HBM traffic (null once the kernels changed)
  read_ceiling   a plain streaming read of the same number of bytes, timed in
                 the same run (one reduction launch over rotated buffers)
  mfma_ceiling   (with the rows; token-batch lines) the rate the token batch's
                 matrix instruction sustains on register operands in the same
                 run, against which each token-batch row's f16 matrix work (twice
                 its algorithmic flops: hi and lo halves) is also given
  cpu_baseline   the f64 oracle on the host: all threads, and one thread
  rows           every other workload of the path timed in the same run, each
                 back to back like the headline: the tiny single expert, one
                 expert of the group, the Q2 group, both groups with 2-byte
                 scales, the four bf16 matvec shapes, the token batch at
                 T = 16, 64 and 256 and the routed batch (16 and 256 tokens,
                 top-2)

`--workload W` prints one line for a single workload instead (used for the
rocprofv3 runs behind profiles/): decode_q4, decode_q2, decode_q4_s16,
decode_q2_s16, decode_q4_e1, tiny, prefill (--tokens), bf16 (--shape), routed
(--tokens --topk), bf16_batch, attn, copy (counter calibration).

Inputs are seeded synthetic weights with the shapes and distributions of the
Metal Compute Kernels page (S-MoE docs) workloads; they stand in for trained
weights.  Weights sit in HBM before the timed region; so that the 256 MB
Infinity Cache cannot serve them, each step cycles through >= 1 GiB of
byte-identical replicas (the tiny single expert excepted: it is latency-bound
and reported as such).

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
# the counter and trace figures in profiles/ are only used while these are unchanged.
KERNEL_SOURCES = {
    "decode": [CSRC + "q_decode.hip", CSRC + "common.h"],
    "prefill": [CSRC + "q_batch.hip", CSRC + "common.h"],
    "bf16": [CSRC + "bf16_matvec.hip", CSRC + "common.h"],
    "attn": [CSRC + "attn.hip", CSRC + "bf16_matvec.hip", CSRC + "common.h"],
}
DECODE_DTYPE = ("x and hidden as 22-bit block fixed point (one exponent per 16-byte code chunk, six signed "
                "4-bit digit planes) times u{bits} codes: exact i32 dot products; f32 per-chunk epilogue and "
                "row sums; f64 router-weighted expert sum")
BATCH_DTYPE = ("exact f16 codes x f16 hi/lo halves of power-of-two-scaled activations (about 22 bits) "
               "-> f32 MFMA accumulate; f32 epilogue")


def kernel_source_hash(kind):
    """Hash of the code (comments and whitespace removed) of the sources behind
    a workload's kernels: a comment edit keeps the profile figures valid, any
    code change voids them."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, p)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()[:16]


def _profile_json(name, kind, suffix):
    path = os.path.join(ROOT, "profiles", f"{name}_{suffix}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    return d if d.get("kernel_source_hash") == kernel_source_hash(kind) else None


def load_traffic(name, kind):
    """Measured HBM bytes per step from the committed rocprofv3 counter runs
    (profiles/<name>_pmc.json), if they were taken on the current kernel
    sources; else None."""
    d = _profile_json(name, kind, "pmc")
    return d.get("traffic_bytes_per_step") if d else None


def load_kernels(name, kind):
    """Per-kernel durations (median, p10, p90) and achieved rates from the
    committed rocprofv3 kernel trace (profiles/<name>_kernels.json), if it was
    taken on the current kernel sources; else None."""
    d = _profile_json(name, kind, "kernels")
    return d.get("kernels") if d else None


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
    base = [to_dev(t) for e in g.experts[:E] for m in (e.gate, e.up, e.down) for t in (m.codes, m.scales)]
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


def time_calls(step, steps, warmup, stream):
    """Warmup, then `steps` back-to-back steps between two HIP events on the
    launch stream (us per step, the figure every rate is computed from); then
    an event pair around each of up to 200 further single calls, for the
    spread of one call's duration (median, p10, p90)."""
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
    nsamp = min(200, max(steps, 20))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsamp)]
    for i in range(nsamp):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    spread = {"median": round(float(np.median(d)), 3), "p10": round(float(np.percentile(d, 10)), 3),
              "p90": round(float(np.percentile(d, 90)), 3), "samples": nsamp}
    return us_step, spread, wall * 1e6 / steps


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle(fn, budget_s, threads=None):
    """Run the f64 oracle repeatedly until budget_s has passed (at least once),
    optionally with a given number of threads; returns (calls, seconds, threads)."""
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    before = oracle.threads()
    if threads:
        oracle.set_threads(threads)
    try:
        used = oracle.threads()
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return n, time.perf_counter() - t0, used
    finally:
        oracle.set_threads(before)


def stream_ptr():
    import torch
    return torch.cuda.current_stream(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------------------
# Decode (T = 1)
# ---------------------------------------------------------------------------

def decode_measure(spec, steps, warmup, n_experts=None, replicas=None):
    """One smoe_expert_ffn call per step on a decode group (optionally its
    first n_experts experts only), rotating device replicas."""
    import torch
    import workloads
    import group_quantized_moe_amd as gq
    L = gq.lib()
    g, x, r = workloads.make_decode_inputs(spec)
    E = n_experts or spec["n_experts"]
    r = r[:E].copy()
    wbytes = g.byte_count() // spec["n_experts"] * E
    # Algorithmic bytes: codes + scales of every matrix, x, out and the router weights, each once.
    nbytes = wbytes + 4 * g.d_model + 4 * g.d_model + 4 * E
    replicas = replicas or replica_count(wbytes)
    arrays, _keep = expert_arrays(gq, g, E, replicas)
    xd, rd = to_dev(x), to_dev(r)
    out = torch.empty(g.d_model, dtype=torch.float32, device="cuda")
    ws = torch.empty(gq.smoe_expert_ffn_workspace(E, g.d_model, g.d_ff, 1), dtype=torch.uint8, device="cuda")
    stream, sp = stream_ptr()
    fmt = g.bits | (gq.SMOE_SCALE_F16 if g.scale_f16 else 0)

    def step(i):
        rc = L.smoe_expert_ffn(arrays[i % replicas], E, rd.data_ptr(), fmt, g.group, g.d_model, g.d_ff, 1,
                               xd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_expert_ffn", rc)

    us, spread, wall = time_calls(step, steps, warmup, stream)
    return dict(g=g, x=x, r=r, E=E, nbytes=nbytes, replicas=replicas, us=us, spread=spread, wall=wall,
                gbs=nbytes / (us * 1e-6) / 1e9)


def decode_row(spec, steps, warmup, n_experts=None, replicas=None, note=None, profile=None):
    m = decode_measure(spec, steps, warmup, n_experts, replicas)
    row = {"us": round(m["us"], 3), "gbs": round(m["gbs"], 1), "frac": round(m["gbs"] / PEAK_HBM_GBS, 4),
           "bound": "hbm", "per_call_us": m["spread"], "algorithmic_bytes": m["nbytes"],
           "replicas_rotated": m["replicas"]}
    if profile:
        row["kernels"] = row_kernels(profile, "decode")
    if note:
        row["note"] = note
    return row


def row_kernels(name, kind):
    """Median / p10 / p90 kernel durations (us) from the committed kernel
    trace of a workload (profiles/<name>_kernels.json) when it was taken on
    the current kernel sources, else None."""
    k = load_kernels(name, kind)
    if not k:
        return None
    return {n: {f: v[f] for f in ("median_us", "p10_us", "p90_us") if f in v} for n, v in k.items()}


def read_ceiling(nbytes, steps, warmup):
    """A plain streaming read of `nbytes` rotating >= 1 GiB of buffers (the
    hand-written read kernel of libsmoe_bench.so), timed like the path; the
    faster of a one-pass grid and a grid of 4 blocks per compute unit."""
    import torch
    import group_quantized_moe_amd as gq
    path = os.path.join(os.path.dirname(gq.LIB_PATH), "libsmoe_bench.so")
    if not os.path.exists(path):
        return None
    B = ctypes.CDLL(path)
    B.smoe_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p]
    n = -(-nbytes // 16) * 16
    reps = replica_count(n)
    bufs = [torch.full((n,), i & 0x7F, dtype=torch.uint8, device="cuda") for i in range(reps)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream, sp = stream_ptr()
    best = None
    for bpc in (0, 4):
        def step(i, bpc=bpc):
            if B.smoe_bench_stream_read(bufs[i % reps].data_ptr(), n, sink.data_ptr(), bpc, sp) != 0:
                raise RuntimeError("stream read launch failed")
        us, spread, _ = time_calls(step, steps, warmup, stream)
        if best is None or us < best[0]:
            best = (us, spread, bpc)
    del bufs
    us, spread, bpc = best
    return {"us": round(us, 3), "gbs": round(n / (us * 1e-6) / 1e9, 1), "frac": round(n / (us * 1e-6) / 1e9 /
            PEAK_HBM_GBS, 4), "bytes": n, "per_call_us": spread,
            "kernel": "k_stream_read (libsmoe_bench.so): 16-byte loads, 4 per thread per pass, "
                      + ("one-pass grid" if bpc == 0 else f"{bpc} blocks per CU")}


def read_ceiling_pair(na, nb, steps, warmup):
    """The same plain read, as two launches per step on one stream: `na`
    bytes, then `nb` bytes (the byte counts of a two-launch path's kernels),
    each rotating >= 1 GiB of buffers; the faster of the two grid shapes."""
    import torch
    import group_quantized_moe_amd as gq
    path = os.path.join(os.path.dirname(gq.LIB_PATH), "libsmoe_bench.so")
    if not os.path.exists(path):
        return None
    B = ctypes.CDLL(path)
    B.smoe_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p]
    sizes = [-(-na // 16) * 16, -(-nb // 16) * 16]
    reps = replica_count(sum(sizes))
    bufs = [[torch.full((n,), i & 0x7F, dtype=torch.uint8, device="cuda") for n in sizes] for i in range(reps)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream, sp = stream_ptr()
    best = None
    for bpc in (0, 4):
        def step(i, bpc=bpc):
            for buf, n in zip(bufs[i % reps], sizes):
                if B.smoe_bench_stream_read(buf.data_ptr(), n, sink.data_ptr(), bpc, sp) != 0:
                    raise RuntimeError("stream read launch failed")
        us, spread, _ = time_calls(step, steps, warmup, stream)
        if best is None or us < best[0]:
            best = (us, spread, bpc)
    del bufs
    us, spread, bpc = best
    return {"us": round(us, 3), "bytes": sizes, "per_call_us": spread,
            "kernel": "k_stream_read twice per step, " + ("one-pass grids" if bpc == 0 else f"{bpc} blocks per CU")}


_MFMA_CEILING = {}


def mfma_ceiling(repeats=10):
    """The rate the token batch's matrix instruction (v_mfma_f32_16x16x32_f16)
    sustains on this GPU with nothing else in the way: the register-only
    kernel of libsmoe_bench.so, 8 blocks of 4 waves per compute unit, timed
    between HIP events (median of `repeats` launches); the 32x32x16 form
    beside it.  Measured once per run."""
    if _MFMA_CEILING:
        return dict(_MFMA_CEILING)
    import torch
    import group_quantized_moe_amd as gq
    path = os.path.join(os.path.dirname(gq.LIB_PATH), "libsmoe_bench.so")
    if not os.path.exists(path):
        return None
    B = ctypes.CDLL(path)
    B.smoe_bench_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream, sp = stream_ptr()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    bpc, iters = 8, 2000
    out = {}
    for shape, name, fl in ((0, "v_mfma_f32_16x16x32_f16", 16384), (1, "v_mfma_f32_32x32x16_f16", 32768)):
        flops = cus * bpc * 4 * iters * 4 * fl
        times = []
        for r in range(repeats + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if B.smoe_bench_mfma_rate(shape, bpc, iters, sink.data_ptr(), sp) != 0:
                raise RuntimeError("mfma rate launch failed")
            e1.record(stream)
            e1.synchronize()
            if r >= 2:
                times.append(e0.elapsed_time(e1) * 1e-3)
        out[name] = round(flops / float(np.median(times)) / 1e12, 1)
    _MFMA_CEILING.update({
        "instruction": "v_mfma_f32_16x16x32_f16",
        "tflops": out["v_mfma_f32_16x16x32_f16"],
        "frac_of_peak": round(out["v_mfma_f32_16x16x32_f16"] / PEAK_F16_TFLOPS, 4),
        "tflops_32x32x16": out["v_mfma_f32_32x32x16_f16"],
        "kernel": "k_mfma_rate (libsmoe_bench.so): 4 independent accumulator chains a wave on register operands, "
                  f"{bpc} blocks of 4 waves per CU, median of {repeats} launches",
    })
    return dict(_MFMA_CEILING)


def decode_line(args, spec, profile, with_rows=False):
    m = decode_measure(spec, args.steps, args.warmup)
    g, E, nbytes = m["g"], m["E"], m["nbytes"]
    line = {
        "metric": f"effective HBM GB/s per Q{g.bits} {E}-expert FFN group (decode, T=1"
                  + (", f16 scales)" if g.scale_f16 else ")"),
        "value": round(m["gbs"], 1),
        "unit": "GB/s",
        "ms_per_step": round(m["us"] / 1e3, 6),
        "us_per_group": round(m["us"], 3),
        "pct_of_hbm_peak": round(100.0 * m["gbs"] / PEAK_HBM_GBS, 2),
        "per_call_us": m["spread"],
        "wall_us_per_step": round(m["wall"], 3),
        "dtype": DECODE_DTYPE.format(bits=g.bits),
        "config": {"workload": spec["name"], "d_model": g.d_model, "d_ff": g.d_ff, "n_experts": E,
                   "bits": g.bits, "group": g.group, "scales": "f16" if g.scale_f16 else "f32", "tokens": 1,
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": m["replicas"],
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "unit_of_work": "one smoe_expert_ffn call: k_gate_up then k_down on one stream",
            "timing": "back-to-back calls between HIP events on the launch stream (the timing of value)",
            "achieved": round(m["gbs"], 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(m["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(profile, "decode"),
            "kernels": load_kernels(profile, "decode"),
        },
    }
    if with_rows:
        line["us_per_expert"] = decode_row(spec, args.steps, args.warmup, n_experts=1)["us"]
    rc = read_ceiling(nbytes, args.steps, args.warmup)
    if rc:
        rc["path_time_over_ceiling"] = round(m["us"] / rc["us"], 3)
        rc["path_frac_of_ceiling"] = round(rc["us"] / m["us"], 4)
        # The same bytes read as the path's two launches read them.
        gu = g.byte_count() // spec["n_experts"] * E * 2 // 3 + 4 * g.d_model
        pair = read_ceiling_pair(gu, nbytes - gu, args.steps, args.warmup)
        if pair:
            pair["path_time_over"] = round(m["us"] / pair["us"], 3)
            rc["two_launches"] = pair
    line["read_ceiling"] = rc
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        x, r = m["x"], m["r"]
        run = lambda: oracle.expert_ffn(g.experts[:E], g.bits, g.group, g.d_model, g.d_ff, x, r[None])
        n, dt, cores = cpu_oracle(run, args.cpu_budget)
        n1, dt1, _ = cpu_oracle(run, max(1.0, args.cpu_budget / 2), threads=1)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole {E}-expert Q{g.bits} groups on {cores} threads ({dt:.1f} s) and {n1} on one "
                         f"thread ({dt1:.1f} s), f64 oracle",
               "us_per_group": round(dt / n * 1e6, 1),
               "single_thread": {"value": round(n1 * nbytes / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                 "us_per_group": round(dt1 / n1 * 1e6, 1)},
               "cpu_model": cpu_model(), "host_threads": os.cpu_count()}
    line["cpu_baseline"] = cpu
    if with_rows:
        line["rows"] = collect_rows(args)
        line["mfma_ceiling"] = mfma_ceiling()
    return line


# ---------------------------------------------------------------------------
# Token batch (T > 1, matrix cores)
# ---------------------------------------------------------------------------

def prefill_measure(T, steps, warmup):
    import torch
    import workloads
    import group_quantized_moe_amd as gq
    L = gq.lib()
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
    ws = torch.empty(gq.smoe_expert_ffn_workspace(E, g.d_model, g.d_ff, T), dtype=torch.uint8, device="cuda")
    stream, sp = stream_ptr()

    def step(i):
        rc = L.smoe_expert_ffn(arrays[i % replicas], E, rd.data_ptr(), 4, 64, g.d_model, g.d_ff, T,
                               xd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_expert_ffn", rc)

    us, spread, wall = time_calls(step, steps, warmup, stream)
    return dict(g=g, X=X, R=R, E=E, T=T, flops=flops, nbytes=nbytes, replicas=replicas, us=us, spread=spread,
                wall=wall, tflops=flops / (us * 1e-6) / 1e12, gbs=nbytes / (us * 1e-6) / 1e9)


def matrix_work(tflops):
    """The f16 matrix work behind an algorithmic rate (hi and lo halves: twice
    the flops) against the measured rate of the instruction that does it."""
    mc = mfma_ceiling()
    if not mc:
        return None
    return {"f16_work_tflops": round(2 * tflops, 2), "instruction_tflops": mc["tflops"],
            "frac_of_instruction_rate": round(2 * tflops / mc["tflops"], 4)}


def prefill_row(T, steps, warmup):
    m = prefill_measure(T, steps, warmup)
    hbm = T <= 16
    return {"us": round(m["us"], 3), "tflops": round(m["tflops"], 2), "gbs": round(m["gbs"], 1),
            "bound": "hbm" if hbm else "mfma",
            "frac": round(m["gbs"] / PEAK_HBM_GBS if hbm else m["tflops"] / PEAK_F16_TFLOPS, 4),
            "frac_hbm": round(m["gbs"] / PEAK_HBM_GBS, 4), "frac_mfma": round(m["tflops"] / PEAK_F16_TFLOPS, 4),
            "matrix_work": matrix_work(m["tflops"]),
            "per_call_us": m["spread"], "algorithmic_flops": m["flops"], "algorithmic_bytes": m["nbytes"],
            "kernels": row_kernels(f"prefill_t{T}", "prefill")}


def prefill_line(args):
    T = args.tokens
    m = prefill_measure(T, args.steps, args.warmup)
    g, E = m["g"], m["E"]
    hbm_bound = T <= 16
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        ns = 4
        X, R = m["X"], m["R"]
        n, dt, cores = cpu_oracle(lambda: oracle.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X[:ns], R[:ns]),
                                  args.cpu_budget)
        cpu = {"value": round(n * ns * 2 * E * 3 * g.d_model * g.d_ff / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": cores, "kind": "oracle",
               "sample": f"{n} calls of {ns} tokens x {E} experts (f64 oracle, {dt:.1f} s)",
               "us_per_token": round(dt / (n * ns) * 1e6, 1), "cpu_model": cpu_model()}
    return {
        "metric": f"prefill tokens/s through 8 Q4 experts (T={T}), with TFLOP/s and HBM GB/s",
        "value": round(T / (m["us"] * 1e-6), 1),
        "unit": "tokens/s",
        "ms_per_step": round(m["us"] / 1e3, 6),
        "us_per_call": round(m["us"], 3),
        "per_call_us": m["spread"],
        "tflops": round(m["tflops"], 2),
        "hbm_gbs": round(m["gbs"], 1),
        "wall_us_per_step": round(m["wall"], 3),
        "dtype": BATCH_DTYPE,
        "config": {"workload": f"prefill_q4_8expert_4096x1536_T{T}", "tokens": T, "d_model": g.d_model,
                   "d_ff": g.d_ff, "n_experts": E, "bits": 4, "group": 64, "algorithmic_flops": m["flops"],
                   "algorithmic_bytes": m["nbytes"], "replicas_rotated": m["replicas"],
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "unit_of_work": "one smoe_expert_ffn call (activation pass, gate_up, down and their finishing passes)",
            "timing": "back-to-back calls between HIP events on the launch stream (the timing of value)",
            "achieved": round(m["gbs"] if hbm_bound else m["tflops"], 2),
            "peak": PEAK_HBM_GBS if hbm_bound else PEAK_F16_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round((m["gbs"] / PEAK_HBM_GBS) if hbm_bound else (m["tflops"] / PEAK_F16_TFLOPS), 4),
            "traffic": load_traffic(f"prefill_t{T}", "prefill"),
            "kernels": load_kernels(f"prefill_t{T}", "prefill"),
            "matrix_work": matrix_work(m["tflops"]),
        },
        "mfma_ceiling": mfma_ceiling(),
        "cpu_baseline": cpu,
    }


def routed_row(T, k, steps, warmup):
    """The routed call of routed_line as a row of the headline line."""
    import types
    l = routed_line(types.SimpleNamespace(steps=steps, warmup=warmup, cpu_budget=0, tokens=T, topk=k))
    rf = l["roofline"]
    return {"us": l["us_per_call"], "tflops": l["tflops"], "gbs": l["hbm_gbs"], "bound": rf["bound"],
            "frac": rf["frac"], "matrix_work": rf["matrix_work"], "per_call_us": l["per_call_us"],
            "experts_used": l["config"]["experts_used"], "algorithmic_flops": l["config"]["algorithmic_flops"],
            "algorithmic_bytes": l["config"]["algorithmic_bytes"],
            "kernels": row_kernels(f"routed_t{T}_k{k}", "prefill")}


def routed_line(args):
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
    ws = torch.empty(gq.smoe_routed_ffn_workspace(E, g.d_model, g.d_ff, T, k), dtype=torch.uint8, device="cuda")
    stream, sp = stream_ptr()

    def step(i):
        rc = L.smoe_routed_ffn(arrays[i % replicas], E, 4, 64, g.d_model, g.d_ff, T, k, idd.data_ptr(),
                               wd.data_ptr(), xd.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_routed_ffn", rc)

    us, spread, wall = time_calls(step, args.steps, args.warmup, stream)
    tflops = flops / (us * 1e-6) / 1e12
    gbs = nbytes / (us * 1e-6) / 1e9
    hbm_bound = T * k <= 16 * E
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        ns = 4
        n, dt, cores = cpu_oracle(lambda: oracle.routed_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X[:ns], ids[:ns],
                                                            w[:ns]), args.cpu_budget)
        cpu = {"value": round(n * ns * 2 * k * 3 * g.d_model * g.d_ff / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": cores, "kind": "oracle",
               "sample": f"{n} calls of {ns} tokens x top-{k} (f64 oracle, {dt:.1f} s)", "cpu_model": cpu_model()}
    return {
        "metric": f"routed prefill tokens/s, {T} tokens x top-{k} of 8 Q4 experts",
        "value": round(T / (us * 1e-6), 1),
        "unit": "tokens/s",
        "ms_per_step": round(us / 1e3, 6),
        "us_per_call": round(us, 3),
        "per_call_us": spread,
        "tflops": round(tflops, 2),
        "hbm_gbs": round(gbs, 1),
        "wall_us_per_step": round(wall, 3),
        "dtype": BATCH_DTYPE,
        "config": {"workload": f"routed_prefill_q4_8expert_4096x1536_T{T}_top{k}", "tokens": T, "top_k": k,
                   "experts_used": len(used), "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                   "replicas_rotated": replicas, "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "unit_of_work": "one smoe_routed_ffn call (slot lists with token prep, gate_up [+ finish], down, combine)",
            "timing": "back-to-back calls between HIP events on the launch stream (the timing of value)",
            "achieved": round(gbs if hbm_bound else tflops, 2),
            "peak": PEAK_HBM_GBS if hbm_bound else PEAK_F16_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round((gbs / PEAK_HBM_GBS) if hbm_bound else (tflops / PEAK_F16_TFLOPS), 4),
            "traffic": load_traffic(f"routed_t{T}_k{k}", "prefill"),
            "kernels": load_kernels(f"routed_t{T}_k{k}", "prefill"),
            "matrix_work": matrix_work(tflops),
        },
        "mfma_ceiling": mfma_ceiling(),
        "cpu_baseline": cpu,
    }


# ---------------------------------------------------------------------------
# bf16 dense matvec
# ---------------------------------------------------------------------------

def bf16_weights(shape_name):
    """(W bf16 bits, x, rows, cols, seed).  The LM head's 622M weights take
    minutes to draw on the host, so its timing input is its seed's first 8192
    rows repeated down the matrix (the same N(0, 0.02) bf16 values and
    layout); its parity test draws the whole matrix."""
    import workloads
    rows, cols, role, seed = {s[2]: s for s in workloads.BF16_SHAPES}[shape_name]
    if rows > 8192:
        W0, x = workloads.make_bf16(8192, cols, seed)
        return ("tile", W0), x, rows, cols, role
    W, x = workloads.make_bf16(rows, cols, seed)
    return ("full", W), x, rows, cols, role


def bf16_measure(shape_name, steps, warmup):
    import torch
    import group_quantized_moe_amd as gq
    L = gq.lib()
    (kind, W), x, rows, cols, role = bf16_weights(shape_name)
    nbytes = rows * cols * 2 + cols * 4 + rows * 4
    replicas = replica_count(rows * cols * 2)
    if kind == "tile":
        W0 = to_dev(W)
        Wd = W0.repeat(-(-rows // W0.shape[0]), 1)[:rows].contiguous()
        del W0
    else:
        Wd = to_dev(W)
    reps = [Wd] + [Wd.clone() for _ in range(replicas - 1)]
    xd = to_dev(x)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    stream, sp = stream_ptr()

    def step(i):
        rc = L.matvec_bf16(reps[i % replicas].data_ptr(), rows, cols, xd.data_ptr(), y.data_ptr(), None, 0, sp)
        if rc != 0:
            raise gq.SmoeError("matvec_bf16", rc)

    us, spread, wall = time_calls(step, steps, warmup, stream)
    return dict(W=W, kind=kind, x=x, rows=rows, cols=cols, role=role, nbytes=nbytes, replicas=replicas, us=us,
                spread=spread, wall=wall, gbs=nbytes / (us * 1e-6) / 1e9)


def bf16_row(shape_name, steps, warmup):
    m = bf16_measure(shape_name, steps, warmup)
    row = {"us": round(m["us"], 3), "gbs": round(m["gbs"], 1), "frac": round(m["gbs"] / PEAK_HBM_GBS, 4),
           "bound": "hbm", "per_call_us": m["spread"], "algorithmic_bytes": m["nbytes"],
           "replicas_rotated": m["replicas"]}
    rc = read_ceiling(m["nbytes"], steps, warmup)
    if rc:
        row["read_ceiling_us"] = rc["us"]
    row["kernels"] = row_kernels(f"bf16_{m['role']}", "bf16")
    if m["kind"] == "tile":
        row["note"] = "weights: the seed's first 8192 rows repeated (timing input)"
    return row


def bf16_line(args):
    m = bf16_measure(args.shape, args.steps, args.warmup)
    rows, cols, role, nbytes = m["rows"], m["cols"], m["role"], m["nbytes"]
    cpu = None
    if args.cpu_budget > 0 and m["kind"] == "full":
        import oracle
        W, x = m["W"], m["x"]
        n, dt, cores = cpu_oracle(lambda: oracle.matvec_bf16(W, x), args.cpu_budget)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole {rows}x{cols} matvecs (f64 oracle, {dt:.1f} s)", "cpu_model": cpu_model()}
    return {
        "metric": f"effective HBM GB/s of the bf16 matvec {rows}x{cols} ({role})",
        "value": round(m["gbs"], 1),
        "unit": "GB/s",
        "ms_per_step": round(m["us"] / 1e3, 6),
        "us_per_call": round(m["us"], 3),
        "per_call_us": m["spread"],
        "pct_of_hbm_peak": round(100.0 * m["gbs"] / PEAK_HBM_GBS, 2),
        "wall_us_per_step": round(m["wall"], 3),
        "dtype": "bf16 W (widened exactly) x f32 x -> f32 FMA",
        "config": {"workload": f"bf16_{role}_{rows}x{cols}", "rows": rows, "cols": cols,
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": m["replicas"],
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "unit_of_work": "one matvec_bf16 call (one launch)",
            "timing": "back-to-back calls between HIP events on the launch stream (the timing of value)",
            "achieved": round(m["gbs"], 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(m["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(f"bf16_{role}", "bf16"),
            "kernels": load_kernels(f"bf16_{role}", "bf16"),
        },
        "read_ceiling": read_ceiling(nbytes, args.steps, args.warmup),
        "cpu_baseline": cpu,
    }


def bf16_batch_line(args):
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
    stream, sp = stream_ptr()

    def step(i):
        rc = L.matvec_bf16_batch(arrays[i % replicas], len(jobs), sp)
        if rc != 0:
            raise gq.SmoeError("matvec_bf16_batch", rc)

    def step_separate(i):
        for w, y, (r, c, _, _) in zip(reps[i % replicas], ys, jobs):
            rc = L.matvec_bf16(w.data_ptr(), r, c, xd.data_ptr(), y.data_ptr(), None, 0, sp)
            if rc != 0:
                raise gq.SmoeError("matvec_bf16", rc)

    us, spread, wall = time_calls(step, args.steps, args.warmup, stream)
    us_sep, spread_sep, _ = time_calls(step_separate, args.steps, args.warmup, stream)
    gbs = nbytes / (us * 1e-6) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        n, dt, cores = cpu_oracle(lambda: [oracle.matvec_bf16(W, x) for W in Ws], args.cpu_budget)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole q/k/v batches (f64 oracle, {dt:.1f} s)", "cpu_model": cpu_model()}
    shapes = "+".join(f"{r}x{c}" for r, c, _, _ in jobs)
    return {
        "metric": f"effective HBM GB/s of one batched bf16 matvec launch ({shapes}, shared x)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "ms_per_step": round(us / 1e3, 6),
        "us_per_call": round(us, 3),
        "per_call_us": spread,
        "us_per_call_separate_launches": round(us_sep, 3),
        "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "wall_us_per_step": round(wall, 3),
        "dtype": "bf16 W (widened exactly) x f32 x -> f32 FMA",
        "config": {"workload": f"bf16_batch_qkv_{shapes}", "jobs": [list(j[:3]) for j in jobs],
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": replicas,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "unit_of_work": "one matvec_bf16_batch call (one launch)",
            "timing": "back-to-back calls between HIP events on the launch stream (the timing of value)",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": load_traffic("bf16_batch_qkv", "bf16"),
            "kernels": load_kernels("bf16_batch_qkv", "bf16"),
        },
        "cpu_baseline": cpu,
    }


def attn_line(args):
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
    stream, sp = stream_ptr()

    def step(i):
        r = i % replicas
        rc = L.smoe_attn_decode(ctypes.byref(structs[r]), dm, H, KV, hd, xd.data_ptr(), pos, spec["rope_base"],
                                reps[r][6].data_ptr(), reps[r][7].data_ptr(), ctx, out.data_ptr(), ws.data_ptr(),
                                ws.numel(), sp)
        if rc != 0:
            raise gq.SmoeError("smoe_attn_decode", rc)

    us, spread, wall = time_calls(step, args.steps, args.warmup, stream)
    gbs = nbytes / (us * 1e-6) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        n, dt, cores = cpu_oracle(lambda: oracle.attn_decode(w, x, pos, spec["rope_base"], K, V), args.cpu_budget)
        cpu = {"value": round(n * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n} whole attention blocks at position {pos} (f64 oracle, {dt:.1f} s)",
               "us_per_block": round(dt / n * 1e6, 1), "cpu_model": cpu_model()}
    return {
        "metric": "effective HBM GB/s per decode attention block (64/4 heads x 128, 4096-position f32 KV cache)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "ms_per_step": round(us / 1e3, 6),
        "us_per_block": round(us, 3),
        "per_call_us": spread,
        "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "wall_us_per_step": round(wall, 3),
        "dtype": "bf16 x f32 -> f32 projections, f32 attention",
        "config": {"workload": spec["name"], "d_model": dm, "n_head": H, "n_kv": KV, "head_dim": hd,
                   "max_ctx": ctx, "pos": pos, "rope_base": spec["rope_base"],
                   "algorithmic_bytes_per_step": nbytes, "replicas_rotated": replicas,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "unit_of_work": "one smoe_attn_decode call = qkv batch + partial (norm, rotation, append, chunk "
                            "attention) + combine + o_proj on one stream",
            "timing": "back-to-back calls between HIP events on the launch stream (the timing of value)",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": load_traffic("attn_decode", "attn"),
            "kernels": load_kernels("attn_decode", "attn"),
        },
        "cpu_baseline": cpu,
    }


def copy_line(args):
    """A plain device-to-device copy of 256 MiB (torch's copy kernel): the
    counter runs divide FETCH_SIZE / WRITE_SIZE of a kernel by what the same
    counters read for this copy of known size."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream, _ = stream_ptr()
    us, spread, wall = time_calls(lambda i: dst.copy_(src), args.steps, args.warmup, stream)
    return {"metric": "device-to-device copy of 256 MiB (counter calibration)",
            "value": round(2 * n / (us * 1e-6) / 1e9, 1), "unit": "GB/s (read + write)",
            "ms_per_step": round(us / 1e3, 6), "bytes_read": n, "bytes_written": n,
            "dtype": "u8", "config": {"workload": "copy_256MiB"}}


def collect_rows(args):
    """Every other workload of the path, each timed back to back in this run."""
    import workloads
    s, w = args.steps, args.warmup
    rows = {}

    def add(name, fn):
        t0 = time.perf_counter()
        rows[name] = fn()
        print(f"[bench] row {name}: {rows[name]['us']} us ({time.perf_counter() - t0:.1f} s)", file=sys.stderr,
              flush=True)

    add("decode_q4_tiny_1expert_256x512",
        lambda: decode_row(workloads.TINY, s, w, replicas=16, profile="tiny",
                           note="latency-bound: the 16 rotated replicas fit in the caches (hot)"))
    add("decode_q4_1expert_4096x1536",
        lambda: decode_row(workloads.Q4_GROUP8, s, w, n_experts=1, profile="decode_q4_e1"))
    add("decode_q2_8expert_4096x1536", lambda: decode_row(workloads.Q2_GROUP8, s, w, profile="decode_q2"))
    add("decode_q4_8expert_4096x1536_f16scales",
        lambda: decode_row(workloads.Q4_GROUP8_S16, s, w, profile="decode_q4_s16"))
    add("decode_q2_8expert_4096x1536_f16scales",
        lambda: decode_row(workloads.Q2_GROUP8_S16, s, w, profile="decode_q2_s16"))
    for rows_, cols, role, _ in workloads.BF16_SHAPES:
        add(f"bf16_{role}_{rows_}x{cols}", lambda role=role: bf16_row(role, s, w))
    for T in sorted(workloads.BATCH_TOKENS):
        add(f"prefill_q4_8expert_T{T}", lambda T=T: prefill_row(T, s, w))
    for T, k in ((16, 2), (256, 2)):
        add(f"routed_q4_8expert_T{T}_top{k}", lambda T=T, k=k: routed_row(T, k, s, w))
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "decode_q4", "decode_q2", "decode_q4_s16", "decode_q2_s16", "decode_q4_e1",
                             "tiny", "prefill", "bf16", "bf16_batch", "routed", "attn", "copy"])
    ap.add_argument("--tokens", type=int, default=16, help="prefill / routed: tokens per call")
    ap.add_argument("--topk", type=int, default=2, help="routed: experts per token")
    ap.add_argument("--shape", default="q_proj", help="bf16: q_proj, o_proj, kv_proj or lm_head")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline, all threads (half as much on one thread; "
                         "0 to skip)")
    ap.add_argument("--no-rows", action="store_true", help="headline: skip the other workloads' rows")
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
    wl = args.workload
    if wl == "headline":
        line = decode_line(args, workloads.Q4_GROUP8, "decode_q4", with_rows=not args.no_rows)
    elif wl.startswith("decode_") and wl != "decode_q4_e1":
        spec = {"decode_q4": workloads.Q4_GROUP8, "decode_q2": workloads.Q2_GROUP8,
                "decode_q4_s16": workloads.Q4_GROUP8_S16, "decode_q2_s16": workloads.Q2_GROUP8_S16}[wl]
        line = decode_line(args, spec, wl)
    elif wl in ("decode_q4_e1", "tiny"):
        spec = workloads.Q4_GROUP8 if wl == "decode_q4_e1" else workloads.TINY
        m = decode_measure(spec, args.steps, args.warmup, n_experts=1, replicas=16 if wl == "tiny" else None)
        line = {"metric": f"us per call, one Q4 expert ({spec['d_model']}x{spec['d_ff']}, decode)",
                "value": round(m["us"], 3), "unit": "us", "higher_is_better": False,
                "ms_per_step": round(m["us"] / 1e3, 6), "gbs": round(m["gbs"], 1), "per_call_us": m["spread"],
                "dtype": DECODE_DTYPE.format(bits=4),
                "config": {"workload": f"{spec['name']}_e1" if wl == "decode_q4_e1" else spec["name"],
                           "algorithmic_bytes_per_step": m["nbytes"], "replicas_rotated": m["replicas"]}}
    elif wl == "prefill":
        line = prefill_line(args)
    elif wl == "copy":
        line = copy_line(args)
    elif wl == "routed":
        line = routed_line(args)
    elif wl == "bf16_batch":
        line = bf16_batch_line(args)
    elif wl == "attn":
        line = attn_line(args)
    else:
        line = bf16_line(args)
    head = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded; stands in for trained weights)"}
    rest = {k: v for k, v in line.items() if k not in ("metric", "value", "unit")}
    head.update({k: rest.pop(k) for k in ("higher_is_better",) if k in rest})
    print(json.dumps({**{k: line[k] for k in ("metric", "value", "unit")}, **head, **rest}), flush=True)


if __name__ == "__main__":
    main()
