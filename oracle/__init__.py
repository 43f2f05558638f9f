"""ctypes front end of the f64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this module.  It shares no code with the GPU library
(``group_quantized_moe_amd``) and never imports it.

The arrays it takes are the host arrays produced by ``workloads``: packed code
bytes (uint8), f32 scales, f32 activations, bf16 bit patterns (uint16).  Every
result comes back as f64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (-O2, no fast-math, OpenMP over rows)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _QMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Expert(ctypes.Structure):
    _fields_ = [("gate", _QMat), ("up", _QMat), ("down", _QMat)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"oracle library not built: {LIB_PATH} (run oracle.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, l, i = ctypes.c_void_p, ctypes.c_long, ctypes.c_int
        L.oracle_threads.restype = i
        L.oracle_unpack.argtypes = [vp, i, l, l, vp]
        L.oracle_dequant.argtypes = [vp, vp, i, i, l, l, vp]
        L.oracle_qmatvec.argtypes = [vp, vp, i, i, l, l, vp, vp]
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_gate_up.argtypes = [vp, vp, i, i, l, l, vp, vp]
        L.oracle_down.argtypes = [vp, i, i, l, l, vp, vp]
        L.oracle_expert_ffn.argtypes = [vp, i, vp, i, i, l, l, l, vp, vp]
        L.oracle_matvec_bf16.argtypes = [vp, l, l, vp, vp]
        L.oracle_f16_widen.argtypes = [vp, l, vp]
        L.oracle_routed_ffn.argtypes = [vp, i, i, i, l, l, l, i, vp, vp, vp, vp]
        for name in ("oracle_routed_ffn", "oracle_f16_widen", "oracle_unpack", "oracle_dequant", "oracle_qmatvec", "oracle_gate_up",
                     "oracle_down", "oracle_expert_ffn", "oracle_matvec_bf16"):
            getattr(L, name).restype = i
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _ok(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: arguments outside the definitions (rc={rc})")


def threads() -> int:
    return lib().oracle_threads()


def unpack(codes, bits, rows, cols):
    codes, pc = _c(codes, np.uint8)
    out = np.empty((rows, cols), dtype=np.uint8)
    _ok(lib().oracle_unpack(pc, bits, rows, cols, out.ctypes.data_as(ctypes.c_void_p)), "unpack")
    return out


def dequant(codes, scales, bits, group, rows, cols):
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(_scales_f32(scales), np.float32)
    w = np.empty((rows, cols), dtype=np.float64)
    _ok(lib().oracle_dequant(pc, ps, bits, group, rows, cols,
                             w.ctypes.data_as(ctypes.c_void_p)), "dequant")
    return w


def qmatvec(codes, scales, bits, group, rows, cols, x):
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(_scales_f32(scales), np.float32)
    x, px = _c(x, np.float64)
    y = np.empty(rows, dtype=np.float64)
    _ok(lib().oracle_qmatvec(pc, ps, bits, group, rows, cols, px,
                             y.ctypes.data_as(ctypes.c_void_p)), "qmatvec")
    return y


def silu(t: float) -> float:
    return lib().oracle_silu(float(t))


def f16_widen(h):
    """f32 values of IEEE binary16 patterns (uint16 or float16 array), by the
    oracle's own decoder."""
    h = np.ascontiguousarray(h)
    bits = h.view(np.uint16) if h.dtype == np.float16 else h.astype(np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _ok(lib().oracle_f16_widen(bits.ctypes.data_as(ctypes.c_void_p), bits.size,
                               out.ctypes.data_as(ctypes.c_void_p)), "f16_widen")
    return out


def _scales_f32(scales):
    """A matrix's scales as f32: 2-byte (float16) scales are widened exactly."""
    return f16_widen(scales) if np.asarray(scales).dtype == np.float16 else scales


def _qmat_struct(m, keep):
    c, pc = _c(m.codes, np.uint8)
    s, ps = _c(_scales_f32(m.scales), np.float32)
    keep += [c, s]
    return _QMat(pc, ps)


def gate_up(expert, bits, group, d_ff, d_model, x):
    keep = []
    G, U = _qmat_struct(expert.gate, keep), _qmat_struct(expert.up, keep)
    x, px = _c(x, np.float32)
    h = np.empty(d_ff, dtype=np.float64)
    _ok(lib().oracle_gate_up(ctypes.byref(G), ctypes.byref(U), bits, group, d_ff, d_model,
                             px, h.ctypes.data_as(ctypes.c_void_p)), "gate_up")
    return h


def down(expert, bits, group, d_model, d_ff, hidden):
    keep = []
    D = _qmat_struct(expert.down, keep)
    hidden, ph = _c(hidden, np.float64)
    out = np.empty(d_model, dtype=np.float64)
    _ok(lib().oracle_down(ctypes.byref(D), bits, group, d_model, d_ff, ph,
                          out.ctypes.data_as(ctypes.c_void_p)), "down")
    return out


def expert_ffn(experts, bits, group, d_model, d_ff, x, route_w=None):
    """x: f32 [T, d_model] (or [d_model]); route_w: f32 [T, n_experts] or None (all ones).

    Returns f64 [T, d_model] (or [d_model] when x is one vector)."""
    keep = []
    arr = (_Expert * len(experts))()
    for k, e in enumerate(experts):
        arr[k] = _Expert(_qmat_struct(e.gate, keep), _qmat_struct(e.up, keep),
                         _qmat_struct(e.down, keep))
    x = np.asarray(x, dtype=np.float32)
    single = x.ndim == 1
    X, px = _c(x.reshape(-1, d_model), np.float32)
    T = X.shape[0]
    pr = None
    if route_w is not None:
        R, pr = _c(np.asarray(route_w, dtype=np.float32).reshape(T, len(experts)), np.float32)
        keep.append(R)
    out = np.empty((T, d_model), dtype=np.float64)
    _ok(lib().oracle_expert_ffn(arr, len(experts), pr, bits, group, d_model, d_ff, T, px,
                                out.ctypes.data_as(ctypes.c_void_p)), "expert_ffn")
    return out[0] if single else out


def routed_ffn(experts, bits, group, d_model, d_ff, x, ids, w):
    """x f32 [T, d_model]; ids int32 [T, top_k] (expert of each slot); w f32 [T, top_k].
    Returns f64 [T, d_model]: per token, the router-weighted sum of its slots'
    expert FFNs (slots with an id outside [0, n_experts) add nothing)."""
    keep = []
    arr = (_Expert * len(experts))()
    for k, e in enumerate(experts):
        arr[k] = _Expert(_qmat_struct(e.gate, keep), _qmat_struct(e.up, keep),
                         _qmat_struct(e.down, keep))
    X, px = _c(np.asarray(x, dtype=np.float32).reshape(-1, d_model), np.float32)
    T = X.shape[0]
    I, pi = _c(np.asarray(ids).reshape(T, -1), np.int32)
    W, pw = _c(np.asarray(w).reshape(T, -1), np.float32)
    out = np.empty((T, d_model), dtype=np.float64)
    _ok(lib().oracle_routed_ffn(arr, len(experts), bits, group, d_model, d_ff, T, I.shape[1], pi, pw, px,
                                out.ctypes.data_as(ctypes.c_void_p)), "routed_ffn")
    return out


def matvec_bf16(W, x):
    W, pw = _c(W, np.uint16)
    rows, cols = W.shape
    x, px = _c(x, np.float32)
    y = np.empty(rows, dtype=np.float64)
    _ok(lib().oracle_matvec_bf16(pw, rows, cols, px, y.ctypes.data_as(ctypes.c_void_p)),
        "matvec_bf16")
    return y
