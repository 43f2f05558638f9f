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
        L.oracle_set_threads.argtypes = [i]
        L.oracle_set_threads.restype = None
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
        d = ctypes.c_double
        L.oracle_head_rmsnorm.argtypes = [vp, l, l, vp, d, vp]
        L.oracle_rope.argtypes = [vp, l, l, l, d]
        L.oracle_gqa_attend.argtypes = [vp, l, l, l, vp, vp, l, l, vp]
        L.oracle_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, l, l, l, l, vp, l, d, vp, vp, l, vp, vp, vp]
        for name in ("oracle_routed_ffn", "oracle_f16_widen", "oracle_unpack", "oracle_dequant", "oracle_qmatvec", "oracle_gate_up",
                     "oracle_down", "oracle_expert_ffn", "oracle_matvec_bf16", "oracle_head_rmsnorm", "oracle_rope",
                     "oracle_gqa_attend", "oracle_attn_decode"):
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


def set_threads(n: int) -> None:
    """Threads of the oracle's row loops from now on (results do not depend on it)."""
    lib().oracle_set_threads(int(n))


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


# ---------------------------------------------------------------------------
# Decode attention block (Metal Compute Kernels page of the S-MoE docs,
# section "GPU-Resident Decode Attention").

def head_rmsnorm(x, w, eps=1e-6):
    """x: [n_heads, hd]; w: f32 [hd].  y[h] = x[h] / sqrt(mean(x[h]^2) + eps) * w."""
    X, px = _c(np.asarray(x, dtype=np.float64), np.float64)
    n_heads, hd = X.shape
    W, pw = _c(w, np.float32)
    y = np.empty_like(X)
    _ok(lib().oracle_head_rmsnorm(px, n_heads, hd, pw, eps, y.ctypes.data_as(ctypes.c_void_p)), "head_rmsnorm")
    return y


def rope(x, pos, base):
    """x: [n_heads, hd]; returns a rotated copy (pair (i, i + hd/2), angle pos * base^(-2i/hd))."""
    X = np.array(x, dtype=np.float64, order="C", copy=True)
    n_heads, hd = X.shape
    _ok(lib().oracle_rope(X.ctypes.data_as(ctypes.c_void_p), n_heads, hd, pos, base), "rope")
    return X


def gqa_attend(q, K, V, n_ctx):
    """q: [n_head, hd]; K, V: f32 [n_kv, ctx_stride, hd].  Returns att f64 [n_head, hd]."""
    Q, pq = _c(np.asarray(q, dtype=np.float64), np.float64)
    n_head, hd = Q.shape
    Kc, pk = _c(K, np.float32)
    Vc, pv = _c(V, np.float32)
    n_kv, stride, _ = Kc.shape
    att = np.empty((n_head, hd), dtype=np.float64)
    _ok(lib().oracle_gqa_attend(pq, n_head, n_kv, hd, pk, pv, stride, n_ctx, att.ctypes.data_as(ctypes.c_void_p)),
        "gqa_attend")
    return att


def attn_decode(w, x, pos, rope_base, k_cache, v_cache):
    """One token of the decode attention block.

    w: object with wq, wk, wv, wo (uint16 bf16 patterns) and q_norm, k_norm (f32);
    x f32 [d_model]; k_cache, v_cache f32 [n_kv, ctx_stride, hd] (not modified:
    the oracle works on copies).  Returns (out f64 [d_model], q_rot f64
    [n_head, hd], att f64 [n_head, hd], k_cache', v_cache') where the primed
    caches are copies with row pos written."""
    keep = []
    def arr(a, dt):
        A, p = _c(a, dt)
        keep.append(A)
        return A, p
    Kc = np.array(k_cache, dtype=np.float32, order="C", copy=True)
    Vc = np.array(v_cache, dtype=np.float32, order="C", copy=True)
    n_kv, stride, hd = Kc.shape
    Wq, pq = arr(w.wq, np.uint16)
    _, pk = arr(w.wk, np.uint16)
    _, pv = arr(w.wv, np.uint16)
    Wo, po = arr(w.wo, np.uint16)
    _, pqn = arr(w.q_norm, np.float32)
    _, pkn = arr(w.k_norm, np.float32)
    X, px = arr(x, np.float32)
    d_model = X.shape[0]
    n_head = Wq.shape[0] // hd
    out = np.empty(d_model, dtype=np.float64)
    q_rot = np.empty((n_head, hd), dtype=np.float64)
    att = np.empty((n_head, hd), dtype=np.float64)
    vpp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _ok(lib().oracle_attn_decode(pq, pk, pv, po, pqn, pkn, d_model, n_head, n_kv, hd, px, pos, float(rope_base),
                                 vpp(Kc), vpp(Vc), stride, vpp(out), vpp(q_rot), vpp(att)), "attn_decode")
    return out, q_rot, att, Kc, Vc
