"""Python binding of libsmoe.so (group-quantised routed-expert FFN decode path
and bf16 matvec on MI355X).

Argument marshalling only: every function takes torch tensors that live on the
GPU, checks dtype / device / contiguity, reads sizes off the tensor shapes, and
passes raw device pointers plus the current HIP stream to the C function of
the same name (declared in include/smoe.h).  No step of the computation runs
here.  If the library is missing the first call raises; nothing falls back.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmoe.so")

SMOE_OK = 0
SMOE_MAX_EXPERTS = 16
SMOE_SCALE_F16 = 0x100   # ORed into `bits`: 2-byte IEEE binary16 scales instead of f32
SMOE_NOALLOC_SCRATCH_BYTES = 1 << 20

EXPORTS = ("smoe_gate_up", "smoe_down", "smoe_expert_ffn_workspace", "smoe_expert_ffn", "smoe_expert_ffn_noalloc",
           "matvec_bf16_workspace", "matvec_bf16", "matvec_bf16_batch", "smoe_routed_ffn_workspace",
           "smoe_routed_ffn", "smoe_attn_decode_workspace", "smoe_attn_decode", "smoe_status_str")
SMOE_MAX_BF16_JOBS = 16
SMOE_MAX_ATTN_GROUP = 16


class SmoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {smoe_status_str(status)} (status {status})")


class QMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Expert(ctypes.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat)]


class AttnWeights(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("wv", ctypes.c_void_p),
                ("wo", ctypes.c_void_p), ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p)]


class Bf16Job(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("rows", ctypes.c_int), ("cols", ctypes.c_int)]


_lib = None


def lib():
    """The loaded libsmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libsmoe.so is not built ({LIB_PATH}); run "
                               "`python -m group_quantized_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.smoe_gate_up.argtypes = [vp, vp, i, i, i, i, vp, vp, vp]
        L.smoe_down.argtypes = [vp, i, i, i, i, vp, vp, vp]
        L.smoe_expert_ffn_workspace.argtypes = [i, i, i, i]
        L.smoe_expert_ffn_workspace.restype = sz
        L.smoe_expert_ffn.argtypes = [vp, i, vp, i, i, i, i, i, vp, vp, vp, sz, vp]
        L.smoe_expert_ffn_noalloc.argtypes = [vp, i, vp, i, i, i, i, i, vp, vp, vp]
        L.matvec_bf16_workspace.argtypes = [i, i]
        L.matvec_bf16_workspace.restype = sz
        L.matvec_bf16.argtypes = [vp, i, i, vp, vp, vp, sz, vp]
        L.matvec_bf16_batch.argtypes = [vp, i, vp]
        L.smoe_routed_ffn_workspace.argtypes = [i, i, i, i, i]
        L.smoe_routed_ffn_workspace.restype = sz
        L.smoe_routed_ffn.argtypes = [vp, i, i, i, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]
        L.smoe_attn_decode_workspace.argtypes = [i, i, i, i, i]
        L.smoe_attn_decode_workspace.restype = sz
        L.smoe_attn_decode.argtypes = [vp, i, i, i, i, vp, i, ctypes.c_double, vp, vp, i, vp, vp, sz, vp]
        L.smoe_attn_decode.restype = i
        L.smoe_status_str.argtypes = [i]
        L.smoe_status_str.restype = ctypes.c_char_p
        for name in ("smoe_gate_up", "smoe_down", "smoe_expert_ffn", "smoe_expert_ffn_noalloc", "matvec_bf16"):
            getattr(L, name).restype = i
        _lib = L
    return _lib


def smoe_status_str(status: int) -> str:
    return lib().smoe_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != SMOE_OK:
        raise SmoeError(fn, status)


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _qmat(codes, scales, name, bits):
    """Scales must be float16 when `bits` carries SMOE_SCALE_F16, else float32."""
    import torch
    sdt = torch.float16 if bits & SMOE_SCALE_F16 else torch.float32
    return QMat(_dev(codes, torch.uint8, name + ".codes"), _dev(scales, sdt, name + ".scales"))


def _dims(codes, bits):
    """(rows, cols) of a packed matrix [rows, cols*bits/8]."""
    return codes.shape[0], codes.shape[1] * 8 // (bits & ~SMOE_SCALE_F16)


def smoe_gate_up(gate_codes, gate_scales, up_codes, up_scales, bits, group, x, hidden, stream=None):
    """hidden[d_ff] = SiLU(G x) * (U x); G, U packed [d_ff, d_model*bits/8]."""
    import torch
    d_ff, d_model = _dims(gate_codes, bits)
    G, U = _qmat(gate_codes, gate_scales, "gate", bits), _qmat(up_codes, up_scales, "up", bits)
    _check("smoe_gate_up", lib().smoe_gate_up(
        ctypes.byref(G), ctypes.byref(U), bits, group, d_ff, d_model,
        _dev(x, torch.float32, "x"), _dev(hidden, torch.float32, "hidden"), _stream(stream)))


def smoe_down(down_codes, down_scales, bits, group, hidden, out, stream=None):
    """out[d_model] = D hidden; D packed [d_model, d_ff*bits/8]."""
    import torch
    d_model, d_ff = _dims(down_codes, bits)
    D = _qmat(down_codes, down_scales, "down", bits)
    _check("smoe_down", lib().smoe_down(
        ctypes.byref(D), bits, group, d_model, d_ff, _dev(hidden, torch.float32, "hidden"),
        _dev(out, torch.float32, "out"), _stream(stream)))


def smoe_expert_ffn_workspace(n_experts, d_model, d_ff, T=1) -> int:
    return int(lib().smoe_expert_ffn_workspace(n_experts, d_model, d_ff, T))


def _expert_array(experts, bits=4):
    """experts: sequence of objects with .gate/.up/.down, each with .codes/.scales
    (torch GPU tensors), or 6-tuples (gc, gs, uc, us, dc, ds); scales float16
    when `bits` carries SMOE_SCALE_F16, else float32."""
    arr = (Expert * len(experts))()
    for k, e in enumerate(experts):
        if isinstance(e, (tuple, list)):
            gc, gs, uc, us, dc, ds = e
        else:
            gc, gs, uc, us, dc, ds = (e.gate.codes, e.gate.scales, e.up.codes, e.up.scales,
                                      e.down.codes, e.down.scales)
        arr[k] = Expert(_qmat(gc, gs, f"experts[{k}].gate", bits), _qmat(uc, us, f"experts[{k}].up", bits),
                        _qmat(dc, ds, f"experts[{k}].down", bits))
    return arr


def _first_gate_codes(experts):
    e = experts[0]
    return e[0] if isinstance(e, (tuple, list)) else e.gate.codes


def smoe_expert_ffn(experts, bits, group, x, out, route_w=None, workspace=None, stream=None):
    """out[T, d_model] = sum_e route_w[t, e] * FFN_e(x[t]).

    x, out: f32 [T, d_model] (or [d_model] for one token); route_w: f32 [T, n] or None;
    workspace: uint8 GPU tensor of at least smoe_expert_ffn_workspace(...) bytes."""
    import torch
    d_ff, d_model = _dims(_first_gate_codes(experts), bits)
    T = x.numel() // d_model
    arr = _expert_array(experts, bits)
    pr = None if route_w is None else _dev(route_w, torch.float32, "route_w")
    if workspace is None:
        raise ValueError("smoe_expert_ffn needs a caller-owned workspace tensor")
    pw = _dev(workspace, torch.uint8, "workspace")
    _check("smoe_expert_ffn", lib().smoe_expert_ffn(
        arr, len(experts), pr, bits, group, d_model, d_ff, T, _dev(x, torch.float32, "x"),
        _dev(out, torch.float32, "out"), pw, workspace.numel(), _stream(stream)))


def smoe_expert_ffn_noalloc(experts, bits, group, x, out, route_w=None, stream=None):
    """smoe_expert_ffn on the library's static per-GPU scratch array: no
    workspace, nothing allocated.  Calls that may overlap on one GPU race."""
    import torch
    d_ff, d_model = _dims(_first_gate_codes(experts), bits)
    T = x.numel() // d_model
    arr = _expert_array(experts, bits)
    pr = None if route_w is None else _dev(route_w, torch.float32, "route_w")
    _check("smoe_expert_ffn_noalloc", lib().smoe_expert_ffn_noalloc(
        arr, len(experts), pr, bits, group, d_model, d_ff, T, _dev(x, torch.float32, "x"),
        _dev(out, torch.float32, "out"), _stream(stream)))


def matvec_bf16_workspace(rows, cols) -> int:
    return int(lib().matvec_bf16_workspace(rows, cols))


def matvec_bf16(W, x, y, workspace=None, stream=None):
    """y[rows] = W x with W bf16 [rows, cols] (torch.bfloat16 or raw int16 bits)."""
    import torch
    if W.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError("W must be torch.bfloat16 (or int16 bit patterns)")
    rows, cols = W.shape
    _dev(W, W.dtype, "W")
    pw, nw = (None, 0) if workspace is None else (_dev(workspace, torch.uint8, "workspace"),
                                                    workspace.numel())
    _check("matvec_bf16", lib().matvec_bf16(
        W.data_ptr(), rows, cols, _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"),
        pw, nw, _stream(stream)))


def bf16_job_array(jobs):
    """ctypes array of smoe_bf16_job from (W, x, y) torch tensors (W bf16 or
    int16 bit patterns [rows, cols], x f32 [cols], y f32 [rows])."""
    import torch
    arr = (Bf16Job * len(jobs))()
    for j, (W, x, y) in enumerate(jobs):
        if W.dtype not in (torch.bfloat16, torch.int16):
            raise TypeError("W must be torch.bfloat16 (or int16 bit patterns)")
        rows, cols = W.shape
        arr[j] = Bf16Job(_dev(W, W.dtype, "W"), _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"),
                         rows, cols)
    return arr


def matvec_bf16_batch(jobs, stream=None):
    """y_j = W_j x_j for a list of (W, x, y) tensor triples, in one launch."""
    arr = bf16_job_array(jobs)
    _check("matvec_bf16_batch", lib().matvec_bf16_batch(arr, len(jobs), _stream(stream)))


def smoe_routed_ffn_workspace(n_experts, d_model, d_ff, T, top_k) -> int:
    return int(lib().smoe_routed_ffn_workspace(n_experts, d_model, d_ff, T, top_k))


def smoe_routed_ffn(experts, bits, group, x, expert_ids, expert_w, out, workspace, stream=None):
    """out[T, d_model] = per token, sum over its top_k slots of w * FFN_id(x[t]).

    expert_ids: int32 [T, top_k] GPU tensor; expert_w: f32 [T, top_k]; x, out: f32 [T, d_model];
    workspace: uint8 GPU tensor of at least smoe_routed_ffn_workspace(...) bytes."""
    import torch
    d_ff, d_model = _dims(_first_gate_codes(experts), bits)
    T, top_k = expert_ids.shape
    arr = _expert_array(experts, bits)
    _check("smoe_routed_ffn", lib().smoe_routed_ffn(
        arr, len(experts), bits, group, d_model, d_ff, T, top_k, _dev(expert_ids, torch.int32, "expert_ids"),
        _dev(expert_w, torch.float32, "expert_w"), _dev(x, torch.float32, "x"), _dev(out, torch.float32, "out"),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def smoe_attn_decode_workspace(d_model, n_head, n_kv, head_dim, max_ctx) -> int:
    return int(lib().smoe_attn_decode_workspace(d_model, n_head, n_kv, head_dim, max_ctx))


def _bf16(t, name):
    import torch
    if t.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError(f"{name} must be torch.bfloat16 (or int16 bit patterns)")
    return _dev(t, t.dtype, name)


def smoe_attn_decode(wq, wk, wv, wo, q_norm, k_norm, x, pos, rope_base, k_cache, v_cache, out, workspace,
                     stream=None):
    """One token's decode attention block; appends k, v at `pos` in the caches.

    wq [n_head*hd, d_model], wk/wv [n_kv*hd, d_model], wo [d_model, n_head*hd]: bf16;
    q_norm, k_norm f32 [hd]; x, out f32 [d_model]; k_cache, v_cache f32
    [n_kv, max_ctx, hd]; workspace uint8 of smoe_attn_decode_workspace(...) bytes."""
    import torch
    n_kv, max_ctx, hd = k_cache.shape
    d_model = x.numel()
    n_head = wq.shape[0] // hd
    w = AttnWeights(_bf16(wq, "wq"), _bf16(wk, "wk"), _bf16(wv, "wv"), _bf16(wo, "wo"),
                    _dev(q_norm, torch.float32, "q_norm"), _dev(k_norm, torch.float32, "k_norm"))
    _check("smoe_attn_decode", lib().smoe_attn_decode(
        ctypes.byref(w), d_model, n_head, n_kv, hd, _dev(x, torch.float32, "x"), int(pos), float(rope_base),
        _dev(k_cache, torch.float32, "k_cache"), _dev(v_cache, torch.float32, "v_cache"), max_ctx,
        _dev(out, torch.float32, "out"), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))
