"""Pins for the f64 oracle that do not depend on the oracle itself.

Each check compares what a given build of ``oracle.c`` returns with something
fixed outside it: hand-worked closed forms (``golden/``), exact rational
arithmetic through the page's per-group affine identity, an independent
bit-level unpacker, IEEE bf16 bit patterns, and mathematical identities of
SiLU.  The checks take a ``ctypes.CDLL`` so that the same pins can be run on
deliberately broken copies of the oracle (see ``test_oracle_mutants.py``).

Sources: Metal Compute Kernels (S-MoE docs), sections "Fused FFN Kernels --
One Simdgroup Per Output Row" (affine codes, Z, group scales, SiLU(gate)*up,
down projection), "Layout assumptions the kernels rely on" (group and chunk
contract), "Coalesced Dense Matvec -- the Same Contract for bf16" and
"GPU-Resident Decode Attention" (QK RMS norm, RoPE, KV append, GQA attention).
"""
from __future__ import annotations

import ctypes
import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

vp, cl, ci = ctypes.c_void_p, ctypes.c_long, ctypes.c_int


def bind(L):
    L.oracle_unpack.argtypes = [vp, ci, cl, cl, vp]
    L.oracle_qmatvec.argtypes = [vp, vp, ci, ci, cl, cl, vp, vp]
    L.oracle_silu.argtypes = [ctypes.c_double]
    L.oracle_silu.restype = ctypes.c_double
    L.oracle_gate_up.argtypes = [vp, vp, ci, ci, cl, cl, vp, vp]
    L.oracle_down.argtypes = [vp, ci, ci, cl, cl, vp, vp]
    L.oracle_expert_ffn.argtypes = [vp, ci, vp, ci, ci, cl, cl, cl, vp, vp]
    L.oracle_matvec_bf16.argtypes = [vp, cl, cl, vp, vp]
    L.oracle_f16_widen.argtypes = [vp, cl, vp]
    L.oracle_routed_ffn.argtypes = [vp, ci, ci, ci, cl, cl, cl, ci, vp, vp, vp, vp]
    cd = ctypes.c_double
    L.oracle_head_rmsnorm.argtypes = [vp, cl, cl, vp, cd, vp]
    L.oracle_rope.argtypes = [vp, cl, cl, cl, cd]
    L.oracle_gqa_attend.argtypes = [vp, cl, cl, cl, vp, vp, cl, cl, vp]
    L.oracle_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, cl, cl, cl, cl, vp, cl, cd, vp, vp, cl, vp, vp, vp]
    return L


def _p(a):
    return a.ctypes.data_as(vp)


class _QMat(ctypes.Structure):
    _fields_ = [("codes", vp), ("scales", vp)]


class _Expert(ctypes.Structure):
    _fields_ = [("gate", _QMat), ("up", _QMat), ("down", _QMat)]


def qmatvec(L, codes, scales, bits, group, x):
    rows = codes.shape[0]
    cols = codes.shape[1] * 8 // bits
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty(rows, np.float64)
    rc = L.oracle_qmatvec(_p(codes), _p(scales), bits, group, rows, cols, _p(x), _p(y))
    assert rc == 0
    return y


def unpack(L, codes, bits):
    rows = codes.shape[0]
    cols = codes.shape[1] * 8 // bits
    codes = np.ascontiguousarray(codes, np.uint8)
    out = np.empty((rows, cols), np.uint8)
    assert L.oracle_unpack(_p(codes), bits, rows, cols, _p(out)) == 0
    return out


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """Independent packer for test inputs: lay each code's bits out LSB first
    and let numpy pack the bit stream little-endian within each byte."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    bitplanes = ((codes[..., None] >> np.arange(bits, dtype=np.uint8)) & 1).astype(np.uint8)
    return np.packbits(bitplanes.reshape(rows, cols * bits), axis=1, bitorder="little")


def unpack_bits(packed: np.ndarray, bits: int) -> np.ndarray:
    """Independent unpacker: explode bytes to bits (LSB first), regroup."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    stream = np.unpackbits(packed, axis=1, bitorder="little").reshape(rows, -1, bits)
    weights = (1 << np.arange(bits)).astype(np.uint8)
    return (stream * weights).sum(axis=2).astype(np.uint8)


def affine_exact(codes: np.ndarray, scales, bits: int, group: int, x) -> list:
    """Row dot products in exact rationals through the page's per-group
    identity: sum_j w_j x_j = sum_g s_g * ((sum_{j in g} code_j x_j) / Z - sum_{j in g} x_j)."""
    Z = Fraction(15, 2) if bits == 4 else Fraction(3, 2)
    xs = [Fraction(float(v)) for v in x]
    out = []
    for r in range(codes.shape[0]):
        total = Fraction(0)
        for g in range(codes.shape[1] // group):
            cols = range(g * group, (g + 1) * group)
            cx = sum(int(codes[r, j]) * xs[j] for j in cols)
            sx = sum(xs[j] for j in cols)
            total += Fraction(float(scales[r][g])) * (cx / Z - sx)
        out.append(total)
    return out


def load_worked_examples():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)["examples"]


def load_bf16_patterns():
    with open(os.path.join(GOLDEN, "bf16_patterns.json")) as f:
        return json.load(f)["patterns"]


# --------------------------------------------------------------------------
# Core pins, each returning a list of failure strings (empty = pass).
# --------------------------------------------------------------------------

def pin_worked_examples(L):
    fails = []
    for ex in load_worked_examples():
        bits = ex["bits"]
        packed = np.array([list(bytes.fromhex(h)) for h in ex["packed_hex"]], np.uint8)
        codes = np.array(ex["codes"], np.uint8)
        if not np.array_equal(unpack(L, packed, bits), codes):
            fails.append(f"{ex['name']}: unpacked codes differ from the hand-packed bytes")
        y = qmatvec(L, packed, np.array(ex["scales"], np.float32), bits, ex["group"],
                    np.array(ex["x"], np.float64))
        for r, e in enumerate(ex["expected"]):
            want = float(Fraction(e))
            if abs(y[r] - want) > 8 * np.finfo(np.float64).eps * max(1.0, abs(want)):
                fails.append(f"{ex['name']} row {r}: {y[r]!r} != {e}")
    return fails


def pin_unpack_exhaustive(L):
    """Every code value at every in-byte position, against the bit-level unpacker."""
    fails = []
    for bits in (4, 2):
        per = 8 // bits
        allbytes = np.arange(256, dtype=np.uint8).reshape(1, 256)
        got = unpack(L, allbytes, bits)
        want = unpack_bits(allbytes, bits)
        if not np.array_equal(got, want):
            fails.append(f"Q{bits}: unpack disagrees with bit-level unpack")
        # each code value alone at each position, others zero
        for pos in range(per):
            for v in range(1 << bits):
                codes = np.zeros((1, 2 * per), np.uint8)
                codes[0, per + pos] = v
                if not np.array_equal(unpack(L, pack_bits(codes, bits), bits), codes):
                    fails.append(f"Q{bits}: value {v} at position {pos} not recovered")
    return fails


def pin_affine_identity(L, seed=7):
    """Random tiny matrices with dyadic scales and dyadic x: the oracle's f64
    explicit-dequant sum must equal the exact rational affine-epilogue value
    to within the f64 rounding of its own sum."""
    rng = np.random.default_rng(seed)
    fails = []
    for bits, rows, cols, group in ((4, 3, 128, 64), (4, 4, 256, 64), (2, 3, 128, 64),
                                    (2, 2, 256, 128), (4, 2, 96, 32)):
        codes = rng.integers(0, 1 << bits, size=(rows, cols), dtype=np.uint8)
        scales = (rng.integers(1, 64, size=(rows, cols // group)) / 1024.0).astype(np.float32)
        x = rng.integers(-512, 512, size=cols) / 128.0
        y = qmatvec(L, pack_bits(codes, bits), scales, bits, group, x)
        exact = affine_exact(codes, scales, bits, group, x)
        Z = 7.5 if bits == 4 else 1.5
        for r in range(rows):
            mag = sum(abs((int(c) - Z) / Z * float(scales[r][j // group]) * x[j])
                      for j, c in enumerate(codes[r]))
            bound = 4 * cols * np.finfo(np.float64).eps * max(mag, 1e-300)
            if abs(y[r] - float(exact[r])) > bound:
                fails.append(f"Q{bits} {rows}x{cols} g{group} row {r}: "
                             f"{y[r]!r} vs exact {float(exact[r])!r}")
    return fails


def pin_silu(L):
    """SiLU(t) = t * sigmoid(t): SiLU(ln 3) = (3/4) ln 3 and SiLU(-ln 3) = -(1/4) ln 3
    because sigmoid(ln 3) = 3/4; SiLU(0) = 0; SiLU(t) - SiLU(-t) = t; SiLU(t) -> t for
    large t and -> 0 for very negative t."""
    fails = []
    s = L.oracle_silu
    ln3 = math.log(3.0)
    checks = [(s(ln3), 0.75 * ln3), (s(-ln3), -0.25 * ln3), (s(0.0), 0.0),
              (s(40.0), 40.0), (s(-800.0), 0.0)]
    for got, want in checks:
        if abs(got - want) > 4e-16 * max(1.0, abs(want)):
            fails.append(f"silu: {got!r} != {want!r}")
    for t in (0.1, 0.5, 1.0, 2.5, 7.0):
        if abs((s(t) - s(-t)) - t) > 4e-16 * max(1.0, t):
            fails.append(f"silu({t}) - silu(-{t}) != {t}")
    return fails


def pin_bf16(L):
    """IEEE bf16 patterns widen exactly; small-integer rows sum exactly."""
    fails = []
    pats = load_bf16_patterns()
    W = np.array([[int(p["bits"], 16)] for p in pats], np.uint16)
    x = np.ones(1, np.float32)
    y = np.empty(len(pats), np.float64)
    assert L.oracle_matvec_bf16(_p(W), len(pats), 1, _p(x), _p(y)) == 0
    for p, v in zip(pats, y):
        if v != float(p["value"]):
            fails.append(f"bf16 {p['bits']}: {v!r} != {p['value']}")
    # integers -8..8 are exact in bf16 (bits = f32 bits >> 16); with integer x the
    # dot product is an exact integer
    rng = np.random.default_rng(3)
    ints = rng.integers(-8, 9, size=(5, 64)).astype(np.float32)
    Wi = (ints.view(np.uint32) >> 16).astype(np.uint16)
    xi = rng.integers(-100, 101, size=64).astype(np.float32)
    yi = np.empty(5, np.float64)
    assert L.oracle_matvec_bf16(_p(Wi), 5, 64, _p(xi), _p(yi)) == 0
    want = ints.astype(np.int64) @ xi.astype(np.int64)
    if not np.array_equal(yi, want.astype(np.float64)):
        fails.append("bf16 integer matvec not exact")
    return fails


def load_f16_patterns():
    with open(os.path.join(GOLDEN, "f16_patterns.json")) as f:
        return json.load(f)["patterns"]


def pin_f16(L):
    """2-byte scales: IEEE binary16 patterns worked by hand widen to their
    values, and all 65536 patterns agree with numpy's binary16 (NaN for NaN)."""
    fails = []
    pats = load_f16_patterns()
    h = np.array([int(p["bits"], 16) for p in pats], np.uint16)
    out = np.empty(len(pats), np.float32)
    assert L.oracle_f16_widen(_p(h), len(pats), _p(out)) == 0
    for p, v in zip(pats, out):
        want = float(p["value"])
        if not (v == want and np.signbit(v) == np.signbit(want)):
            fails.append(f"f16 {p['bits']}: {v!r} != {p['value']}")
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = np.empty(allh.size, np.float32)
    assert L.oracle_f16_widen(_p(allh), allh.size, _p(got)) == 0
    ref = allh.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    if not (np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))):
        fails.append("f16 widening differs from numpy's binary16 on some pattern")
    return fails


def make_expert(rng, d_model, d_ff, bits, group):
    def m(rows, cols):
        codes = rng.integers(0, 1 << bits, size=(rows, cols), dtype=np.uint8)
        scales = rng.uniform(0.01, 0.05, size=(rows, cols // group)).astype(np.float32)
        return pack_bits(codes, bits), scales
    return dict(gate=m(d_ff, d_model), up=m(d_ff, d_model), down=m(d_model, d_ff))


def expert_struct(experts):
    arr = (_Expert * len(experts))()
    for k, e in enumerate(experts):
        arr[k] = _Expert(*[_QMat(_p(e[n][0]), _p(e[n][1])) for n in ("gate", "up", "down")])
    return arr


def ffn(L, experts, bits, group, d_model, d_ff, X, R=None):
    X = np.ascontiguousarray(X, np.float32).reshape(-1, d_model)
    T = X.shape[0]
    out = np.empty((T, d_model), np.float64)
    pr = None
    if R is not None:
        R = np.ascontiguousarray(R, np.float32).reshape(T, len(experts))
        pr = _p(R)
    arr = expert_struct(experts)
    assert L.oracle_expert_ffn(arr, len(experts), pr, bits, group, d_model, d_ff, T,
                               _p(X), _p(out)) == 0
    return out


def numpy_ffn_one(e, bits, group, x):
    """Independent route: bit-level unpack, vectorised dequant, BLAS products."""
    Z = 7.5 if bits == 4 else 1.5

    def W(name):
        packed, scales = e[name]
        c = unpack_bits(packed, bits).astype(np.float64)
        s = np.repeat(scales.astype(np.float64), group, axis=1)
        return (c - Z) / Z * s
    x = np.asarray(x, np.float64)
    g, u = W("gate") @ x, W("up") @ x
    h = g / (1.0 + np.exp(-g)) * u
    return W("down") @ h


def pin_ffn_composition(L, seed=11):
    """Multi-expert, multi-token FFN against the BLAS route, the router-weighted
    combine, and the one-hot / zero-scale special cases."""
    fails = []
    rng = np.random.default_rng(seed)
    for bits in (4, 2):
        d_model, d_ff, group = 128, 192, 64
        exps = [make_expert(rng, d_model, d_ff, bits, group) for _ in range(3)]
        X = rng.standard_normal((2, d_model)).astype(np.float32)
        R = rng.uniform(0.1, 1.0, size=(2, 3)).astype(np.float32)
        out = ffn(L, exps, bits, group, d_model, d_ff, X, R)
        for t in range(2):
            want = sum(float(R[t, k]) * numpy_ffn_one(exps[k], bits, group, X[t]) for k in range(3))
            err = np.max(np.abs(out[t] - want)) / max(1.0, np.max(np.abs(want)))
            if err > 1e-12:
                fails.append(f"Q{bits} token {t}: FFN vs BLAS route rel err {err:.3g}")
        onehot = np.zeros((2, 3), np.float32)
        onehot[:, 0] = 1.0
        sel = ffn(L, exps, bits, group, d_model, d_ff, X, onehot)
        solo = ffn(L, exps[:1], bits, group, d_model, d_ff, X, None)
        if not np.array_equal(sel, solo):
            fails.append(f"Q{bits}: one-hot router does not select expert 0")
        # zero up-projection scales: hidden = SiLU(g) * 0 = 0, so the output is 0
        z = dict(exps[0])
        z["up"] = (exps[0]["up"][0], np.zeros_like(exps[0]["up"][1]))
        zero = ffn(L, [z], bits, group, d_model, d_ff, X, None)
        if np.any(zero != 0.0):
            fails.append(f"Q{bits}: zero up scales do not give a zero output")
    return fails


def routed(L, experts, bits, group, d_model, d_ff, X, ids, w):
    X = np.ascontiguousarray(X, np.float32).reshape(-1, d_model)
    T = X.shape[0]
    ids = np.ascontiguousarray(ids, np.int32).reshape(T, -1)
    w = np.ascontiguousarray(w, np.float32).reshape(T, -1)
    out = np.empty((T, d_model), np.float64)
    arr = expert_struct(experts)
    assert L.oracle_routed_ffn(arr, len(experts), bits, group, d_model, d_ff, T, ids.shape[1], _p(ids), _p(w),
                               _p(X), _p(out)) == 0
    return out


def pin_routed(L, seed=13):
    """Routed experts (each token through its own slots) against the BLAS
    route, and its special cases: routing every token to every expert in
    ascending order with weights r is the dense router-weighted FFN (same
    sums, same order: bitwise); slots with an id outside [0, n) add nothing;
    a single slot of weight 1 is that expert alone."""
    fails = []
    rng = np.random.default_rng(seed)
    for bits in (4, 2):
        d_model, d_ff, group, n, T = 128, 192, 64, 4, 3
        exps = [make_expert(rng, d_model, d_ff, bits, group) for _ in range(n)]
        X = rng.standard_normal((T, d_model)).astype(np.float32)
        ids = np.array([[2, 0], [1, 3], [3, 2]], np.int32)
        w = rng.uniform(0.1, 1.0, size=(T, 2)).astype(np.float32)
        out = routed(L, exps, bits, group, d_model, d_ff, X, ids, w)
        for t in range(T):
            want = sum(float(w[t, s]) * numpy_ffn_one(exps[ids[t, s]], bits, group, X[t]) for s in range(2))
            err = np.max(np.abs(out[t] - want)) / max(1.0, np.max(np.abs(want)))
            if err > 1e-12:
                fails.append(f"Q{bits} token {t}: routed vs BLAS route rel err {err:.3g}")
        R = rng.uniform(0.1, 1.0, size=(T, n)).astype(np.float32)
        full = routed(L, exps, bits, group, d_model, d_ff, X, np.tile(np.arange(n, dtype=np.int32), (T, 1)), R)
        if not np.array_equal(full, ffn(L, exps, bits, group, d_model, d_ff, X, R)):
            fails.append(f"Q{bits}: full ascending routing differs from the dense FFN")
        skip = routed(L, exps, bits, group, d_model, d_ff, X, np.c_[ids[:, :1], [[-1], [n], [7]]], np.c_[w[:, :1], w[:, 1:]])
        if not np.array_equal(skip, routed(L, exps, bits, group, d_model, d_ff, X, ids[:, :1], w[:, :1])):
            fails.append(f"Q{bits}: out-of-range slots changed the result")
        one = routed(L, exps, bits, group, d_model, d_ff, X[:1], np.array([[3]], np.int32), np.ones((1, 1), np.float32))
        if not np.array_equal(one, ffn(L, exps[3:4], bits, group, d_model, d_ff, X[:1], None)):
            fails.append(f"Q{bits}: a single weight-1 slot is not that expert alone")
    return fails


# ---------------------------------------------------------------------------
# Decode attention block (section "GPU-Resident Decode Attention": per-head
# QK RMS norm with 1e-6 under the root, RoPE, K/V appended to the cache,
# causal GQA attention, output projection).

def _rmsnorm(L, x, w, eps=1e-6):
    x = np.ascontiguousarray(x, np.float64)
    w = np.ascontiguousarray(w, np.float32)
    y = np.empty_like(x)
    assert L.oracle_head_rmsnorm(_p(x), x.shape[0], x.shape[1], _p(w), eps, _p(y)) == 0
    return y


def _rope(L, x, pos, base):
    x = np.array(x, np.float64, order="C", copy=True)
    assert L.oracle_rope(_p(x), x.shape[0], x.shape[1], pos, base) == 0
    return x


def _attend(L, q, K, V, n_ctx):
    q = np.ascontiguousarray(q, np.float64)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    att = np.empty_like(q)
    assert L.oracle_gqa_attend(_p(q), q.shape[0], K.shape[0], q.shape[1], _p(K), _p(V), K.shape[1], n_ctx,
                               _p(att)) == 0
    return att


def pin_head_rmsnorm(L):
    """Closed forms of x / sqrt(mean x^2 + eps) * w."""
    fails = []
    hd, eps = 8, 1e-6
    w = np.array([1.0, 2.0, 0.5, -1.0, 3.0, 1.0, 0.25, 4.0], np.float32)
    # a constant row c: every entry is c / sqrt(c^2 + eps) * w[d]
    c = 0.75
    y = _rmsnorm(L, np.full((1, hd), c), w)
    want = c / math.sqrt(c * c + eps) * w.astype(np.float64)
    if not np.allclose(y[0], want, rtol=1e-14, atol=0):
        fails.append("constant row")
    # a spike a e_k: entry k is a / sqrt(a^2 / hd + eps) * w[k], the rest 0; a
    # small a makes eps matter (a^2 / hd = 1.25e-7)
    for a, k in ((1e-3, 3), (-5.0, 6), (2.0, 0)):
        x = np.zeros((1, hd))
        x[0, k] = a
        y = _rmsnorm(L, x, w)
        want = np.zeros(hd)
        want[k] = a / math.sqrt(a * a / hd + eps) * float(w[k])
        if not np.allclose(y[0], want, rtol=1e-13, atol=0):
            fails.append(f"spike a={a} at {k}")
    # heads are normalised on their own: scaling one head leaves the others
    x = np.arange(1.0, 17.0).reshape(2, hd)
    y1 = _rmsnorm(L, x, w)
    x2 = x.copy()
    x2[1] *= 1000.0
    y2 = _rmsnorm(L, x2, w)
    if not np.array_equal(y1[0], y2[0]):
        fails.append("a head's norm depends on another head")
    # a zero row stays zero
    if np.any(_rmsnorm(L, np.zeros((1, hd)), w)):
        fails.append("zero row")
    return fails


def pin_rope(L):
    """Rotations of basis vectors by the defined angles, and invariants."""
    fails = []
    # hd = 4, base 1e4: pair (x0, x2) turns by pos * 1, pair (x1, x3) by pos * 1e4^(-1/2) = pos / 100
    for pos in (1, 3):
        t0, t1 = float(pos), pos / 100.0
        y = _rope(L, np.eye(4), pos, 1e4)
        want = np.array([[math.cos(t0), 0, math.sin(t0), 0],
                         [0, math.cos(t1), 0, math.sin(t1)],
                         [-math.sin(t0), 0, math.cos(t0), 0],
                         [0, -math.sin(t1), 0, math.cos(t1)]])
        if not np.allclose(y, want, rtol=0, atol=1e-15):
            fails.append(f"basis rotation at pos {pos}")
    rng = np.random.default_rng(23)
    x = rng.standard_normal((3, 16))
    if not np.array_equal(_rope(L, x, 0, 1e6), x):
        fails.append("position 0 is not the identity")
    y = _rope(L, x, 77, 1e6)
    # each pair keeps its length
    if not np.allclose(x[:, :8] ** 2 + x[:, 8:] ** 2, y[:, :8] ** 2 + y[:, 8:] ** 2, rtol=1e-13):
        fails.append("pair lengths change")
    # the dot product of two rotated vectors depends on the position difference only
    a, b = x[0:1], x[1:2]
    d1 = float(_rope(L, a, 40, 1e6)[0] @ _rope(L, b, 25, 1e6)[0])
    d2 = float(_rope(L, a, 115, 1e6)[0] @ _rope(L, b, 100, 1e6)[0])
    if abs(d1 - d2) > 1e-12 * max(1.0, abs(d1)):
        fails.append("rotated dot products depend on the absolute position")
    return fails


def pin_gqa_attend(L):
    """One position, per-group constant values, a two-key closed form, the causal bound."""
    fails = []
    rng = np.random.default_rng(29)
    n_head, n_kv, hd, stride = 8, 2, 4, 5
    q = rng.standard_normal((n_head, hd))
    K = rng.standard_normal((n_kv, stride, hd)).astype(np.float32)
    V = rng.standard_normal((n_kv, stride, hd)).astype(np.float32)
    # one position: every head returns its group's value row
    att = _attend(L, q, K, V, 1)
    for h in range(n_head):
        if not np.array_equal(att[h], V[h // (n_head // n_kv), 0].astype(np.float64)):
            fails.append(f"single position, head {h}")
            break
    # values constant over positions (g + 1 in group g): the weights do not matter
    Vc = np.empty_like(V)
    for g in range(n_kv):
        Vc[g] = g + 1.0
    att = _attend(L, q, K, Vc, 4)
    want = np.array([[h // (n_head // n_kv) + 1.0] * hd for h in range(n_head)])
    if not np.allclose(att, want, rtol=1e-15, atol=0):
        fails.append("query heads read the wrong KV head")
    # two keys: scores s/sqrt(hd) and 0, values e0 and e1 -> (p, 1 - p, 0, 0), p = 1/(1 + e^(-s/2))
    s = 1.7
    q2 = np.zeros((n_head, hd))
    q2[:, 0] = s
    K2 = np.zeros((n_kv, stride, hd), np.float32)
    K2[:, 0, 0] = 1.0
    V2 = np.zeros((n_kv, stride, hd), np.float32)
    V2[:, 0, 0] = 1.0
    V2[:, 1, 1] = 1.0
    att = _attend(L, q2, K2, V2, 2)
    p = 1.0 / (1.0 + math.exp(-s / 2.0))
    if not np.allclose(att, np.tile([p, 1.0 - p, 0.0, 0.0], (n_head, 1)), rtol=1e-14, atol=1e-16):
        fails.append("two-key softmax closed form")
    # positions at and past n_ctx are never read
    K3, V3 = K.copy(), V.copy()
    K3[:, 3:] = 1e4
    V3[:, 3:] = -7.0
    if not np.array_equal(_attend(L, q, K3, V3, 3), _attend(L, q, K, V, 3)):
        fails.append("positions past the window are read")
    # ... and the last position of the window is
    V4 = V.copy()
    V4[:, 2] += 1.0
    if np.array_equal(_attend(L, q, K, V4, 3), _attend(L, q, K, V, 3)):
        fails.append("the window's last position is not read")
    return fails


def _bf16_bits(a):
    return (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def pin_attn_block(L):
    """Compositions with selection weights: at position 0 the output is the
    value row, gathered per group; with zero keys the window averages."""
    fails = []
    rng = np.random.default_rng(31)
    n_head, n_kv, hd, stride = 4, 2, 8, 6
    d_model = n_head * hd
    wq = _bf16_bits(rng.standard_normal((n_head * hd, d_model)).astype(np.float32) * 0.1)
    wk = _bf16_bits(rng.standard_normal((n_kv * hd, d_model)).astype(np.float32) * 0.1)
    sel = np.zeros((n_kv * hd, d_model), np.float32)
    sel[np.arange(n_kv * hd), np.arange(n_kv * hd)] = 1.0   # v = x[: n_kv * hd]
    wv = _bf16_bits(sel)
    wo = _bf16_bits(np.eye(d_model, dtype=np.float32))      # out = att
    qn = (1.0 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    kn = (1.0 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    x = rng.standard_normal(d_model).astype(np.float32)

    def block(wk_, pos, K, V):
        K = np.array(K, np.float32, order="C", copy=True)
        V = np.array(V, np.float32, order="C", copy=True)
        out = np.empty(d_model)
        rc = L.oracle_attn_decode(_p(wq), _p(wk_), _p(wv), _p(wo), _p(qn), _p(kn), d_model, n_head, n_kv, hd,
                                  _p(x), pos, 1e6, _p(K), _p(V), stride, _p(out), None, None)
        assert rc == 0
        return out, K, V

    K0 = rng.standard_normal((n_kv, stride, hd)).astype(np.float32)
    V0 = rng.standard_normal((n_kv, stride, hd)).astype(np.float32)
    out, K, V = block(wk, 0, K0, V0)
    want = np.concatenate([x[(h // (n_head // n_kv)) * hd:(h // (n_head // n_kv) + 1) * hd] for h in range(n_head)])
    if not np.array_equal(out, want.astype(np.float64)):
        fails.append("position 0: out is not the gathered value rows")
    if not np.array_equal(V[:, 0], x[: n_kv * hd].reshape(n_kv, hd)):
        fails.append("position 0: the value row appended is not v")
    if not (np.array_equal(K[:, 1:], K0[:, 1:]) and np.array_equal(V[:, 1:], V0[:, 1:])):
        fails.append("rows other than pos changed")
    # zero key weights: k = 0 after norm and rotation, every score is q . 0 = 0,
    # so the window 0..pos averages its values (the new one is v)
    pos = 3
    zk = np.zeros_like(wk)
    Kz = np.zeros((n_kv, stride, hd), np.float32)
    Vz = np.zeros((n_kv, stride, hd), np.float32)
    for g in range(n_kv):
        for j in range(pos):
            Vz[g, j] = 10.0 * g + j + 1.0
    out, K, V = block(zk, pos, Kz, Vz)
    want = []
    for h in range(n_head):
        g = h // (n_head // n_kv)
        want.append((Vz[g, :pos].astype(np.float64).sum(axis=0) + x[g * hd:(g + 1) * hd]) / (pos + 1))
    if not np.allclose(out, np.concatenate(want), rtol=1e-14, atol=1e-15):
        fails.append("zero keys: the window 0..pos is not averaged")
    if np.any(K[:, pos]):
        fails.append("zero keys: the appended key is not 0")
    return fails


CORE_PINS = [pin_worked_examples, pin_unpack_exhaustive, pin_affine_identity, pin_silu,
             pin_bf16, pin_f16, pin_ffn_composition, pin_routed, pin_head_rmsnorm, pin_rope,
             pin_gqa_attend, pin_attn_block]


def run_core_pins(L):
    fails = []
    for pin in CORE_PINS:
        try:
            fails += [f"{pin.__name__}: {m}" for m in pin(L)]
        except Exception as exc:   # a broken oracle may refuse its arguments
            fails.append(f"{pin.__name__}: raised {type(exc).__name__}: {exc}")
    return fails
