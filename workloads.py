"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module draws random numbers and shapes them into the arrays the
expert-FFN and bf16-matvec workloads take.  It holds none of the method's
arithmetic: no unpacking of codes, no dequantisation, no dot products and no
activation.  Packed code bytes are drawn directly as independent uniform
bytes: a uniform byte is, bit for bit, two independent uniform 4-bit codes or
four independent uniform 2-bit codes, so no packing step is needed here and
neither side of the comparison has to trust the other's bit order.

Every array comes from its own PCG64 stream keyed by ``SeedSequence([seed,
*tags])``.  Only the raw 64-bit words of that bit generator are used
(``random_raw``), and uniform and normal variates are derived from them here
by a fixed recipe, so the bytes do not depend on numpy's ``Generator``
sampling methods:

* uniform on [lo, hi): ``lo + (hi - lo) * (u >> 11) * 2**-53`` in f64, then f32;
* standard normal: Box-Muller on two such uniforms in f64, then f32;
* bf16 weights: f32 normal times sigma, rounded to bf16 by round-to-nearest-even
  on the f32 bit pattern.

Workload shapes follow the Metal Compute Kernels page of the S-MoE docs
(d_model 4096 staged input, 1536-row gate_up grids, the bf16 projection table
and the LM head), with f32 scales per 64-column group.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Stream tags.  Each (seed, tags) pair names one independent stream.
_MAT = {"gate": 0, "up": 1, "down": 2}
_KIND_CODES, _KIND_SCALES = 0, 1
_TAG_X, _TAG_ROUTER, _TAG_XBATCH, _TAG_BF16_W, _TAG_BF16_X = 100, 101, 102, 200, 201

_CHUNK = 1 << 22  # variates generated per block, to bound temporary memory


def _stream(seed: int, tags) -> np.random.PCG64:
    return np.random.PCG64(np.random.SeedSequence([int(seed)] + [int(t) for t in tags]))


def random_bytes(seed: int, tags, nbytes: int) -> np.ndarray:
    """``nbytes`` independent uniform bytes (uint8)."""
    n64 = (nbytes + 7) // 8
    raw = _stream(seed, tags).random_raw(n64).astype("<u8", copy=False)
    return raw.view(np.uint8)[:nbytes].copy()


def _unit_uniform(bg: np.random.PCG64, n: int) -> np.ndarray:
    """n doubles in [0, 1) with 53 random bits each."""
    return (bg.random_raw(n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_f32(seed: int, tags, n: int, lo: float, hi: float) -> np.ndarray:
    bg = _stream(seed, tags)
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = (lo + (hi - lo) * _unit_uniform(bg, m)).astype(np.float32)
    return out


def normal_f32(seed: int, tags, n: int, sigma: float = 1.0) -> np.ndarray:
    """n standard-normal variates times ``sigma`` (Box-Muller in f64), as f32."""
    bg = _stream(seed, tags)
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        half = (m + 1) // 2
        u1 = 1.0 - _unit_uniform(bg, half)          # (0, 1]: log is finite
        u2 = _unit_uniform(bg, half)
        r = np.sqrt(-2.0 * np.log(u1))
        z = np.empty(2 * half, dtype=np.float64)
        z[0::2] = r * np.cos(2.0 * np.pi * u2)
        z[1::2] = r * np.sin(2.0 * np.pi * u2)
        out[s:s + m] = (z[:m] * sigma).astype(np.float32)
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round f32 values to bf16 (round to nearest, ties to even); uint16 bits.

    Inputs here are finite, so no NaN handling is needed.
    """
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_normal(seed: int, tags, rows: int, cols: int, sigma: float) -> np.ndarray:
    """bf16 bits [rows, cols] of N(0, sigma^2), generated in row blocks."""
    out = np.empty((rows, cols), dtype=np.uint16)
    block = max(1, _CHUNK // cols)
    for b, r0 in enumerate(range(0, rows, block)):
        r1 = min(rows, r0 + block)
        vals = normal_f32(seed, tuple(tags) + (b,), (r1 - r0) * cols, sigma)
        out[r0:r1] = f32_to_bf16_bits(vals).reshape(r1 - r0, cols)
    return out


def softmax_f32(logits: np.ndarray) -> np.ndarray:
    """Router weights: softmax over the last axis in f64, returned as f32."""
    l64 = logits.astype(np.float64)
    e = np.exp(l64 - l64.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


# ----------------------------------------------------------------------------
# Quantised expert weights
# ----------------------------------------------------------------------------

@dataclass
class QMat:
    """One packed matrix: ``codes`` uint8 [rows, cols*bits/8], ``scales`` [rows, cols/group],
    f32, or float16 for the 2-byte scale layout."""
    codes: np.ndarray
    scales: np.ndarray


@dataclass
class Expert:
    gate: QMat   # [d_ff, d_model]
    up: QMat     # [d_ff, d_model]
    down: QMat   # [d_model, d_ff]


@dataclass
class ExpertGroup:
    bits: int
    group: int
    d_model: int
    d_ff: int
    experts: list = field(default_factory=list)
    scale_f16: bool = False

    def byte_count(self) -> int:
        return sum(m.codes.nbytes + m.scales.nbytes
                   for e in self.experts for m in (e.gate, e.up, e.down))


def qmat(seed: int, expert: int, name: str, rows: int, cols: int, bits: int, group: int,
         scale_lo: float = 0.01, scale_hi: float = 0.05, scale_f16: bool = False) -> QMat:
    """Codes uniform; scales U[scale_lo, scale_hi) as f32, or those f32 values
    rounded to the nearest binary16 (ties to even) for the 2-byte layout."""
    if (cols * bits) % 8 or cols % group:
        raise ValueError("cols must fill whole bytes and whole groups")
    m = _MAT[name]
    codes = random_bytes(seed, (expert, m, _KIND_CODES), rows * cols * bits // 8)
    scales = uniform_f32(seed, (expert, m, _KIND_SCALES), rows * (cols // group), scale_lo, scale_hi)
    if scale_f16:
        scales = scales.astype(np.float16)
    return QMat(codes.reshape(rows, cols * bits // 8), scales.reshape(rows, cols // group))


def expert_group(seed: int, n_experts: int, d_model: int, d_ff: int, bits: int,
                 group: int = 64, scale_f16: bool = False) -> ExpertGroup:
    g = ExpertGroup(bits=bits, group=group, d_model=d_model, d_ff=d_ff, scale_f16=scale_f16)
    for e in range(n_experts):
        g.experts.append(Expert(
            gate=qmat(seed, e, "gate", d_ff, d_model, bits, group, scale_f16=scale_f16),
            up=qmat(seed, e, "up", d_ff, d_model, bits, group, scale_f16=scale_f16),
            down=qmat(seed, e, "down", d_model, d_ff, bits, group, scale_f16=scale_f16)))
    return g


def widened_scales(g: ExpertGroup) -> ExpertGroup:
    """The same group with every 2-byte scale stored as the f32 of equal value."""
    w = ExpertGroup(bits=g.bits, group=g.group, d_model=g.d_model, d_ff=g.d_ff, scale_f16=False)
    for e in g.experts:
        w.experts.append(Expert(*[QMat(m.codes, m.scales.astype(np.float32)) for m in (e.gate, e.up, e.down)]))
    return w


def activation(seed: int, d_model: int) -> np.ndarray:
    return normal_f32(seed, (_TAG_X,), d_model)


def activation_batch(seed: int, T: int, d_model: int) -> np.ndarray:
    return normal_f32(seed, (_TAG_XBATCH,), T * d_model).reshape(T, d_model)


def router_weights(seed: int, n_experts: int, T: int = 1) -> np.ndarray:
    """f32 [T, n_experts]: softmax of N(0,1) f32 logits per token."""
    return softmax_f32(normal_f32(seed, (_TAG_ROUTER,), T * n_experts).reshape(T, n_experts))


# ----------------------------------------------------------------------------
# Named workloads
# ----------------------------------------------------------------------------

TINY = dict(name="q4_tiny_1expert_256x512", seed=0, n_experts=1, d_model=256, d_ff=512, bits=4)
Q4_GROUP8 = dict(name="q4_8expert_4096x1536", seed=1, n_experts=8, d_model=4096, d_ff=1536, bits=4)
Q2_GROUP8 = dict(name="q2_8expert_4096x1536", seed=2, n_experts=8, d_model=4096, d_ff=1536, bits=2)
# The same groups with 2-byte (binary16) scales: same codes, scales rounded to f16.
Q4_GROUP8_S16 = dict(Q4_GROUP8, name="q4_8expert_4096x1536_f16scales", scale_f16=True)
Q2_GROUP8_S16 = dict(Q2_GROUP8, name="q2_8expert_4096x1536_f16scales", scale_f16=True)
BF16_SHAPES = [  # (rows, cols, role, seed)
    (8192, 4096, "q_proj", 30),
    (4096, 8192, "o_proj", 31),
    (512, 4096, "kv_proj", 32),
    (151936, 4096, "lm_head", 33),
]
BATCH_TOKENS = {16: 40, 64: 41, 256: 42}   # T -> seed of X; weights are Q4_GROUP8's
# One launch of several bf16 matvecs: a token's attention input projections
# (q, k, v) over one shared x.  (rows, cols, role, seed of W); x uses the first seed.
BF16_BATCH = [
    (8192, 4096, "q_proj", 34),
    (512, 4096, "k_proj", 35),
    (512, 4096, "v_proj", 36),
]


def make_group(spec: dict) -> ExpertGroup:
    return expert_group(spec["seed"], spec["n_experts"], spec["d_model"], spec["d_ff"], spec["bits"],
                        scale_f16=spec.get("scale_f16", False))


def make_decode_inputs(spec: dict):
    """(ExpertGroup, x f32 [d_model], router f32 [n_experts]) for a decode group."""
    g = make_group(spec)
    x = activation(spec["seed"], spec["d_model"])
    r = router_weights(spec["seed"], spec["n_experts"])[0]
    return g, x, r


def make_bf16(rows: int, cols: int, seed: int, sigma: float = 0.02):
    """(W bf16 bits uint16 [rows, cols], x f32 [cols])."""
    W = bf16_normal(seed, (_TAG_BF16_W,), rows, cols, sigma)
    x = normal_f32(seed, (_TAG_BF16_X,), cols)
    return W, x


def make_bf16_batch(jobs=BF16_BATCH):
    """([W bf16 bits uint16 [rows, cols] per job], x f32 [cols]) with one x
    shared by all jobs (all jobs must have the same cols)."""
    cols = jobs[0][1]
    assert all(j[1] == cols for j in jobs)
    Ws = [bf16_normal(seed, (_TAG_BF16_W,), rows, cols, 0.02) for rows, _, _, seed in jobs]
    return Ws, normal_f32(jobs[0][3], (_TAG_BF16_X,), cols)


ROUTED = dict(T=256, top_k=2, seed=43)   # routed prefill over Q4_GROUP8's 8 experts


def top_k_routing(seed: int, T: int, n_experts: int, top_k: int):
    """Synthetic top-k routing: per token, N(0,1) f32 logits over the experts;
    ids = the top_k largest (ties to the lower id), weights = softmax of those
    logits.  Returns (ids int32 [T, top_k], w f32 [T, top_k])."""
    logits = normal_f32(seed, (_TAG_ROUTER, 1), T * n_experts).reshape(T, n_experts)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    return ids, softmax_f32(np.take_along_axis(logits, ids, axis=1))


def make_routed_inputs(T: int, top_k: int, seed: int = 43, n_experts: int = 8, d_model: int = 4096):
    """(X f32 [T, d_model], ids int32 [T, top_k], w f32 [T, top_k])."""
    ids, w = top_k_routing(seed, T, n_experts, top_k)
    return activation_batch(seed, T, d_model), ids, w


def make_batch_inputs(T: int, seed: int | None = None, d_model: int = 4096):
    """(X f32 [T, d_model], router f32 [T, 8]) for the token-batch workload."""
    seed = BATCH_TOKENS[T] if seed is None else seed
    return activation_batch(seed, T, d_model), router_weights(seed, 8, T)


# ----------------------------------------------------------------------------
# Decode attention block (section "GPU-Resident Decode Attention"): the bf16
# projection table's shapes (q 8192 x 4096, k/v 512 x 4096, o 4096 x 8192),
# i.e. 64 query heads and 4 KV heads of 128 dimensions, a 4096-position f32
# KV cache, and the newest token at the cache's last position.
_TAG_ATTN = 300
ATTN = dict(name="attn_decode_4096_h64_kv4_d128", seed=50, d_model=4096, n_head=64, n_kv=4, head_dim=128,
            max_ctx=4096, pos=4095, rope_base=1e6)
# A small block for parity at every position of a short cache.
ATTN_SMALL = dict(name="attn_decode_256_h8_kv2_d64", seed=51, d_model=256, n_head=8, n_kv=2, head_dim=64,
                  max_ctx=100, pos=37, rope_base=1e4)


@dataclass
class AttnWeights:
    wq: np.ndarray       # bf16 bits [n_head*hd, d_model]
    wk: np.ndarray       # bf16 bits [n_kv*hd, d_model]
    wv: np.ndarray       # bf16 bits [n_kv*hd, d_model]
    wo: np.ndarray       # bf16 bits [d_model, n_head*hd]
    q_norm: np.ndarray   # f32 [hd]
    k_norm: np.ndarray   # f32 [hd]


def attn_weights(seed: int, d_model: int, n_head: int, n_kv: int, head_dim: int) -> AttnWeights:
    """Projections bf16 ~ N(0, 0.02^2); norm gains f32 1 + N(0, 0.1^2)."""
    nq, nk = n_head * head_dim, n_kv * head_dim
    return AttnWeights(
        wq=bf16_normal(seed, (_TAG_ATTN, 0), nq, d_model, 0.02),
        wk=bf16_normal(seed, (_TAG_ATTN, 1), nk, d_model, 0.02),
        wv=bf16_normal(seed, (_TAG_ATTN, 2), nk, d_model, 0.02),
        wo=bf16_normal(seed, (_TAG_ATTN, 3), d_model, nq, 0.02),
        q_norm=(1.0 + normal_f32(seed, (_TAG_ATTN, 4), head_dim, 0.1)).astype(np.float32),
        k_norm=(1.0 + normal_f32(seed, (_TAG_ATTN, 5), head_dim, 0.1)).astype(np.float32))


def kv_cache(seed: int, n_kv: int, max_ctx: int, head_dim: int):
    """(K, V) f32 [n_kv, max_ctx, head_dim], N(0, 1) entries: cached keys are
    RMS-normed rows (unit RMS before the gain) and values are projections of
    unit-variance inputs by N(0, 0.02^2) weights over 4096 columns (RMS about 1.3),
    so unit-variance draws stand in for both."""
    K = normal_f32(seed, (_TAG_ATTN, 6), n_kv * max_ctx * head_dim).reshape(n_kv, max_ctx, head_dim)
    V = normal_f32(seed, (_TAG_ATTN, 7), n_kv * max_ctx * head_dim).reshape(n_kv, max_ctx, head_dim)
    return K, V


def make_attn_inputs(spec: dict):
    """(AttnWeights, x f32 [d_model], K, V) for an attention workload."""
    w = attn_weights(spec["seed"], spec["d_model"], spec["n_head"], spec["n_kv"], spec["head_dim"])
    x = normal_f32(spec["seed"], (_TAG_ATTN, 8), spec["d_model"])
    K, V = kv_cache(spec["seed"], spec["n_kv"], spec["max_ctx"], spec["head_dim"])
    return w, x, K, V
