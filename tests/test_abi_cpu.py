"""The C ABI without a GPU: the library loads, exports every function that
include/smoe.h declares, and refuses every out-of-contract argument with the
documented status before it touches the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smoe.h")


@pytest.fixture(scope="module")
def gq():
    import group_quantized_moe_amd as gq
    if not os.path.exists(gq.LIB_PATH):
        from group_quantized_moe_amd import build
        build.build()
    gq.lib()
    return gq


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert set(declared_functions()) == {
        "smoe_gate_up", "smoe_down", "smoe_expert_ffn_workspace", "smoe_expert_ffn", "smoe_expert_ffn_noalloc",
        "matvec_bf16_workspace", "matvec_bf16", "matvec_bf16_batch", "smoe_routed_ffn_workspace",
        "smoe_routed_ffn", "smoe_attn_decode_workspace", "smoe_attn_decode", "smoe_status_str"}


def test_library_exports_every_declared_symbol(gq):
    L = ctypes.CDLL(gq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(gq.EXPORTS) == set(declared_functions())


def test_status_strings(gq):
    for s in range(0, -10, -1):
        assert gq.smoe_status_str(s) not in ("", "unknown status")
    assert gq.smoe_status_str(-99) == "unknown status"


# Fake, well-aligned device addresses: every call below must be refused (or
# reach the device check) before anything dereferences them.
A = 0x10000000
QM = lambda base: ctypes.byref(__import__("group_quantized_moe_amd").QMat(base, base + 0x1000000))


def gate_up(L, bits=4, group=64, d_ff=512, d_model=256, x=A + 0x8000000, h=A + 0x9000000, g=A, u=A + 0x4000000):
    import group_quantized_moe_amd as gq
    return L.smoe_gate_up(ctypes.byref(gq.QMat(g, g + 0x1000000)), ctypes.byref(gq.QMat(u, u + 0x1000000)),
                          bits, group, d_ff, d_model, x, h, None)


def test_gate_up_refusals(gq):
    L = gq.lib()
    assert gate_up(L, bits=3) == -2
    assert gate_up(L, bits=8) == -2
    assert gate_up(L, group=48) == -3              # not a multiple of 32
    assert gate_up(L, bits=2, group=32) == -3      # 2-bit needs multiples of 64
    assert gate_up(L, group=512) == -3             # does not divide d_model = 256
    assert gate_up(L, d_model=80) == -4            # not a multiple of 32
    assert gate_up(L, d_ff=0) == -4
    assert gate_up(L, d_model=16384) == -4         # above SMOE_MAX_QCOLS
    assert gate_up(L, x=0) == -1
    assert gate_up(L, g=A + 8) == -5               # codes not 16-byte aligned
    assert gate_up(L, x=A + 0x8000004) == -5       # x not 16-byte aligned
    assert gate_up(L, h=A + 0x100) == -7           # hidden inside the gate codes
    assert gate_up(L, h=A + 0x8000000 + 512) == -7 # hidden inside x
    assert gate_up(L) == -8                        # all valid: no gfx950 device here


def test_down_and_bf16_refusals(gq):
    L = gq.lib()
    D = gq.QMat(A, A + 0x1000000)
    assert L.smoe_down(ctypes.byref(D), 4, 64, 256, 512, A + 0x8000000, A + 0x8000000, None) == -7
    assert L.smoe_down(ctypes.byref(D), 4, 64, 256, 500, A + 0x8000000, A + 0x9000000, None) == -4
    assert L.smoe_down(ctypes.byref(D), 4, 64, 256, 512, A + 0x8000000, A + 0x9000000, None) == -8
    assert L.matvec_bf16(A, 16, 12, A + 0x8000000, A + 0x9000000, None, 0, None) == -4
    assert L.matvec_bf16(A + 2, 16, 16, A + 0x8000000, A + 0x9000000, None, 0, None) == -5
    assert L.matvec_bf16(A, 16, 16, A + 0x8000000, A + 16, None, 0, None) == -7
    assert L.matvec_bf16(A, 16, 16, A + 0x8000000, A + 0x9000000, None, 0, None) == -8
    assert L.matvec_bf16_workspace(512, 4096) == 0


def test_scale_format_flag(gq):
    """Unknown format bits are refused; f16 scales need 2-byte alignment only."""
    L = gq.lib()
    F16 = gq.SMOE_SCALE_F16
    G = gq.QMat(A, A + 0x1000000)
    U = gq.QMat(A + 0x2000000, A + 0x3000000)
    x, h = A + 0x8000000, A + 0x9000000
    args = lambda bits: (ctypes.byref(G), ctypes.byref(U), bits, 64, 512, 256, x, h, None)
    assert L.smoe_gate_up(*args(4 | 0x200)) == -2
    assert L.smoe_gate_up(*args(8 | F16)) == -2
    assert L.smoe_gate_up(*args(4 | F16)) == -8           # valid: reaches the device check
    U2 = gq.QMat(A + 0x2000000, A + 0x3000002)             # scales 2-byte aligned
    a2 = (ctypes.byref(G), ctypes.byref(U2), 4 | F16, 64, 512, 256, x, h, None)
    assert L.smoe_gate_up(*a2) == -8
    a2f = (ctypes.byref(G), ctypes.byref(U2), 4, 64, 512, 256, x, h, None)
    assert L.smoe_gate_up(*a2f) == -5                      # f32 scales need 4-byte alignment
    U1 = gq.QMat(A + 0x2000000, A + 0x3000001)
    assert L.smoe_gate_up(ctypes.byref(G), ctypes.byref(U1), 4 | F16, 64, 512, 256, x, h, None) == -5
    # hidden inside the gate scales: 512 rows x 4 groups x 2 bytes = 4096 bytes of f16 scales
    assert L.smoe_gate_up(ctypes.byref(G), ctypes.byref(U), 4 | F16, 64, 512, 256, x, A + 0x1000000 + 4092, None) == -7
    assert L.smoe_gate_up(ctypes.byref(G), ctypes.byref(U), 4 | F16, 64, 512, 256, x, A + 0x1000000 + 4096, None) == -8


def test_routed_ffn_refusals(gq):
    """smoe_routed_ffn checks its arguments before touching the device."""
    L = gq.lib()
    n, T, k, dm, dff = 2, 8, 2, 256, 512
    arr = (gq.Expert * n)()
    for e in range(n):
        b = A + 0x1000000 * (1 + 6 * e)
        arr[e] = gq.Expert(gq.QMat(b, b + 0x1000000), gq.QMat(b + 0x2000000, b + 0x3000000),
                           gq.QMat(b + 0x4000000, b + 0x5000000))
    ids, w, x, out = A + 0x70000000, A + 0x71000000, A + 0x72000000, A + 0x73000000
    need = L.smoe_routed_ffn_workspace(n, dm, dff, T, k)
    assert need > 0 and L.smoe_routed_ffn_workspace(n, dm, dff, T, 0) == 0
    ws = A + 0x40000000
    call = lambda **o: L.smoe_routed_ffn(arr, o.get("n", n), o.get("bits", 4), o.get("group", 64), dm, dff,
                                         o.get("T", T), o.get("k", k), o.get("ids", ids), o.get("w", w), x,
                                         o.get("out", out), ws, o.get("need", need), None)
    assert call() == -8                       # valid: reaches the device check
    assert call(ids=None) == -1
    assert call(k=0) == -4 and call(k=17) == -4 and call(T=0) == -4 and call(n=17) == -4
    assert call(group=96) == -3               # the routed path tiles groups of 32 and 64 only
    assert call(w=w + 2) == -5
    assert call(need=need - 1) == -6
    assert call(out=ids) == -7                # out overlaps the slot ids
    assert call(bits=3) == -2


def test_bf16_batch_refusals(gq):
    """Every out-of-contract batch is refused before the device is touched;
    a valid one reaches the device check (-8 without a GPU)."""
    L = gq.lib()
    J = gq.Bf16Job

    def call(*jobs, n=None):
        arr = (J * max(1, len(jobs)))(*jobs)
        return L.matvec_bf16_batch(arr, len(jobs) if n is None else n, None)

    W0, W1 = A, A + 0x1000000
    x0, y0, y1 = A + 0x8000000, A + 0x9000000, A + 0xA000000
    ok0, ok1 = J(W0, x0, y0, 512, 4096), J(W1, x0, y1, 64, 4096)
    assert L.matvec_bf16_batch(None, 1, None) == -1
    assert call(ok0, n=0) == -4
    assert call(*([ok0] * 17)) == -4                      # above SMOE_MAX_BF16_JOBS
    assert call(ok0, J(W1, None, y1, 64, 4096)) == -1
    assert call(ok0, J(W1, x0, y1, 64, 4092)) == -4        # cols % 8
    assert call(ok0, J(W1, x0, y1, 0, 4096)) == -4
    assert call(ok0, J(W1, x0, y1, 64, 16392)) == -4       # above SMOE_MAX_BF16_COLS
    assert call(ok0, J(W1 + 8, x0, y1, 64, 4096)) == -5
    assert call(ok0, J(W1, x0 + 4, y1, 64, 4096)) == -5
    assert call(ok0, J(W1, x0, y0 + 64, 64, 4096)) == -7   # y overlaps another job's y
    assert call(ok0, J(W1, x0, W0 + 4096, 64, 4096)) == -7  # y overlaps another job's W
    assert call(ok0, J(W1, x0, x0 + 256, 64, 4096)) == -7   # y overlaps a shared x
    assert call(ok0, ok1) == -8                           # valid (shared x): reaches the device check
    assert call(*([J(W0, x0, A + 0xB000000 + 0x10000 * k, 512, 4096) for k in range(16)])) == -8


def test_expert_ffn_refusals(gq):
    L = gq.lib()
    n = 2
    arr = (gq.Expert * n)()
    for k in range(n):
        b = A + k * 0x10000000
        arr[k] = gq.Expert(gq.QMat(b, b + 0x1000000), gq.QMat(b + 0x2000000, b + 0x3000000),
                           gq.QMat(b + 0x4000000, b + 0x5000000))
    X, OUT, WS = 0x80000000, 0x90000000, 0xA0000000
    need = L.smoe_expert_ffn_workspace(n, 256, 512, 1)
    assert need >= 4 * n * 512
    call = lambda **kw: L.smoe_expert_ffn(
        arr, kw.get("n", n), kw.get("route", None), 4, 64, 256, 512, kw.get("T", 1), X,
        kw.get("out", OUT), kw.get("ws", WS), kw.get("wsb", need), None)
    assert call(n=0) == -4
    assert call(n=17) == -4
    assert call(T=0) == -4
    assert call(ws=0) == -6
    assert call(wsb=need - 1) == -6
    assert call(ws=WS + 64) == -5                  # workspace must be 256-byte aligned
    assert call(out=WS + 256) == -7                # out inside the workspace
    assert call(out=A + 0x100) == -7               # out inside expert 0's gate codes
    assert call() == -8


def test_expert_ffn_noalloc_refusals(gq):
    """The no-allocation variant checks what smoe_expert_ffn checks, and
    refuses a call whose workspace would exceed its static scratch array
    before it looks at the device."""
    L = gq.lib()
    n = 8
    arr = (gq.Expert * n)()
    for k in range(n):
        b = A + k * 0x10000000
        arr[k] = gq.Expert(gq.QMat(b, b + 0x1000000), gq.QMat(b + 0x2000000, b + 0x3000000),
                           gq.QMat(b + 0x4000000, b + 0x5000000))
    X, OUT = 0x900000000, 0xA00000000
    call = lambda **kw: L.smoe_expert_ffn_noalloc(
        arr, kw.get("n", n), None, kw.get("bits", 4), 64, kw.get("dm", 4096), kw.get("dff", 1536),
        kw.get("T", 1), kw.get("x", X), kw.get("out", OUT), None)
    assert gq.SMOE_NOALLOC_SCRATCH_BYTES == 1 << 20
    assert L.smoe_expert_ffn_workspace(16, 8192, 8192, 1) <= gq.SMOE_NOALLOC_SCRATCH_BYTES  # every decode call fits
    assert L.smoe_expert_ffn_workspace(8, 4096, 1536, 64) > gq.SMOE_NOALLOC_SCRATCH_BYTES
    assert call(T=64) == -6                        # beyond the scratch array
    assert call(n=0) == -4
    assert call(bits=3) == -2
    assert call(x=X + 4) == -5
    assert call(out=A + 0x100) == -7               # out inside expert 0's gate codes
    assert call() == -8                            # all valid: no gfx950 device here


def test_expert_ffn_batch_refusals(gq):
    """T > 1: workspace sizing and the token-batch refusals (group outside the
    batch tiling, T above the limit), all decided before the device query."""
    L = gq.lib()
    n, T = 2, 40
    arr = (gq.Expert * n)()
    for k in range(n):
        b = A + k * 0x10000000
        arr[k] = gq.Expert(gq.QMat(b, b + 0x1000000), gq.QMat(b + 0x2000000, b + 0x3000000),
                           gq.QMat(b + 0x4000000, b + 0x5000000))
    X, OUT, WS = 0x80000000, 0x90000000, 0xA0000000
    need = L.smoe_expert_ffn_workspace(n, 320, 640, T)
    # hi/lo halves of X and H plus one exponent per 32 columns at least.
    assert need >= 4 * T * 320 + 4 * n * T * 640 + 4 * T * 10 + 4 * n * T * 20
    assert L.smoe_expert_ffn_workspace(n, 320, 640, 65537) == 0
    call = lambda **kw: L.smoe_expert_ffn(
        arr, n, None, kw.get("bits", 4), kw.get("group", 64), 320, 640, kw.get("T", T), X, OUT, WS,
        kw.get("wsb", need), None)
    assert call(group=160) == -3                   # valid for decode, not for the batch tiling
    # Groups of 96 and 128 columns are decode-only (T = 1); the batch takes 32 or 64.
    call2 = lambda bits, group: L.smoe_expert_ffn(arr, n, None, bits, group, 384, 768, T, X, OUT, WS, 1 << 30, None)
    assert call2(4, 96) == -3 and call2(4, 128) == -3 and call2(2, 128) == -3
    assert call2(4, 64) == -8 and call2(4, 32) == -8 and call2(2, 64) == -8
    assert call(bits=2, group=32) == -3
    assert call(T=65537) == -4
    assert call(wsb=need - 1) == -6
    assert call() == -8
    assert call(group=32) == -8
    assert call(bits=2, group=64) == -8


def test_attn_decode_refusals(gq):
    """smoe_attn_decode checks shapes, pointers, alignment, workspace and
    aliasing before touching the device; a valid call reaches the device check."""
    L = gq.lib()
    dm, H, KV, hd, ctx = 4096, 64, 4, 128, 4096
    need = L.smoe_attn_decode_workspace(dm, H, KV, hd, ctx)
    assert need > 0
    assert L.smoe_attn_decode_workspace(dm, H, KV, 96, ctx) == 0          # head_dim 64 or 128
    assert L.smoe_attn_decode_workspace(dm, H, 3, hd, ctx) == 0           # n_head % n_kv
    assert L.smoe_attn_decode_workspace(dm, 64, 2, hd, ctx) == 0          # 32 query heads per KV head
    assert L.smoe_attn_decode_workspace(dm + 4, H, KV, hd, ctx) == 0      # d_model % 8
    G = 1 << 28
    wq, wk, wv, wo = A, A + G, A + 2 * G, A + 3 * G
    qn, kn, x, out = A + 4 * G, A + 4 * G + 0x10000, A + 4 * G + 0x20000, A + 4 * G + 0x30000
    kc, vc, ws = A + 5 * G, A + 6 * G, A + 7 * G

    def call(**o):
        w = gq.AttnWeights(o.get("wq", wq), wk, wv, o.get("wo", wo), qn, kn)
        return L.smoe_attn_decode(ctypes.byref(w), o.get("dm", dm), H, KV, o.get("hd", hd), o.get("x", x),
                                  o.get("pos", ctx - 1), o.get("base", 1e6), o.get("kc", kc), vc, ctx,
                                  o.get("out", out), o.get("ws", ws), o.get("need", need), None)
    assert call() == -8                        # valid: reaches the device check
    assert call(pos=0) == -8
    assert call(wq=None) == -1 and call(x=None) == -1 and call(kc=None) == -1
    assert call(pos=ctx) == -4 and call(pos=-1) == -4 and call(base=0.0) == -4 and call(base=-1.0) == -4
    assert call(hd=96) == -4 and call(dm=4100) == -4
    assert call(wo=wo + 2) == -5 and call(x=x + 4) == -5 and call(kc=kc + 4) == -5
    assert call(need=need - 1) == -6 and call(ws=None) == -6
    assert call(ws=ws + 64) == -5
    assert call(out=x) == -7                   # out overlaps x
    assert call(out=kc + 64) == -7             # out overlaps the K cache
    assert call(kc=vc) == -7                   # the caches overlap
    assert call(ws=wq) == -7                   # the workspace overlaps Wq
