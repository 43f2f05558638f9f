"""GPU parity of the decode path (one token) against the f64 oracle, through
the C ABI, on the workload shapes and on ragged / edge shapes."""
import numpy as np
import pytest

import workloads
from gpu_helpers import assert_nonfinite_like, assert_parity, assert_relative, dev, dev_experts, run_ffn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gq():
    import torch
    import group_quantized_moe_amd as gq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gq.lib()
    return gq


def gate_up_gpu(gq, e, bits, group, x):
    import torch
    d_ff = e.gate.codes.shape[0]
    h = torch.empty(d_ff, dtype=torch.float32, device="cuda")
    gq.smoe_gate_up(e.gate.codes, e.gate.scales, e.up.codes, e.up.scales, bits, group, dev(x), h)
    torch.cuda.synchronize()
    return h.cpu().numpy()


def down_gpu(gq, e, bits, group, h32):
    import torch
    d_model = e.down.codes.shape[0]
    out = torch.empty(d_model, dtype=torch.float32, device="cuda")
    gq.smoe_down(e.down.codes, e.down.scales, bits, group, dev(h32), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_tiny_expert_stages_and_ffn(gq, oracle_lib):
    """Single 4-bit expert, d_model 256 / d_ff 512: each stage and the whole FFN."""
    g, x, _ = workloads.make_decode_inputs(workloads.TINY)
    e, de = g.experts[0], dev_experts(g)[0]
    h_ref = oracle_lib.gate_up(e, 4, 64, g.d_ff, g.d_model, x)
    assert_parity(gate_up_gpu(gq, de, 4, 64, x), h_ref, "tiny gate_up")
    h32 = h_ref.astype(np.float32)
    y_ref = oracle_lib.down(e, 4, 64, g.d_model, g.d_ff, h32.astype(np.float64))
    assert_parity(down_gpu(gq, de, 4, 64, h32), y_ref, "tiny down")
    out_ref = oracle_lib.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, x)
    assert_parity(run_ffn(gq, dev_experts(g), 4, 64, x), out_ref, "tiny expert FFN")


@pytest.mark.parametrize("spec", [workloads.Q4_GROUP8, workloads.Q2_GROUP8], ids=lambda s: s["name"])
def test_decode_group(gq, oracle_lib, spec):
    """8 routed experts at d_model 4096 / d_ff 1536, router-weighted sum, full output."""
    g, x, r = workloads.make_decode_inputs(spec)
    de = dev_experts(g)
    out_ref = oracle_lib.expert_ffn(g.experts, g.bits, 64, g.d_model, g.d_ff, x, r[None])
    assert_parity(run_ffn(gq, de, g.bits, 64, x, route=r), out_ref, spec["name"])
    for k in (0, len(g.experts) - 1):
        h_ref = oracle_lib.gate_up(g.experts[k], g.bits, 64, g.d_ff, g.d_model, x)
        assert_parity(gate_up_gpu(gq, de[k], g.bits, 64, x), h_ref, f"{spec['name']} gate_up e{k}")


def test_decode_group_deterministic_and_invariants(gq):
    """Repeated calls agree bitwise.  The experts' rows are added in ascending
    expert order in f64 from each expert's f32 row, and the sum is rounded to
    f32 once, so, bit for bit: doubling every down scale doubles every
    expert's row and so the output (a power of two commutes with every
    rounding), and a one-hot router reproduces the single-expert call."""
    g, x, r = workloads.make_decode_inputs(workloads.Q4_GROUP8)
    de = dev_experts(g)
    a = run_ffn(gq, de, 4, 64, x, route=r)
    b = run_ffn(gq, de, 4, 64, x, route=r)
    assert np.array_equal(a, b)
    de2 = [type(e)(e.gate, e.up, type(e.down)(e.down.codes, e.down.scales * 2)) for e in de]
    assert np.array_equal(run_ffn(gq, de2, 4, 64, x, route=r), 2 * a)
    onehot = np.zeros(8, np.float32)
    onehot[3] = 1.0
    sel = run_ffn(gq, de, 4, 64, x, route=onehot)
    solo = run_ffn(gq, de[3:4], 4, 64, x)
    assert np.array_equal(sel, solo)


def test_workspace_any_contents_and_reuse(gq, oracle_lib):
    """Nothing in the decode workspace needs to be zero: a workspace full of
    0xFF bytes (NaN patterns), reused across calls with 8 and 3 experts,
    gives the oracle's output and the same bits as a fresh zeroed one."""
    import torch
    g, x, r = workloads.make_decode_inputs(workloads.Q4_GROUP8)
    de = dev_experts(g)
    nbytes = gq.smoe_expert_ffn_workspace(8, g.d_model, g.d_ff, 1)
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
    out = torch.empty(g.d_model, dtype=torch.float32, device="cuda")
    xd, rd = dev(x), dev(r)
    results = []
    for i in range(4):
        gq.smoe_expert_ffn(de, 4, 64, xd, out, route_w=rd, workspace=ws)
        torch.cuda.synchronize()
        results.append(out.cpu().numpy().copy())
        gq.smoe_expert_ffn(de[:3], 4, 64, xd, out, route_w=rd[:3].contiguous(), workspace=ws)
    torch.cuda.synchronize()
    three = out.cpu().numpy().copy()
    for res in results[1:]:
        assert np.array_equal(res, results[0])
    assert np.array_equal(results[0], run_ffn(gq, de, 4, 64, x, route=r)), "0xFF workspace vs a zeroed one"
    want = oracle_lib.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, x, r[None])
    assert_parity(results[0], want, "8 experts on a reused 0xFF workspace")
    want3 = oracle_lib.expert_ffn(g.experts[:3], 4, 64, g.d_model, g.d_ff, x, r[None, :3])
    assert_parity(three, want3, "3 experts on the same workspace")


@pytest.fixture(scope="module", params=[workloads.Q4_GROUP8, workloads.Q2_GROUP8], ids=lambda s: s["name"])
def group8(request):
    g, x, r = workloads.make_decode_inputs(request.param)
    return g, x, r, dev_experts(g)


def _magnitude_cases(x):
    x = x.astype(np.float64)
    big = x.copy()
    big[37] = 2.0 ** 30          # one element 2^30 above the rest of its 32-column chunk
    # (Much further out, the f32 hidden vector itself overflows or underflows:
    # h is about x^2 times the weights squared.)
    return [("x*2^30", x * 2.0 ** 30), ("x*2^-30", x * 2.0 ** -30), ("one element 2^30", big)]


def test_decode_magnitudes(gq, oracle_lib, group8):
    """The 8-expert group (4- and 2-bit) with x scaled far from 1 and with one
    element far above the rest of its chunk: the output matches the oracle to
    the expected level at its own scale (the per-chunk fixed point and the
    expert sum have no range limit), and each call is followed by a normal
    call on the same workspace that matches the oracle as usual.  An all-zero
    x gives exactly zero."""
    import torch
    g, x, r, de = group8
    nbytes = gq.smoe_expert_ffn_workspace(8, g.d_model, g.d_ff, 1)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(g.d_model, dtype=torch.float32, device="cuda")
    rd = dev(r)

    def call(xv):
        gq.smoe_expert_ffn(de, g.bits, 64, dev(np.asarray(xv, np.float32)), out, route_w=rd, workspace=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy().copy()

    normal = oracle_lib.expert_ffn(g.experts, g.bits, 64, g.d_model, g.d_ff, x, r[None])
    for name, xv in _magnitude_cases(x):
        xv32 = xv.astype(np.float32)
        want = oracle_lib.expert_ffn(g.experts, g.bits, 64, g.d_model, g.d_ff, xv32, r[None])
        assert_relative(call(xv32), want, f"Q{g.bits} group, {name}")
        assert_parity(call(x), normal, f"Q{g.bits} group, normal call after {name}")
    assert not np.any(call(np.zeros(g.d_model, np.float32))), "all-zero x"
    assert_parity(call(x), normal, f"Q{g.bits} group, normal call after zero x")


@pytest.mark.parametrize("bad", ["nan", "inf", "-inf"])
def test_decode_nonfinite_input(gq, oracle_lib, group8, bad):
    """A non-finite element of x: the output is non-finite where the oracle's
    is (every row, since every weight is nonzero), for the 8-expert call and
    for smoe_gate_up; the next normal call on the same workspace is exact as
    usual."""
    import torch
    g, x, r, de = group8
    xb = x.copy()
    xb[1000] = np.float32(bad)
    nbytes = gq.smoe_expert_ffn_workspace(8, g.d_model, g.d_ff, 1)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(g.d_model, dtype=torch.float32, device="cuda")
    gq.smoe_expert_ffn(de, g.bits, 64, dev(xb), out, route_w=dev(r), workspace=ws)
    torch.cuda.synchronize()
    want = oracle_lib.expert_ffn(g.experts, g.bits, 64, g.d_model, g.d_ff, xb, r[None])
    assert not np.any(np.isfinite(want))
    assert_nonfinite_like(out.cpu().numpy(), want, f"Q{g.bits} group, x[1000]={bad}")
    h_want = oracle_lib.gate_up(g.experts[0], g.bits, 64, g.d_ff, g.d_model, xb)
    assert_nonfinite_like(gate_up_gpu(gq, de[0], g.bits, 64, xb), h_want, f"Q{g.bits} gate_up, x[1000]={bad}")
    gq.smoe_expert_ffn(de, g.bits, 64, dev(x), out, route_w=dev(r), workspace=ws)
    torch.cuda.synchronize()
    normal = oracle_lib.expert_ffn(g.experts, g.bits, 64, g.d_model, g.d_ff, x, r[None])
    assert_parity(out.cpu().numpy(), normal, f"Q{g.bits} group, normal call after {bad}")


def test_single_expert_per_expert_call(gq, oracle_lib):
    """One expert of the 4096 / 1536 group on its own (the unit a GPU holds
    when the group is split by expert), router weight absent (1)."""
    g, x, _ = workloads.make_decode_inputs(workloads.Q4_GROUP8)
    de = dev_experts(g)
    for k in (0, 5):
        want = oracle_lib.expert_ffn([g.experts[k]], 4, 64, g.d_model, g.d_ff, x)
        assert_parity(run_ffn(gq, [de[k]], 4, 64, x), want, f"Q4 expert {k} alone")


EDGE = [  # bits, group, d_model, d_ff, n_experts
    (4, 32, 96, 160, 3),      # three / five 16-byte chunks per row: ragged slices
    (2, 64, 192, 320, 2),
    (4, 128, 512, 384, 1),
    (2, 128, 256, 768, 5),
    (4, 64, 256, 64, 16),     # the most experts one call takes
    (4, 64, 8192, 128, 1),    # the widest gate/up row
    (2, 64, 8192, 128, 1),
    (4, 64, 64, 8192, 2),     # the widest down row
    (4, 64, 1536, 4096, 8),   # down rows wider than gate/up rows
    (4, 32, 32, 32, 1),       # a single chunk per row
]


@pytest.mark.parametrize("bits,group,d_model,d_ff,n", EDGE,
                         ids=lambda v: str(v))
def test_edge_shapes(gq, oracle_lib, bits, group, d_model, d_ff, n):
    g = workloads.expert_group(100 + d_model + d_ff + n, n, d_model, d_ff, bits, group)
    x = workloads.activation(7, d_model)
    r = workloads.router_weights(8, n)[0]
    out_ref = oracle_lib.expert_ffn(g.experts, bits, group, d_model, d_ff, x, r[None])
    assert_parity(run_ffn(gq, dev_experts(g), bits, group, x, route=r), out_ref,
                  f"edge Q{bits} g{group} {d_model}x{d_ff} E{n}")


def test_gpu_refuses_misaligned_codes(gq):
    import torch
    g, x, _ = workloads.make_decode_inputs(workloads.TINY)
    de = dev_experts(g)[0]
    flat = torch.empty(de.gate.codes.numel() + 16, dtype=torch.uint8, device="cuda")
    shifted = flat[8:8 + de.gate.codes.numel()].view(de.gate.codes.shape)
    h = torch.empty(g.d_ff, dtype=torch.float32, device="cuda")
    with pytest.raises(gq.SmoeError) as ei:
        gq.smoe_gate_up(shifted, de.gate.scales, de.up.codes, de.up.scales, 4, 64, dev(x), h)
    assert ei.value.status == -5


def test_decode_every_maximum(gq, oracle_lib):
    """One decode call at every shape limit at once: 16 experts (the most one
    call takes) whose gate, up and down matrices are all 8192 x 8192 (the
    widest rows on both passes), 4-bit codes, about 1.6 GB of weights; every
    output row against the oracle."""
    g = workloads.expert_group(4401, 16, 8192, 8192, 4, 64)
    x = workloads.activation(4402, 8192)
    r = workloads.router_weights(4403, 16)[0]
    want = oracle_lib.expert_ffn(g.experts, 4, 64, 8192, 8192, x, r[None])
    assert_parity(run_ffn(gq, dev_experts(g), 4, 64, x, route=r), want, "decode 16 experts of 8192 x 8192")
