"""GPU parity of the decode path (one token) against the f64 oracle, through
the C ABI, on the workload shapes and on ragged / edge shapes."""
import numpy as np
import pytest

import workloads
from gpu_helpers import assert_parity, dev, dev_experts, run_ffn

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
    """Repeated calls agree bitwise.  The experts' outputs are summed exactly on
    a 2^-32 grid (each term rounded once to a multiple of 2^-32) and the sum is
    rounded to f32 once, so: doubling every down scale doubles the output to
    within that rounding (E * 2^-33 plus one f32 rounding of the result), and a
    one-hot router reproduces the single-expert call to within 2^-33."""
    import torch
    g, x, r = workloads.make_decode_inputs(workloads.Q4_GROUP8)
    de = dev_experts(g)
    a = run_ffn(gq, de, 4, 64, x, route=r)
    b = run_ffn(gq, de, 4, 64, x, route=r)
    assert np.array_equal(a, b)
    de2 = [type(e)(e.gate, e.up, type(e.down)(e.down.codes, e.down.scales * 2)) for e in de]
    a2 = run_ffn(gq, de2, 4, 64, x, route=r).astype(np.float64)
    bound = 8 * 2.0 ** -33 * 2 + np.spacing(np.abs(2 * a).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(a2 - 2 * a.astype(np.float64)) <= bound)
    onehot = np.zeros(8, np.float32)
    onehot[3] = 1.0
    sel = run_ffn(gq, de, 4, 64, x, route=onehot).astype(np.float64)
    solo = run_ffn(gq, de[3:4], 4, 64, x).astype(np.float64)
    assert np.all(np.abs(sel - solo) <= 2.0 ** -33 + np.spacing(np.abs(solo).astype(np.float32)))
    torch.cuda.synchronize()


def test_workspace_reuse_leaves_counters_zero(gq):
    """One workspace across many calls and shapes: every call gives the same
    result, and every synchronisation counter is back to zero afterwards."""
    import torch
    g, x, r = workloads.make_decode_inputs(workloads.Q4_GROUP8)
    de = dev_experts(g)
    nbytes = gq.smoe_expert_ffn_workspace(8, g.d_model, g.d_ff, 1)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(g.d_model, dtype=torch.float32, device="cuda")
    xd, rd = dev(x), dev(r)
    results = []
    for i in range(6):
        gq.smoe_expert_ffn(de, 4, 64, xd, out, route_w=rd, workspace=ws)
        torch.cuda.synchronize()
        results.append(out.cpu().numpy().copy())
        # a smaller call (3 experts) on the same workspace in between
        gq.smoe_expert_ffn(de[:3], 4, 64, xd, out, route_w=rd[:3].contiguous(), workspace=ws)
    torch.cuda.synchronize()
    for res in results[1:]:
        assert np.array_equal(res, results[0])
    # the hidden rows are scratch; the per-row expert accumulators that follow
    # them (one 64-bit word per output row) must be zero again
    hidden_bytes = -(-8 * g.d_ff * 4 // 256) * 256
    tail = ws[hidden_bytes:].cpu().numpy()
    assert tail.size >= 8 * g.d_model
    assert not tail.any(), "expert accumulators not reset"


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
