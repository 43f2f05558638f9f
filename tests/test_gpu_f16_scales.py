"""GPU parity of the 2-byte (IEEE binary16) scale layout, through the C ABI.

A matrix with f16 scales is the matrix whose f32 scales hold the same values,
so: the decode groups and the token batch with f16 scales match the oracle
(which widens the scales with its own binary16 decoder) within the bar, and
match the f32-scale path on the widened scales bit for bit (the kernels widen
each scale exactly and use it as an f32 scale).
"""
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


@pytest.fixture(scope="module", params=["q4", "q2"])
def groups(request):
    spec = workloads.Q4_GROUP8_S16 if request.param == "q4" else workloads.Q2_GROUP8_S16
    g = workloads.make_group(spec)
    assert g.experts[0].gate.scales.dtype == np.float16
    w = workloads.widened_scales(g)
    return spec, g, w, dev_experts(g), dev_experts(w)


def test_decode_group_f16_scales(gq, oracle_lib, groups):
    """The 8-expert decode group with f16 scales against the oracle, and bit
    for bit against the f32 path on the widened scales."""
    spec, g, w, dg, dw = groups
    _, x, r = workloads.make_decode_inputs(spec)
    got = run_ffn(gq, dg, g.bits | gq.SMOE_SCALE_F16, 64, x, route=r)
    want = oracle_lib.expert_ffn(g.experts, g.bits, 64, g.d_model, g.d_ff, x, r[None])
    assert_parity(got, want, f"{spec['name']} decode")
    assert np.array_equal(got, run_ffn(gq, dw, g.bits, 64, x, route=r))


@pytest.mark.parametrize("T", [16, 64])
def test_batch_f16_scales(gq, oracle_lib, groups, T):
    """Token batch with f16 scales: every token against the oracle and bit
    for bit against the f32 path."""
    spec, g, w, dg, dw = groups
    X, R = workloads.make_batch_inputs(T)
    got = run_ffn(gq, dg, g.bits | gq.SMOE_SCALE_F16, 64, X, route=R)
    want = oracle_lib.expert_ffn(g.experts, g.bits, 64, g.d_model, g.d_ff, X, R)
    assert_parity(got, want, f"{spec['name']} batch T={T} (every token)")
    assert np.array_equal(got, run_ffn(gq, dw, g.bits, 64, X, route=R))


def test_single_expert_entry_points_f16_scales(gq, oracle_lib):
    """smoe_gate_up and smoe_down with f16 scales, including a scale array that
    is 2-byte but not 4-byte aligned."""
    import torch
    g = workloads.expert_group(31, 1, 512, 384, 4, 64, scale_f16=True)
    e = g.experts[0]
    x = workloads.activation(31, 512)
    fmt = 4 | gq.SMOE_SCALE_F16
    up_s = torch.zeros(e.up.scales.size + 1, dtype=torch.float16, device="cuda")
    up_s[1:] = dev(e.up.scales).reshape(-1)            # data_ptr % 4 == 2
    hidden = torch.empty(384, dtype=torch.float32, device="cuda")
    gq.smoe_gate_up(dev(e.gate.codes), dev(e.gate.scales), dev(e.up.codes), up_s[1:], fmt, 64, dev(x), hidden)
    torch.cuda.synchronize()
    h_want = oracle_lib.gate_up(e, 4, 64, 384, 512, x)
    assert_parity(hidden.cpu().numpy(), h_want, "gate_up f16 scales")
    h32 = h_want.astype(np.float32)                     # the oracle's hidden is down's input
    out = torch.empty(512, dtype=torch.float32, device="cuda")
    gq.smoe_down(dev(e.down.codes), dev(e.down.scales), fmt, 64, dev(h32), out)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), oracle_lib.down(e, 4, 64, 512, 384, h32.astype(np.float64)), "down f16 scales")


def test_f16_scale_dtype_must_match_flag(gq):
    """The binding refuses f32 scale tensors with the f16 flag (and f16 without it)."""
    g = workloads.expert_group(32, 1, 256, 256, 4, 64, scale_f16=True)
    de = dev_experts(g)
    with pytest.raises(TypeError):
        run_ffn(gq, de, 4, 64, workloads.activation(32, 256))
    dw = dev_experts(workloads.widened_scales(g))
    with pytest.raises(TypeError):
        run_ffn(gq, dw, 4 | gq.SMOE_SCALE_F16, 64, workloads.activation(32, 256))
