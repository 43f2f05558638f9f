"""The no-allocation entry point smoe_expert_ffn_noalloc, through the C ABI:
it gives the same bits as smoe_expert_ffn with a caller workspace (the same
kernels run on the library's static scratch array instead), on two calls in a
row whose second is smaller, and refuses a call whose workspace would exceed
the array."""
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


def noalloc(gq, de, bits, group, x, route=None):
    import torch
    d_model = de[0].gate.codes.shape[1] * 8 // (bits & 0xFF)
    xd = dev(np.asarray(x, np.float32))
    T = xd.numel() // d_model
    out = torch.full((T * d_model,), float("nan"), dtype=torch.float32, device="cuda")
    rd = None if route is None else dev(np.asarray(route, np.float32))
    gq.smoe_expert_ffn_noalloc(de, bits, group, xd, out, route_w=rd)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(T, d_model) if T > 1 else out.cpu().numpy()


def test_noalloc_matches_workspace_entry_two_calls(gq, oracle_lib):
    """The Q4 8-expert group, then the smaller tiny expert, then a 2-token
    batch of a small expert: each bit for bit equal to smoe_expert_ffn with
    its own workspace, and within the bar of the oracle."""
    g, x, r = workloads.make_decode_inputs(workloads.Q4_GROUP8)
    de = dev_experts(g)
    big = noalloc(gq, de, 4, 64, x, r)
    assert np.array_equal(big, run_ffn(gq, de, 4, 64, x, route=r))
    assert_parity(big, oracle_lib.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, x, r[None]), "noalloc Q4 group")

    t, xt, _ = workloads.make_decode_inputs(workloads.TINY)
    dt = dev_experts(t)
    small = noalloc(gq, dt, 4, 64, xt)
    assert np.array_equal(small, run_ffn(gq, dt, 4, 64, xt))
    assert_parity(small, oracle_lib.expert_ffn(t.experts, 4, 64, t.d_model, t.d_ff, xt), "noalloc tiny, second call")

    sg = workloads.expert_group(901, 1, 256, 256, 4, 64)
    X = workloads.activation_batch(902, 2, 256)
    R = workloads.router_weights(903, 1, 2)
    assert gq.smoe_expert_ffn_workspace(1, 256, 256, 2) <= gq.SMOE_NOALLOC_SCRATCH_BYTES
    dsg = dev_experts(sg)
    batch = noalloc(gq, dsg, 4, 64, X, R)
    assert np.array_equal(batch, run_ffn(gq, dsg, 4, 64, X, route=R))
    assert_parity(batch, oracle_lib.expert_ffn(sg.experts, 4, 64, 256, 256, X, R), "noalloc 2-token batch")


def test_noalloc_refuses_beyond_the_array(gq):
    """The 64-token batch of the 8-expert group needs more scratch than the
    array holds: SMOE_ERR_WORKSPACE, and the output is untouched."""
    import torch
    g = workloads.make_group(workloads.Q4_GROUP8)
    assert gq.smoe_expert_ffn_workspace(8, g.d_model, g.d_ff, 64) > gq.SMOE_NOALLOC_SCRATCH_BYTES
    X, R = workloads.make_batch_inputs(64)
    out = torch.full((64 * g.d_model,), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(gq.SmoeError) as ei:
        gq.smoe_expert_ffn_noalloc(dev_experts(g), 4, 64, dev(X), out, route_w=dev(R))
    assert ei.value.status == -6
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
