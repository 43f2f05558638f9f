"""GPU parity of the routed (top-k) token batch against the f64 oracle,
through the C ABI: each token runs only through its slots' experts, and its
output is the router-weighted sum of those experts' FFNs."""
import numpy as np
import pytest

import workloads
from gpu_helpers import assert_parity, dev, dev_experts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gq():
    import torch
    import group_quantized_moe_amd as gq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gq.lib()
    return gq


@pytest.fixture(scope="module")
def q4_group8():
    g = workloads.make_group(workloads.Q4_GROUP8)
    return g, dev_experts(g)


def run_routed(gq, de, bits, group, X, ids, w):
    import torch
    X = np.asarray(X, np.float32)
    T, d_model = X.shape
    d_ff = de[0].gate.codes.shape[0]
    out = torch.empty(T * d_model, dtype=torch.float32, device="cuda")
    ws = torch.empty(gq.smoe_routed_ffn_workspace(len(de), d_model, d_ff, T, ids.shape[1]), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0xA5)   # nothing in the workspace needs to be zero: fill it with garbage
    gq.smoe_routed_ffn(de, bits, group, dev(X), dev(np.asarray(ids, np.int32)), dev(np.asarray(w, np.float32)),
                       out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(T, d_model)


def test_routed_prefill_workload(gq, oracle_lib, q4_group8):
    """256 tokens, top-2 of 8 Q4 experts: every token against the oracle, and
    a second call bit for bit equal (deterministic)."""
    g, de = q4_group8
    cfg = workloads.ROUTED
    X, ids, w = workloads.make_routed_inputs(cfg["T"], cfg["top_k"], cfg["seed"])
    got = run_routed(gq, de, 4, 64, X, ids, w)
    want = oracle_lib.routed_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X, ids, w)
    assert_parity(got, want, "routed T=256 top-2 (every token)")
    assert np.array_equal(got, run_routed(gq, de, 4, 64, X, ids, w))


@pytest.mark.parametrize("k", [4, 8])
def test_routed_prefill_top4_top8(gq, oracle_lib, q4_group8, k):
    """256 tokens, top-4 and top-8 of 8 Q4 experts (32- and 64-token tiles):
    every token against the oracle."""
    g, de = q4_group8
    X, ids, w = workloads.make_routed_inputs(256, k, 4251 + k)
    got = run_routed(gq, de, 4, 64, X, ids, w)
    want = oracle_lib.routed_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X, ids, w)
    assert_parity(got, want, f"routed T=256 top-{k} (every token)")


def test_routed_full_routing_equals_dense(gq, q4_group8):
    """Every token to every expert with the dense router's weights is the
    dense token batch (different kernels and order: within the bar)."""
    g, de = q4_group8
    X, R = workloads.make_batch_inputs(16)
    ids = np.tile(np.arange(8, dtype=np.int32), (16, 1))
    got = run_routed(gq, de, 4, 64, X, ids, R)
    import torch
    from gpu_helpers import run_ffn
    assert_parity(got, run_ffn(gq, de, 4, 64, X, route=R).reshape(16, -1), "routed full vs dense")


ROUTED_EDGE = [  # bits, group, d_model, d_ff, n_experts, T, top_k, routing
    (4, 64, 256, 512, 4, 1, 2, "topk"),
    (4, 64, 256, 512, 4, 5, 1, "topk"),
    (4, 32, 96, 160, 3, 33, 2, "topk"),
    (2, 64, 256, 384, 4, 70, 3, "topk"),
    (4, 64, 256, 512, 6, 40, 2, "skewed"),      # every token's first slot on expert 0
    (4, 64, 256, 512, 4, 20, 3, "holes"),       # some slots out of range
    (4, 64, 8192, 128, 2, 9, 1, "topk"),
    (4, 64, 384, 320, 3, 50, 2, "topk"),       # 6 and 5 groups: partial iterations in routed mode
    (4, 64, 384, 320, 2, 200, 2, "topk"),      # 64-token tiles with gate_up split in 2 (finishing pass)
    # T <= 16 with d_ff <= 1536 (streaming kernels, one token tile per expert):
    (4, 64, 256, 512, 6, 12, 2, "sparse"),     # experts 2..5 without slots: their blocks have nothing to do
    (4, 64, 256, 512, 4, 9, 3, "holes"),       # slots out of range are never processed
    (2, 64, 256, 384, 4, 10, 2, "topk"),       # 2-bit codes
    (4, 32, 96, 160, 3, 7, 2, "topk"),         # 32-column groups, partial row tiles of an expert
    (4, 64, 64, 2048, 2, 8, 1, "topk"),        # d_ff 2048 > 1536: the tiled kernels instead
]


@pytest.mark.parametrize("bits,group,d_model,d_ff,n,T,k,routing", ROUTED_EDGE, ids=lambda v: str(v))
def test_routed_edge_shapes(gq, oracle_lib, bits, group, d_model, d_ff, n, T, k, routing):
    g = workloads.expert_group(700 + d_model + T, n, d_model, d_ff, bits, group)
    X = workloads.activation_batch(701 + T, T, d_model)
    ids, w = workloads.top_k_routing(702 + T, T, n, k)
    if routing == "skewed":
        ids[:, 0] = 0
        ids[:, 1] = np.where(ids[:, 1] == 0, 1, ids[:, 1])
    if routing == "holes":
        ids[::3, 1] = -1
        ids[1::4, 2] = n
    if routing == "sparse":   # every token to experts 0 and 1 only
        ids[:, 0] = 0
        ids[:, 1] = 1
    got = run_routed(gq, dev_experts(g), bits, group, X, ids, w)
    want = oracle_lib.routed_ffn(g.experts, bits, group, d_model, d_ff, X, ids, w)
    assert_parity(got, want, f"routed Q{bits} g{group} {d_model}x{d_ff} E={n} T={T} k={k} {routing}")


def test_routed_f16_scales_and_duplicate_tokens(gq, oracle_lib):
    """f16 scales on the routed path; equal tokens with equal routing give
    equal rows."""
    g = workloads.expert_group(710, 4, 256, 512, 4, 64, scale_f16=True)
    X = workloads.activation_batch(711, 12, 256)
    X[7] = X[2]
    ids, w = workloads.top_k_routing(712, 12, 4, 2)
    ids[7], w[7] = ids[2], w[2]
    got = run_routed(gq, dev_experts(g), 4 | gq.SMOE_SCALE_F16, 64, X, ids, w)
    assert_parity(got, oracle_lib.routed_ffn(g.experts, 4, 64, 256, 512, X, ids, w), "routed f16 scales")
    assert np.array_equal(got[7], got[2])


def test_cross_block_sums_repeated(gq, oracle_lib, q4_group8):
    """The sums that blocks hand to one another through the workspace (each
    writes its partial sums at agent scope, waits for them, then counts
    itself in; the block that completes the count adds them all), run 100
    times back to back on one workspace without a synchronisation between
    calls: every output bitwise equal to the first, the first against the
    oracle.  64 tokens x top-2 of 8 experts is the routed path with 16-token
    tiles, whose gate_up K splits are added this way; a 12-token batch with
    d_ff 8192 is the streaming down pass, whose six column chunks per row
    group are added this way."""
    import torch
    reps = 100
    g, de = q4_group8
    X, ids, w = workloads.make_routed_inputs(64, 2, 4301)
    want = oracle_lib.routed_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X, ids, w)
    Xd, idd, wd = dev(X), dev(ids), dev(w)
    ws = torch.empty(gq.smoe_routed_ffn_workspace(8, g.d_model, g.d_ff, 64, 2), dtype=torch.uint8, device="cuda")
    outs = torch.empty(reps, 64 * g.d_model, dtype=torch.float32, device="cuda")
    for r in range(reps):
        gq.smoe_routed_ffn(de, 4, 64, Xd, idd, wd, outs[r], ws)
    torch.cuda.synchronize()
    got = outs.cpu().numpy()
    assert_parity(got[0].reshape(64, -1), want, "routed T=64 top-2, first of 100 calls")
    for r in range(1, reps):
        assert np.array_equal(got[r], got[0]), f"routed T=64 top-2: call {r} differs from the first"

    gs = workloads.expert_group(4302, 2, 64, 8192, 4, 64)
    Xs = workloads.activation_batch(4303, 12, 64)
    Rs = workloads.router_weights(4304, 2, 12)
    wants = oracle_lib.expert_ffn(gs.experts, 4, 64, 64, 8192, Xs, Rs)
    des, Xsd, Rsd = dev_experts(gs), dev(Xs), dev(Rs)
    ws2 = torch.empty(gq.smoe_expert_ffn_workspace(2, 64, 8192, 12), dtype=torch.uint8, device="cuda")
    outs2 = torch.empty(reps, 12 * 64, dtype=torch.float32, device="cuda")
    for r in range(reps):
        gq.smoe_expert_ffn(des, 4, 64, Xsd, outs2[r], route_w=Rsd, workspace=ws2)
    torch.cuda.synchronize()
    got2 = outs2.cpu().numpy()
    assert_parity(got2[0].reshape(12, -1), wants, "batch T=12 d_ff 8192, first of 100 calls")
    for r in range(1, reps):
        assert np.array_equal(got2[r], got2[0]), f"batch T=12 d_ff 8192: call {r} differs from the first"


def test_routed_most_tokens(gq, oracle_lib):
    """65536 tokens, top-2 of 4 small Q4 experts (32768 slots per expert on
    average): every token against the oracle."""
    T = 65536
    g = workloads.expert_group(4421, 4, 64, 128, 4, 64)
    X = workloads.activation_batch(4412, T, 64)
    ids, w = workloads.top_k_routing(4422, T, 4, 2)
    want = oracle_lib.routed_ffn(g.experts, 4, 64, 64, 128, X, ids, w)
    assert_parity(run_routed(gq, dev_experts(g), 4, 64, X, ids, w), want, "routed T=65536 top-2")
