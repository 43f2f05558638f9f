"""GPU parity of the token-batch path (T > 1, matrix cores) against the f64
oracle, through the C ABI: the prefill workload (8 Q4 experts at d_model 4096 /
d_ff 1536, T = 16, 64, 256), ragged and edge shapes, and the per-token
invariants of the batch (a row equals the one-token result, duplicated tokens
give identical rows)."""
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


@pytest.fixture(scope="module")
def q4_group8():
    g = workloads.make_group(workloads.Q4_GROUP8)
    return g, dev_experts(g)


@pytest.mark.parametrize("T", sorted(workloads.BATCH_TOKENS))
def test_prefill_workload(gq, oracle_lib, q4_group8, T):
    """All T tokens through all 8 experts, router-weighted sum; every token
    against the oracle."""
    g, de = q4_group8
    X, R = workloads.make_batch_inputs(T)
    got = run_ffn(gq, de, 4, 64, X, route=R)
    want = oracle_lib.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X, R)
    assert_parity(got, want, f"prefill T={T} (every token)")


@pytest.mark.parametrize("k", [0, 7])
def test_prefill_single_expert(gq, oracle_lib, q4_group8, k):
    """One expert of the workload on its own (route weights absent = 1)."""
    g, de = q4_group8
    X, _ = workloads.make_batch_inputs(16)
    got = run_ffn(gq, [de[k]], 4, 64, X)
    want = oracle_lib.expert_ffn([g.experts[k]], 4, 64, g.d_model, g.d_ff, X)
    assert_parity(got, want, f"prefill T=16 expert {k} alone")


def test_batch_rows_match_decode_and_duplicates(gq, q4_group8):
    """Row t of a batch equals the decode result for X[t] (within the bar: a
    different kernel); identical tokens in different tiles give identical rows."""
    g, de = q4_group8
    X, R = workloads.make_batch_inputs(16)
    Xd = np.concatenate([X, X[::-1], X[:5]])          # T = 37: three token tiles, ragged
    Rd = np.concatenate([R, R[::-1], R[:5]])
    got = run_ffn(gq, de, 4, 64, Xd, route=Rd)
    for t in range(16):
        assert np.array_equal(got[t], got[31 - t]), f"token {t} and its duplicate differ"
    for t in range(5):
        assert np.array_equal(got[t], got[32 + t]), f"token {t} and its duplicate differ"
    for t in (0, 9, 15):
        one = run_ffn(gq, de, 4, 64, X[t], route=R[t])
        assert_parity(got[t], one, f"batch row {t} vs decode")


def test_batch_deterministic(gq, q4_group8):
    g, de = q4_group8
    X, R = workloads.make_batch_inputs(64)
    a = run_ffn(gq, de, 4, 64, X, route=R)
    b = run_ffn(gq, de, 4, 64, X, route=R)
    assert np.array_equal(a, b)


def test_batch_workspace_any_contents_and_reuse(gq, oracle_lib, q4_group8):
    """Batches of at most 16 tokens add the down pass's chunk sums inside the
    kernel through per-row-group counters kept in the workspace, which every
    call zeroes itself: a workspace full of 0xFF bytes, reused for 16, 64 and
    again 16 tokens, gives the oracle's rows and the same bits as a fresh
    zeroed one."""
    import torch
    g, de = q4_group8
    X16, R16 = workloads.make_batch_inputs(16)
    X64, R64 = workloads.make_batch_inputs(64)
    nbytes = max(gq.smoe_expert_ffn_workspace(8, g.d_model, g.d_ff, T) for T in (16, 64))
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")

    def call(X, R):
        T = X.shape[0]
        out = torch.empty(T * g.d_model, dtype=torch.float32, device="cuda")
        gq.smoe_expert_ffn(de, 4, 64, dev(X), out, route_w=dev(R), workspace=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy().reshape(T, g.d_model)

    first = call(X16, R16)
    want = oracle_lib.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, X16, R16)
    assert_parity(first, want, "T=16 on a 0xFF workspace")
    mid = call(X64, R64)
    assert np.array_equal(mid, run_ffn(gq, de, 4, 64, X64, route=R64)), "T=64 on a reused workspace"
    again = call(X16, R16)
    assert np.array_equal(first, again), "T=16 after T=64 on the same workspace"
    assert np.array_equal(first, run_ffn(gq, de, 4, 64, X16, route=R16)), "0xFF workspace vs a zeroed one"


BATCH_EDGE = [  # bits, group, d_model, d_ff, n_experts, T
    (4, 64, 256, 512, 2, 2),
    (4, 64, 256, 512, 1, 17),
    (4, 32, 96, 160, 3, 5),
    (4, 32, 96, 160, 3, 33),
    (4, 64, 8192, 128, 1, 3),
    (4, 64, 64, 8192, 2, 18),
    (4, 64, 256, 64, 16, 4),
    (2, 64, 256, 384, 3, 20),
    (2, 64, 192, 128, 1, 65),
    (4, 64, 384, 320, 2, 9),     # 6 gate_up groups in 2 K splits (the second ends in a dead step), 5 down groups
    (2, 64, 320, 448, 3, 40),    # 5 and 7 groups: partial 4-group code units and scale quads on both passes
    # T <= 16 (streaming kernels):
    (2, 64, 256, 384, 3, 7),     # 2-bit codes, one phase of 4 groups (the rest of it dead)
    (4, 64, 64, 8192, 2, 12),    # d_ff 8192: six down chunks per expert, the last partial; half a row group
    (4, 32, 1088, 96, 2, 16),    # 34 groups: three phases (an odd count), the last partial; one sparse chunk
    (2, 64, 320, 448, 3, 16),    # 5 and 7 groups: a partial phase and a partial chunk, 2-bit codes
]


@pytest.mark.parametrize("bits,group,d_model,d_ff,n,T", BATCH_EDGE,
                         ids=lambda v: str(v))
def test_batch_edge_shapes(gq, oracle_lib, bits, group, d_model, d_ff, n, T):
    g = workloads.expert_group(100 + d_model + d_ff + T, n, d_model, d_ff, bits, group)
    X = workloads.activation_batch(200 + T, T, d_model)
    R = workloads.router_weights(300 + T, n, T)
    got = run_ffn(gq, dev_experts(g), bits, group, X, route=R)
    want = oracle_lib.expert_ffn(g.experts, bits, group, d_model, d_ff, X, R)
    assert_parity(got, want, f"batch Q{bits} g{group} {d_model}x{d_ff} E={n} T={T}")


def test_batch_extreme_magnitudes(gq, oracle_lib):
    """Tokens whose scale differs by 2^40 from each other, and an all-zero
    token: the per-group power-of-two scaling keeps each row to the bar of its
    own magnitude."""
    g = workloads.expert_group(7, 2, 256, 512, 4, 64)
    X = workloads.activation_batch(8, 6, 256).astype(np.float64)
    X[1] *= 2.0 ** 20
    X[2] *= 2.0 ** -20
    X[3] = 0.0
    X[4, :64] *= 2.0 ** 30   # one group of one token far above the rest
    X = X.astype(np.float32)
    got = run_ffn(gq, dev_experts(g), 4, 64, X)
    want = oracle_lib.expert_ffn(g.experts, 4, 64, 256, 512, X)
    for t in range(6):
        assert_parity(got[t], want[t], f"extreme token {t}")


def test_batch_refuses_unsupported_group(gq):
    """group 160 is a valid 4-bit group for decode but not for the batch tiling."""
    import torch
    g = workloads.expert_group(9, 1, 320, 160, 4, 160)
    de = dev_experts(g)
    X = dev(workloads.activation_batch(9, 4, 320))
    out = torch.empty(4 * 320, dtype=torch.float32, device="cuda")
    ws = torch.zeros(gq.smoe_expert_ffn_workspace(1, 320, 160, 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(gq.SmoeError) as ei:
        gq.smoe_expert_ffn(de, 4, 160, X, out, workspace=ws)
    assert ei.value.status == -3


def test_batch_most_tokens(gq, oracle_lib):
    """The largest batch a call takes, 65536 tokens (1024 tiles of 64), through
    two small Q4 experts: every token against the oracle."""
    T = 65536
    g = workloads.expert_group(4411, 2, 64, 128, 4, 64)
    X = workloads.activation_batch(4412, T, 64)
    R = workloads.router_weights(4413, 2, T)
    want = oracle_lib.expert_ffn(g.experts, 4, 64, 64, 128, X, R)
    assert_parity(run_ffn(gq, dev_experts(g), 4, 64, X, route=R), want, "batch T=65536")
