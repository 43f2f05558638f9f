"""GPU parity of the decode attention block (smoe_attn_decode) against the f64
oracle, through the C ABI: the output, the appended cache rows, and the rest of
the caches left untouched."""
import numpy as np
import pytest

import workloads
from gpu_helpers import assert_parity, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gq():
    import torch
    import group_quantized_moe_amd as gq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gq.lib()
    return gq


class Block:
    """Device copies of one workload's weights; run() appends at pos in the
    device caches it is given and returns the output."""

    def __init__(self, gq, spec, w):
        import torch
        self.gq, self.spec = gq, spec
        self.w = [dev(w.wq), dev(w.wk), dev(w.wv), dev(w.wo), dev(w.q_norm), dev(w.k_norm)]
        need = gq.smoe_attn_decode_workspace(spec["d_model"], spec["n_head"], spec["n_kv"], spec["head_dim"],
                                             spec["max_ctx"])
        assert need > 0
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        self.out = torch.empty(spec["d_model"], dtype=torch.float32, device="cuda")

    def run(self, x_dev, pos, Kd, Vd):
        import torch
        self.gq.smoe_attn_decode(*self.w, x_dev, pos, self.spec["rope_base"], Kd, Vd, self.out, self.ws)
        torch.cuda.synchronize()
        return self.out.cpu().numpy()


def check_block(gq, oracle_lib, spec, pos, what):
    w, x, K, V = workloads.make_attn_inputs(spec)
    blk = Block(gq, spec, w)
    Kd, Vd = dev(K), dev(V)
    out = blk.run(dev(x), pos, Kd, Vd)
    want, _, _, Kw, Vw = oracle_lib.attn_decode(w, x, pos, spec["rope_base"], K, V)
    assert_parity(out, want, f"{what} out")
    Kg, Vg = Kd.cpu().numpy(), Vd.cpu().numpy()
    assert_parity(Kg[:, pos], Kw[:, pos], f"{what} appended k")
    assert_parity(Vg[:, pos], Vw[:, pos], f"{what} appended v")
    rest = np.ones(spec["max_ctx"], bool)
    rest[pos] = False
    assert np.array_equal(Kg[:, rest], K[:, rest]) and np.array_equal(Vg[:, rest], V[:, rest]), \
        "cache rows other than pos changed"


@pytest.mark.parametrize("pos", [0, 1, 30, 31, 32, 33, 37, 63, 64, 99])
def test_attn_small_positions(gq, oracle_lib, pos):
    """Every chunk boundary of 32 positions, the first and the last cache row."""
    check_block(gq, oracle_lib, workloads.ATTN_SMALL, pos, f"attn small pos {pos}")


@pytest.mark.parametrize("shape", [
    dict(d_model=512, n_head=16, n_kv=1, head_dim=128, max_ctx=70, pos=69),    # 16 query heads per KV head
    dict(d_model=192, n_head=12, n_kv=4, head_dim=64, max_ctx=45, pos=44),     # 3 per KV head
    dict(d_model=256, n_head=2, n_kv=2, head_dim=128, max_ctx=33, pos=32),     # one per KV head
    dict(d_model=8, n_head=1, n_kv=1, head_dim=64, max_ctx=5, pos=3),          # the smallest projections
], ids=lambda s: f"h{s['n_head']}kv{s['n_kv']}d{s['head_dim']}m{s['d_model']}")
def test_attn_group_shapes(gq, oracle_lib, shape):
    spec = dict(shape, seed=52 + shape["n_head"], rope_base=1e4, name="shape")
    check_block(gq, oracle_lib, spec, spec["pos"], f"attn {spec['n_head']}/{spec['n_kv']} heads")


@pytest.mark.parametrize("pos", [0, 2047, 4095])
def test_attn_full_block(gq, oracle_lib, pos):
    """The 64/4-head, 128-dim block over a 4096-position cache, as benchmarked."""
    spec = workloads.ATTN
    check_block(gq, oracle_lib, spec, pos, f"attn full pos {pos}")


@pytest.mark.parametrize("pos", [8191, 16383])
def test_attn_long_context(gq, oracle_lib, pos):
    """A 16384-position cache (512 chunks of 32, merged in 32 ranges of 16):
    the last position and one in the middle of the cache."""
    spec = dict(d_model=256, n_head=8, n_kv=2, head_dim=64, max_ctx=16384, seed=61, rope_base=1e6,
                name="long")
    check_block(gq, oracle_lib, spec, pos, f"attn long context pos {pos}")


def test_attn_sequential_decode(gq, oracle_lib):
    """Forty tokens decoded in turn from an empty cache: each side keeps its own
    cache, and every step's output and appended rows agree."""
    spec = dict(workloads.ATTN_SMALL, max_ctx=40)
    w, _, _, _ = workloads.make_attn_inputs(spec)
    blk = Block(gq, spec, w)
    shape = (spec["n_kv"], spec["max_ctx"], spec["head_dim"])
    K, V = np.zeros(shape, np.float32), np.zeros(shape, np.float32)
    Kd, Vd = dev(K), dev(V)
    xs = workloads.activation_batch(spec["seed"], spec["max_ctx"], spec["d_model"])
    for pos in range(spec["max_ctx"]):
        out = blk.run(dev(xs[pos]), pos, Kd, Vd)
        want, _, _, K, V = oracle_lib.attn_decode(w, xs[pos], pos, spec["rope_base"], K, V)
        assert_parity(out, want, f"sequential step {pos}")
    assert_parity(Kd.cpu().numpy(), K, "sequential K cache")
    assert_parity(Vd.cpu().numpy(), V, "sequential V cache")


def test_attn_deterministic(gq):
    """Two calls on the same inputs give the same bits (the chunk merge runs in
    a fixed order; nothing accumulates atomically)."""
    spec = workloads.ATTN_SMALL
    w, x, K, V = workloads.make_attn_inputs(spec)
    blk = Block(gq, spec, w)
    a = blk.run(dev(x), 77, dev(K), dev(V))
    b = blk.run(dev(x), 77, dev(K), dev(V))
    assert np.array_equal(a, b)
