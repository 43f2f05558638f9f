"""Invariants of the oracle that hold exactly (power-of-two scaling commutes
with rounding; mirroring every code negates every weight exactly), on the
workload shapes and distributions the benchmark uses."""
import numpy as np
import pytest

import workloads
from pins import pack_bits, unpack_bits


@pytest.fixture(scope="module")
def tiny(oracle_lib):
    g, x, _ = workloads.make_decode_inputs(workloads.TINY)
    return oracle_lib, g, x


def _scaled(m, f):
    return workloads.QMat(m.codes, (m.scales * np.float32(f)).astype(np.float32))


def test_up_scale_doubling_doubles_hidden_bitwise(tiny):
    O, g, x = tiny
    e = g.experts[0]
    h = O.gate_up(e, g.bits, g.group, g.d_ff, g.d_model, x)
    e2 = workloads.Expert(e.gate, _scaled(e.up, 2.0), e.down)
    h2 = O.gate_up(e2, g.bits, g.group, g.d_ff, g.d_model, x)
    assert np.array_equal(h2, 2.0 * h)


def test_down_scale_doubling_doubles_out_bitwise(tiny):
    O, g, x = tiny
    e = g.experts[0]
    out = O.expert_ffn([e], g.bits, g.group, g.d_model, g.d_ff, x)
    e2 = workloads.Expert(e.gate, e.up, _scaled(e.down, 2.0))
    out2 = O.expert_ffn([e2], g.bits, g.group, g.d_model, g.d_ff, x)
    assert np.array_equal(out2, 2.0 * out)


@pytest.mark.parametrize("bits", [4, 2])
def test_code_mirror_negates_projection(oracle_lib, bits):
    """code -> (2^b - 1) - code maps (code - Z) to -(code - Z) exactly."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 1 << bits, size=(16, 256), dtype=np.uint8)
    scales = rng.uniform(0.01, 0.05, size=(16, 4)).astype(np.float32)
    x = rng.standard_normal(256)
    y = oracle_lib.qmatvec(pack_bits(codes, bits), scales, bits, 64, 16, 256, x)
    ym = oracle_lib.qmatvec(pack_bits((1 << bits) - 1 - codes, bits), scales, bits, 64, 16, 256, x)
    assert np.array_equal(ym, -y)


def test_bf16_input_doubling_bitwise(oracle_lib):
    W, x = workloads.make_bf16(64, 256, seed=30)
    y = oracle_lib.matvec_bf16(W, x)
    y2 = oracle_lib.matvec_bf16(W, (2 * x).astype(np.float32))
    assert np.array_equal(y2, 2 * y)


def test_token_batch_rows_equal_single_token(oracle_lib):
    g, x, _ = workloads.make_decode_inputs(workloads.TINY)
    X = workloads.activation_batch(9, 3, g.d_model)
    out = oracle_lib.expert_ffn(g.experts, g.bits, g.group, g.d_model, g.d_ff, X)
    for t in range(3):
        one = oracle_lib.expert_ffn(g.experts, g.bits, g.group, g.d_model, g.d_ff, X[t])
        assert np.array_equal(out[t], one)


def test_router_permutation(oracle_lib):
    """Reordering experts together with their router weights changes only the
    order of the combine sum."""
    spec = dict(workloads.TINY, n_experts=3, seed=12)
    g, x, r = workloads.make_decode_inputs(spec)
    out = oracle_lib.expert_ffn(g.experts, g.bits, g.group, g.d_model, g.d_ff, x, r[None])
    perm = [2, 0, 1]
    outp = oracle_lib.expert_ffn([g.experts[k] for k in perm], g.bits, g.group, g.d_model,
                                 g.d_ff, x, r[perm][None])
    assert np.max(np.abs(out - outp)) <= 1e-14 * max(1.0, np.max(np.abs(out)))


def test_dequant_matches_bit_level_route(oracle_lib):
    g, _, _ = workloads.make_decode_inputs(workloads.TINY)
    m = g.experts[0].gate
    w = oracle_lib.dequant(m.codes, m.scales, 4, 64, g.d_ff, g.d_model)
    c = unpack_bits(m.codes, 4).astype(np.float64)
    want = (c - 7.5) / 7.5 * np.repeat(m.scales.astype(np.float64), 64, axis=1)
    assert np.array_equal(w, want)
