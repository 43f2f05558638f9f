"""The seeded input generator: reproducible, correctly shaped, right distributions."""
import numpy as np

import workloads


def test_reproducible_and_independent_streams():
    a = workloads.random_bytes(1, (0, 0, 0), 1000)
    b = workloads.random_bytes(1, (0, 0, 0), 1000)
    c = workloads.random_bytes(1, (0, 1, 0), 1000)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_decode_shapes_and_distributions():
    g, x, r = workloads.make_decode_inputs(workloads.TINY)
    e = g.experts[0]
    assert e.gate.codes.shape == (512, 128) and e.gate.scales.shape == (512, 4)
    assert e.down.codes.shape == (256, 256) and e.down.scales.shape == (256, 8)
    assert x.shape == (256,) and x.dtype == np.float32
    assert 0.01 <= e.gate.scales.min() and e.gate.scales.max() < 0.05
    nib = np.concatenate([e.gate.codes & 15, e.gate.codes >> 4]).astype(np.float64)
    assert abs(nib.mean() - 7.5) < 0.1
    assert abs(float(r.sum()) - 1.0) < 1e-6


def test_normal_moments():
    z = workloads.normal_f32(3, (9,), 200_000).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01


def test_bf16_rounding_ties_to_even():
    f = np.array([1.0, 1.00390625, 1.01171875, -2.5], np.float32)  # 1+2^-8 is a tie
    bits = workloads.f32_to_bf16_bits(f)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def test_attn_inputs_shapes_and_determinism():
    spec = workloads.ATTN_SMALL
    w, x, K, V = workloads.make_attn_inputs(spec)
    nq, nk, hd = spec["n_head"] * spec["head_dim"], spec["n_kv"] * spec["head_dim"], spec["head_dim"]
    assert w.wq.shape == (nq, spec["d_model"]) and w.wq.dtype == np.uint16
    assert w.wk.shape == w.wv.shape == (nk, spec["d_model"])
    assert w.wo.shape == (spec["d_model"], nq)
    assert w.q_norm.shape == w.k_norm.shape == (hd,) and w.q_norm.dtype == np.float32
    assert K.shape == V.shape == (spec["n_kv"], spec["max_ctx"], hd) and K.dtype == np.float32
    w2, x2, K2, _ = workloads.make_attn_inputs(spec)
    assert np.array_equal(w.wo, w2.wo) and np.array_equal(x, x2) and np.array_equal(K, K2)
    assert not np.array_equal(K, V)
