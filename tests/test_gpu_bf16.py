"""GPU parity of the bf16 dense matvec against the f64 oracle, through the C ABI."""
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


def matvec_gpu(gq, W, x):
    import torch
    y = torch.empty(W.shape[0], dtype=torch.float32, device="cuda")
    gq.matvec_bf16(dev(W), dev(x), y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("rows,cols,role,seed", workloads.BF16_SHAPES, ids=lambda v: str(v))
def test_bf16_shapes(gq, oracle_lib, rows, cols, role, seed):
    W, x = workloads.make_bf16(rows, cols, seed)
    y = matvec_gpu(gq, W, x)
    assert_parity(y, oracle_lib.matvec_bf16(W, x), f"bf16 {role} {rows}x{cols}")


@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 24), (1000, 72), (37, 4104), (5, 16384), (4099, 512)])
def test_bf16_edge_shapes(gq, oracle_lib, rows, cols):
    W, x = workloads.make_bf16(rows, cols, seed=rows + cols)
    assert_parity(matvec_gpu(gq, W, x), oracle_lib.matvec_bf16(W, x), f"bf16 {rows}x{cols}")


def test_bf16_small_integers_exact(gq):
    """Integer weights and inputs: every partial sum is an exact f32 integer."""
    rng = np.random.default_rng(1)
    ints = rng.integers(-8, 9, size=(300, 4096)).astype(np.float32)
    W = (ints.view(np.uint32) >> 16).astype(np.uint16)
    x = rng.integers(-16, 17, size=4096).astype(np.float32)
    want = ints.astype(np.int64) @ x.astype(np.int64)
    assert np.array_equal(matvec_gpu(gq, W, x), want.astype(np.float32))


def test_bf16_input_doubling_bitwise(gq):
    W, x = workloads.make_bf16(512, 4096, 32)
    assert np.array_equal(matvec_gpu(gq, W, (2 * x).astype(np.float32)), 2 * matvec_gpu(gq, W, x))
