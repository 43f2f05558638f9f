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


# ---------------------------------------------------------------------------
# matvec_bf16_batch: several independent matvecs in one launch.

def batch_gpu(gq, jobs):
    """jobs: list of (W bits uint16 [rows, cols], x f32 [cols]); a job may pass
    the same numpy array object as an earlier job to share its device copy."""
    import torch
    dW, dx, triples = {}, {}, []
    for W, x in jobs:
        Wd = dW.setdefault(id(W), dev(W))
        xd = dx.setdefault(id(x), dev(x))
        triples.append((Wd, xd, torch.empty(W.shape[0], dtype=torch.float32, device="cuda")))
    gq.matvec_bf16_batch(triples)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for _, _, y in triples]


def test_bf16_batch_qkv(gq, oracle_lib):
    """q, k and v projections of one token over a shared x, one launch."""
    Ws, x = workloads.make_bf16_batch()
    ys = batch_gpu(gq, [(W, x) for W in Ws])
    for (rows, cols, role, _), W, y in zip(workloads.BF16_BATCH, Ws, ys):
        assert_parity(y, oracle_lib.matvec_bf16(W, x), f"batch {role} {rows}x{cols}")


BATCH_MIXED = [(1, 8), (3, 24), (1000, 72), (37, 4104), (5, 16384), (4099, 512), (512, 4096)]


def test_bf16_batch_mixed_shapes(gq, oracle_lib):
    """Different rows and cols in one launch (the lane map is the widest
    job's), each job with its own x."""
    jobs = [workloads.make_bf16(r, c, seed=500 + r + c) for r, c in BATCH_MIXED]
    ys = batch_gpu(gq, jobs)
    for (r, c), (W, x), y in zip(BATCH_MIXED, jobs, ys):
        assert_parity(y, oracle_lib.matvec_bf16(W, x), f"batch job {r}x{c}")


def test_bf16_batch_sixteen_jobs_shared_weight(gq, oracle_lib):
    """The job limit, with one W shared by all jobs and a different x each:
    job j equals the single matvec of its own x within the bar, and equal
    inputs give equal outputs."""
    W, _ = workloads.make_bf16(300, 2048, seed=77)
    xs = [workloads.make_bf16(8, 2048, seed=600 + j)[1] for j in range(15)]
    xs.append(xs[3])
    ys = batch_gpu(gq, [(W, x) for x in xs])
    for j, (x, y) in enumerate(zip(xs, ys)):
        assert_parity(y, oracle_lib.matvec_bf16(W, x), f"shared-W job {j}")
        assert_parity(y, matvec_gpu(gq, W, x), f"shared-W job {j} vs single call")
    assert np.array_equal(ys[15], ys[3])


def test_bf16_batch_small_integers_exact(gq):
    """Integer weights and inputs are exact in every job of a batch."""
    rng = np.random.default_rng(2)
    jobs, wants = [], []
    for rows, cols in [(300, 4096), (17, 1024), (64, 8)]:
        ints = rng.integers(-8, 9, size=(rows, cols)).astype(np.float32)
        W = (ints.view(np.uint32) >> 16).astype(np.uint16)
        x = rng.integers(-16, 17, size=cols).astype(np.float32)
        jobs.append((W, x))
        wants.append((ints.astype(np.int64) @ x.astype(np.int64)).astype(np.float32))
    for y, want in zip(batch_gpu(gq, jobs), wants):
        assert np.array_equal(y, want)
