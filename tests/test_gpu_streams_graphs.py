"""The library's calls under concurrency and HIP graph capture, through the C
ABI.  A call keeps no state between calls beyond its workspace (the one-token
path needs nothing zeroed; the token batch zeroes its own counters with a
kernel, not a memset), so:

- calls on two streams at once, each with its own workspace, give bitwise the
  results they give alone;
- a captured graph of calls (the decode group, the same through the
  no-allocation entry point, a 16-token batch) replays to bitwise the eager
  results, replay after replay, with new inputs copied into its input
  buffers and other work on the device between the replays.
"""
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
def setup(gq):
    import torch
    g, x1, r = workloads.make_decode_inputs(workloads.Q4_GROUP8)
    x2 = workloads.activation(77, g.d_model)
    X1, R16 = workloads.make_batch_inputs(16)
    X2 = workloads.activation_batch(78, 16, g.d_model)
    de = dev_experts(g)
    ws1 = torch.empty(gq.smoe_expert_ffn_workspace(8, g.d_model, g.d_ff, 1), dtype=torch.uint8, device="cuda")
    ws16 = torch.empty(gq.smoe_expert_ffn_workspace(8, g.d_model, g.d_ff, 16), dtype=torch.uint8, device="cuda")
    return dict(g=g, de=de, x1=x1, x2=x2, r_np=r, r=dev(r), X1=X1, X2=X2, R16_np=R16, R16=dev(R16),
                ws1=ws1, ws16=ws16)


def _decode(gq, s, x, out, stream=None):
    gq.smoe_expert_ffn(s["de"], 4, 64, x, out, route_w=s["r"], workspace=s["ws1"], stream=stream)


def _batch(gq, s, X, out, stream=None):
    gq.smoe_expert_ffn(s["de"], 4, 64, X, out, route_w=s["R16"], workspace=s["ws16"], stream=stream)


def _eager(gq, s):
    """Decode and batch results for both inputs, one call at a time on the default stream."""
    import torch
    d = s["g"].d_model
    res = {}
    for name, x in (("x1", s["x1"]), ("x2", s["x2"])):
        out = torch.empty(d, dtype=torch.float32, device="cuda")
        _decode(gq, s, dev(x), out)
        torch.cuda.synchronize()
        res[name] = out.cpu().numpy()
    for name, X in (("X1", s["X1"]), ("X2", s["X2"])):
        out = torch.empty(16 * d, dtype=torch.float32, device="cuda")
        _batch(gq, s, dev(X), out)
        torch.cuda.synchronize()
        res[name] = out.cpu().numpy()
    return res


def test_two_streams_at_once(gq, oracle_lib, setup):
    """The decode group on one stream and the 16-token batch on another, 20
    calls each, interleaved on the host so that the GPU runs them side by
    side: both outputs are bitwise the single-stream ones."""
    import torch
    s = setup
    ref = _eager(gq, s)
    g = s["g"]
    want = oracle_lib.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, s["x1"], s["r_np"])
    assert_parity(ref["x1"], want, "decode group, single stream")
    want = oracle_lib.expert_ffn(g.experts, 4, 64, g.d_model, g.d_ff, s["X1"], s["R16_np"])
    assert_parity(ref["X1"].reshape(16, g.d_model), want, "16-token batch, single stream")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    xa, Xb = dev(s["x1"]), dev(s["X1"])
    oa = torch.empty(g.d_model, dtype=torch.float32, device="cuda")
    ob = torch.empty(16 * g.d_model, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(20):
        with torch.cuda.stream(sa):
            _decode(gq, s, xa, oa)
        with torch.cuda.stream(sb):
            _batch(gq, s, Xb, ob)
    torch.cuda.synchronize()
    assert np.array_equal(oa.cpu().numpy(), ref["x1"]), "decode on a second stream differs"
    assert np.array_equal(ob.cpu().numpy(), ref["X1"]), "batch on a second stream differs"


def test_graph_replays(gq, setup):
    """One captured graph holding the decode group, the same decode through
    smoe_expert_ffn_noalloc (its scratch array instead of the workspace) and
    the 16-token batch.  Five replays, with the inputs switched between two
    vectors / token sets by eager copies, eager work and a synchronisation
    between replays: every replay equals the eager results bitwise."""
    import torch
    s = setup
    ref = _eager(gq, s)
    d = s["g"].d_model
    x_in = dev(s["x1"]).clone()
    X_in = dev(s["X1"]).clone()
    o_dec = torch.empty(d, dtype=torch.float32, device="cuda")
    o_na = torch.empty(d, dtype=torch.float32, device="cuda")
    o_bat = torch.empty(16 * d, dtype=torch.float32, device="cuda")

    def calls():
        _decode(gq, s, x_in, o_dec)
        gq.smoe_expert_ffn_noalloc(s["de"], 4, 64, x_in, o_na, route_w=s["r"])
        _batch(gq, s, X_in, o_bat)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    busy = torch.randn(1 << 20, device="cuda")
    for k, which in enumerate(("1", "2", "1", "2", "1")):
        x_in.copy_(dev(s["x" + which]))
        X_in.copy_(dev(s["X" + which]))
        o_dec.fill_(float("nan"))
        o_na.fill_(float("nan"))
        o_bat.fill_(float("nan"))
        graph.replay()
        busy.mul_(1.0001).add_(0.5)   # other work on the device between replays
        torch.cuda.synchronize()
        assert np.array_equal(o_dec.cpu().numpy(), ref["x" + which]), f"replay {k}: decode"
        assert np.array_equal(o_na.cpu().numpy(), ref["x" + which]), f"replay {k}: no-allocation decode"
        assert np.array_equal(o_bat.cpu().numpy(), ref["X" + which]), f"replay {k}: batch"


def test_graph_replays_attention_and_bf16(gq):
    """A captured graph of the decode attention block (the small workload,
    appending at a fixed position of device caches) and of the batched bf16
    q/k/v matvecs: four replays, the caches reset and the inputs switched
    between two vectors by eager copies between them, each bitwise equal to
    the eager call (output and appended cache rows)."""
    import torch
    spec = workloads.ATTN_SMALL
    w, x1, K0, V0 = workloads.make_attn_inputs(spec)
    x2 = workloads.activation(79, spec["d_model"])
    pos = spec["pos"]
    wd = [dev(w.wq), dev(w.wk), dev(w.wv), dev(w.wo), dev(w.q_norm), dev(w.k_norm)]
    ws = torch.empty(gq.smoe_attn_decode_workspace(spec["d_model"], spec["n_head"], spec["n_kv"], spec["head_dim"],
                                                   spec["max_ctx"]), dtype=torch.uint8, device="cuda")
    Ws, xb1 = workloads.make_bf16_batch()
    xb2 = workloads.activation(80, xb1.size)
    Wd = [dev(W) for W in Ws]

    def attn_eager(x):
        Kd, Vd = dev(K0), dev(V0)
        out = torch.empty(spec["d_model"], dtype=torch.float32, device="cuda")
        gq.smoe_attn_decode(*wd, dev(x), pos, spec["rope_base"], Kd, Vd, out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), Kd[:, pos].cpu().numpy(), Vd[:, pos].cpu().numpy()

    def bf16_eager(x):
        ys = [torch.empty(W.shape[0], dtype=torch.float32, device="cuda") for W in Wd]
        gq.matvec_bf16_batch([(W, dev(x), y) for W, y in zip(Wd, ys)])
        torch.cuda.synchronize()
        return [y.cpu().numpy() for y in ys]

    ref = {"1": (attn_eager(x1), bf16_eager(xb1)), "2": (attn_eager(x2), bf16_eager(xb2))}
    Kd, Vd = dev(K0), dev(V0)
    K0d, V0d = dev(K0), dev(V0)
    xa, xb = dev(x1).clone(), dev(xb1).clone()
    out = torch.empty(spec["d_model"], dtype=torch.float32, device="cuda")
    ys = [torch.empty(W.shape[0], dtype=torch.float32, device="cuda") for W in Wd]

    def calls():
        gq.smoe_attn_decode(*wd, xa, pos, spec["rope_base"], Kd, Vd, out, ws)
        gq.matvec_bf16_batch([(W, xb, y) for W, y in zip(Wd, ys)])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for k, which in enumerate(("1", "2", "1", "2")):
        Kd.copy_(K0d)
        Vd.copy_(V0d)
        xa.copy_(dev(x1 if which == "1" else x2))
        xb.copy_(dev(xb1 if which == "1" else xb2))
        out.fill_(float("nan"))
        for y in ys:
            y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        (o_ref, k_ref, v_ref), y_ref = ref[which]
        assert np.array_equal(out.cpu().numpy(), o_ref), f"replay {k}: attention output"
        assert np.array_equal(Kd[:, pos].cpu().numpy(), k_ref), f"replay {k}: appended k"
        assert np.array_equal(Vd[:, pos].cpu().numpy(), v_ref), f"replay {k}: appended v"
        for j, (y, yr) in enumerate(zip(ys, y_ref)):
            assert np.array_equal(y.cpu().numpy(), yr), f"replay {k}: bf16 job {j}"


def test_graph_replays_routed(gq, setup):
    """A captured graph of the routed batch (64 tokens x top-2 of the Q4
    group: slot lists, 16-token tiles whose K splits are added across blocks,
    the combine pass), replayed three times with the tokens and their routing
    switched by eager copies: each replay bitwise equal to the eager call."""
    import torch
    s = setup
    d = s["g"].d_model
    inputs = {k: workloads.make_routed_inputs(64, 2, seed) for k, seed in (("1", 4501), ("2", 4502))}
    ws = torch.empty(gq.smoe_routed_ffn_workspace(8, d, s["g"].d_ff, 64, 2), dtype=torch.uint8, device="cuda")

    def eager(X, ids, w):
        out = torch.empty(64 * d, dtype=torch.float32, device="cuda")
        gq.smoe_routed_ffn(s["de"], 4, 64, dev(X), dev(ids), dev(w), out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    ref = {k: eager(*v) for k, v in inputs.items()}
    X_in, ids_in, w_in = (dev(a).clone() for a in inputs["1"])
    out = torch.empty(64 * d, dtype=torch.float32, device="cuda")

    def calls():
        gq.smoe_routed_ffn(s["de"], 4, 64, X_in, ids_in, w_in, out, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for k, which in enumerate(("2", "1", "2")):
        for dst, src in zip((X_in, ids_in, w_in), inputs[which]):
            dst.copy_(dev(src))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref[which]), f"replay {k}: routed batch"
