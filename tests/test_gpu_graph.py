"""Calls captured into a HIP graph and replayed give the same bits as the same
calls run eagerly: the split-K decode products (library workspace per stream),
the MLP forward at decode size and the fused-QKV regroup. Each replay follows
eager work that rewrites the inputs in place, and every replay is checked."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import TOL, err, f64, to_dev

pytestmark = pytest.mark.gpu


def _normal(seed, shape, fan_in=None):
    return synth.draw(np.random.default_rng(seed), shape, fan_in)


def test_graph_replays_match_eager():
    dev = "cuda:0"
    N, h, n, k_o, f = 16, 2048, 384, 1024, 512
    X = to_dev(_normal(50, (N, h)))
    W = to_dev(_normal(51, (h, n), h))
    O_r = to_dev(_normal(52, (N, k_o)))
    W_O = to_dev(_normal(53, (k_o, h), k_o))
    W_in = to_dev(_normal(54, (h, 2 * f), h))
    W_out = to_dev(_normal(55, (f, h), f))
    W_qkv = to_dev(_normal(56, (256, (8 + 2 * 2) * 64)))
    Y = torch.empty((N, n), dtype=torch.bfloat16, device=dev)
    P = torch.empty((N, h), dtype=torch.float32, device=dev)
    Z = torch.empty((N, f), dtype=torch.bfloat16, device=dev)
    Hs = torch.empty((N, 2 * f), dtype=torch.bfloat16, device=dev)
    P2 = torch.empty((N, h), dtype=torch.float32, device=dev)
    W_r = torch.empty((256, (8 + 2 * 2) * 64 // 2), dtype=torch.bfloat16, device=dev)

    def calls():
        T.tp_col_linear(X, W, "none", Y=Y)
        T.tp_row_linear_partial(O_r, W_O, P=P)
        T.tp_mlp_shard_fwd(X, W_in, W_out, "swiglu", Z=Z, H_save=Hs, P=P2)
        T.tp_qkv_regroup(W_qkv, 8, 2, 64, 2, 1, W_r=W_r)

    outs = (Y, P, Z, Hs, P2, W_r)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # creates this stream's split-K workspace before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        calls()
    torch.cuda.synchronize()

    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    for r in range(3):
        # new inputs, written in place by eager work, then the graph, then eager
        for t in (X, O_r, W_qkv):
            t.copy_(torch.randn(t.shape, device=dev, generator=gen).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        for o in outs:
            o.fill_(0)
        calls()
        torch.cuda.synchronize()
        for g, e in zip(got, outs):
            assert torch.equal(g.view(torch.int16) if g.dtype == torch.bfloat16 else g.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32)), r
        # and the eager results are right (the decode product against the oracle)
        want = O.col_linear(f64(X), f64(W))
        assert err(f64(Y), want) <= TOL
    del graph


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")  # nothing was enqueued, as intended
def test_capture_before_the_workspace_exists_is_refused():
    # a stream whose split-K workspace does not exist yet cannot create it
    # while it is captured: the call reports it and enqueues nothing
    N, h, n = 16, 2048, 384
    X = to_dev(_normal(60, (N, h)))
    W = to_dev(_normal(61, (h, n), h))
    Y = torch.empty((N, n), dtype=torch.bfloat16, device="cuda:0")
    fresh = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(ValueError, match="captured"):
        with torch.cuda.graph(graph, stream=fresh):
            T.tp_col_linear(X, W, "none", Y=Y)
    torch.cuda.synchronize()
    # the same call outside capture works, after which capture does too
    with torch.cuda.stream(fresh):
        T.tp_col_linear(X, W, "none", Y=Y)
    torch.cuda.synchronize()
    want = O.col_linear(f64(X), f64(W))
    assert err(f64(Y), want) <= TOL
