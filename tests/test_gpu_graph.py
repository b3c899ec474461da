"""Calls captured into a HIP graph and replayed give the same bits as the same
calls run eagerly: the split-K decode products (their workspace allocated by
the binding inside the capture), the MLP forward at decode size, the
fused-QKV regroup, and both chunked calls with their per-chunk events.
Capture works on a fresh stream, with no call before it.
Each replay follows eager work that rewrites the inputs in place, and every
replay is checked."""
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
    assert T.workspace_size("tp_col_linear", N, h, n, 0) > 0        # the decode products are split
    assert T.workspace_size("tp_row_linear_partial", N, k_o, h) > 0
    side = torch.cuda.Stream()        # fresh: nothing has run on it
    side.wait_stream(torch.cuda.current_stream())
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


def test_replay_after_larger_eager_calls_on_the_capture_stream():
    # A captured split product keeps its own workspace: eager calls with
    # larger split workspaces on the same stream afterwards (which a
    # per-stream library buffer would have replaced) leave the replays right.
    dev = "cuda:0"
    N, h, n = 16, 2048, 384
    X = to_dev(_normal(60, (N, h)))
    W = to_dev(_normal(61, (h, n), h))
    Y = torch.empty((N, n), dtype=torch.bfloat16, device=dev)
    fresh = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=fresh):
        T.tp_col_linear(X, W, "none", Y=Y)
    torch.cuda.synchronize()
    Xb = to_dev(_normal(62, (64, 8192)))
    Wb = to_dev(_normal(63, (8192, 1280), 8192))
    small = T.workspace_size("tp_col_linear", N, h, n, 0)
    assert T.workspace_size("tp_col_linear", 64, 8192, 1280, 0) > small
    want = O.col_linear(f64(X), f64(W))
    for r in range(3):
        with torch.cuda.stream(fresh):
            Yb, _ = T.tp_col_linear(Xb, Wb, "none")     # larger split workspace, eager
            Y.fill_(0)
            graph.replay()
        torch.cuda.synchronize()
        assert err(f64(Y), want) <= TOL, r
        assert err(f64(Yb), O.col_linear(f64(Xb), f64(Wb))) <= TOL, r
    del graph


@pytest.mark.parametrize("nchunks", [2, 8])
def test_chunked_calls_with_events_captured(nchunks):
    # Both chunked calls, their events recorded on the capturing stream (and
    # the split products' workspace allocated inside the capture), replayed
    # after eager work that rewrites an input in place: every replay equals
    # the eager calls, which equal the oracle (integer inputs: exact).
    dev = "cuda:0"
    N, k, n = 2048, 1024, 2048
    A = to_dev(synth.int_inputs(70, (N, k)))
    B = to_dev(synth.int_inputs(71, (k, n)))
    Xc = to_dev(synth.int_inputs(72, (N, n)))
    Wc = to_dev(synth.int_inputs(73, (n, k)))
    P = torch.empty((N, n), device=dev, dtype=torch.float32)
    dX = torch.empty((N, n), device=dev, dtype=torch.float32)
    dW = torch.empty((n, k), device=dev, dtype=torch.float32)
    evs = [torch.cuda.Event() for _ in range(2 * nchunks)]
    for e in evs:            # created before the capture
        e.record()
    torch.cuda.synchronize()

    def calls():
        T.tp_row_linear_partial_chunked(A, B, nchunks, P=P, events=evs[:nchunks])
        T.tp_col_linear_bwd_chunked(Xc, Wc, A, nchunks, dX_part=dX, dW=dW, events=evs[nchunks:])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        calls()
    torch.cuda.synchronize()
    outs = (P, dX, dW)
    for r in range(3):
        a_host = synth.int_inputs(74 + r, (N, k))
        A.copy_(to_dev(a_host))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        for o in outs:
            o.fill_(0)
        calls()
        torch.cuda.synchronize()
        for g, e in zip(got, outs):
            assert torch.equal(g.view(torch.int32), e.view(torch.int32)), r
        a64 = synth.bf16_to_f64(a_host)
        assert np.array_equal(f64(P), O.row_linear_partial(a64, synth.bf16_to_f64(synth.int_inputs(71, (k, n)))))
        want_dx, want_dw = O.col_linear_bwd(synth.bf16_to_f64(synth.int_inputs(72, (N, n))),
                                            synth.bf16_to_f64(synth.int_inputs(73, (n, k))), a64)
        assert np.array_equal(f64(dX), want_dx) and np.array_equal(f64(dW), want_dw), r
    del graph
