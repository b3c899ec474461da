"""The row-parallel partial in row chunks (tp_row_linear_partial_chunked):
exact against the oracle on integer inputs for several chunk counts (chunks
that need split-K included), with and without accumulate, every chunk's event
recorded in chunk order; chunk-sized products on the NN mid tiles exact; at
the Llama-3-70B GEMM2 shape, every element of every chunk count against the
fp64 oracle within the tolerance. The column-parallel backward with dX_part
in row chunks (tp_col_linear_bwd_chunked) the same way: exact dX_part and dW
on integer inputs (chunks that split K, empty chunks, accumulate), events in
order and before dW's completion, and the Llama-3-70B MLP shard's dX at every
element for 2, 4 and 8 chunks. For both calls, a second stream that waits for
each chunk's event and copies that chunk out (what an exchange would do)
sees every chunk finished."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import check_errs, err, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,k,n,nchunks", [(1000, 512, 640, 1), (1000, 512, 640, 3), (1000, 2048, 640, 8),
                                           (37, 256, 128, 4), (300, 4096, 320, 2), (1000, 512, 640, 64)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_chunked_partial_exact(N, k, n, nchunks, accumulate):
    Zb, Wb = synth.int_inputs(80, (N, k)), synth.int_inputs(81, (k, n))
    P0 = synth.bf16_to_f64(synth.int_inputs(82, (N, n)))
    P = torch.from_numpy(P0.astype(np.float32)).to("cuda:0")
    events = [torch.cuda.Event(enable_timing=True) for _ in range(nchunks)]
    T.tp_row_linear_partial_chunked(to_dev(Zb), to_dev(Wb), nchunks, P=P, accumulate=accumulate, events=events)
    torch.cuda.synchronize()
    want = O.row_linear_partial(synth.bf16_to_f64(Zb), synth.bf16_to_f64(Wb)) + (P0 if accumulate else 0)
    assert np.array_equal(f64(P), want)
    assert all(e.query() for e in events)
    for a, b in zip(events, events[1:]):
        assert a.elapsed_time(b) >= 0.0


# Chunk-sized fp32 row partials take NN mid tiles (128 x 256 when they fill
# a wave of the 256 CUs, else 128 x 128) over their whole K: the GEMM2 shard
# in 4 chunks (1024 tokens) and 8 chunks (512), here ragged on every edge
# (the last row tile partly filled, widths ending inside a tile) and exact.
@pytest.mark.parametrize("N,k,n", [(1000, 2112, 7936), (500, 2048, 7680), (1024, 2048, 8192), (512, 2048, 8192)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_chunk_sized_partial_mid_tiles_exact(N, k, n, accumulate):
    assert T.workspace_size("tp_row_linear_partial", N, k, n) == 0   # no K split
    Zb, Wb = synth.int_inputs(90, (N, k)), synth.int_inputs(91, (k, n))
    P0 = synth.bf16_to_f64(synth.int_inputs(92, (N, n)))
    big = torch.full((N * n + 256,), 12345.0, dtype=torch.float32, device="cuda:0")
    P = big[:N * n].view(N, n)
    P.copy_(torch.from_numpy(P0.astype(np.float32)))
    T.tp_row_linear_partial(to_dev(Zb), to_dev(Wb), P=P, accumulate=accumulate)
    torch.cuda.synchronize()
    want = O.row_linear_partial(synth.bf16_to_f64(Zb), synth.bf16_to_f64(Wb)) + (P0 if accumulate else 0)
    assert np.array_equal(f64(P), want)
    assert bool(torch.all(big[N * n:] == 12345.0))


def test_chunked_llama_gemm2_against_oracle():
    w = synth.WORKLOADS["llama70b_swiglu_t8"]
    rng = np.random.default_rng(9)
    Zb, Wb = synth.draw(rng, (w.N, w.f)), synth.draw(rng, (w.f, w.h), fan_in=w.F)
    Z, W = to_dev(Zb), to_dev(Wb)
    want = O.row_linear_partial(synth.bf16_to_f64(Zb), synth.bf16_to_f64(Wb))
    errs = {}
    for nchunks in (1, 2, 4, 8):
        got = T.tp_row_linear_partial_chunked(Z, W, nchunks)
        torch.cuda.synchronize()
        errs[f"P, {nchunks} chunks"] = err(f64(got), want)
    check_errs(errs, "llama70b GEMM2 chunked (every element)")



# Chunk-sized dX_part products whose 128 x 256 tiles fill a wave of the 256
# CUs take those NT mid tiles over their whole K: the MLP shard's dX in 4
# chunks (1024 tokens), here also ragged on every edge, exact, with nothing
# written past the output.
@pytest.mark.parametrize("N,k,n", [(1000, 7936, 2112), (900, 8000, 2048), (1024, 8192, 2048)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_chunk_sized_dx_mid_tiles_exact(N, k, n, accumulate):
    assert T.workspace_size("tp_col_linear_bwd", N, k, n) == 0   # no K split
    Wb, dYb = synth.int_inputs(93, (k, n)), synth.int_inputs(94, (N, n))
    D0 = synth.bf16_to_f64(synth.int_inputs(95, (N, k)))
    big = torch.full((N * k + 256,), 12345.0, dtype=torch.float32, device="cuda:0")
    dX = big[:N * k].view(N, k)
    dX.copy_(torch.from_numpy(D0.astype(np.float32)))
    X = torch.empty((N, k), dtype=torch.bfloat16, device="cuda:0")   # not read for dX_part
    T.tp_col_linear_bwd(X, to_dev(Wb), to_dev(dYb), dX_part=dX, want_dw=False, accumulate=accumulate)
    torch.cuda.synchronize()
    want, _ = O.col_linear_bwd(np.zeros((N, k)), synth.bf16_to_f64(Wb), synth.bf16_to_f64(dYb))
    assert np.array_equal(f64(dX), want + (D0 if accumulate else 0))
    assert bool(torch.all(big[N * k:] == 12345.0))

@pytest.mark.parametrize("N,k,n,nchunks", [(1000, 512, 640, 3), (1000, 2048, 640, 8), (37, 256, 128, 4),
                                           (300, 4096, 320, 2), (1024, 2048, 4096, 4), (1000, 640, 2048, 1),
                                           (1000, 512, 640, 64)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_chunked_col_bwd_exact(N, k, n, nchunks, accumulate):
    Xb, Wb, dYb = synth.int_inputs(83, (N, k)), synth.int_inputs(84, (k, n)), synth.int_inputs(85, (N, n))
    D0 = synth.bf16_to_f64(synth.int_inputs(86, (N, k)))
    dX = torch.from_numpy(D0.astype(np.float32)).to("cuda:0")
    events = [torch.cuda.Event(enable_timing=True) for _ in range(nchunks)]
    done = torch.cuda.Event(enable_timing=True)
    _, dW = T.tp_col_linear_bwd_chunked(to_dev(Xb), to_dev(Wb), to_dev(dYb), nchunks, dX_part=dX,
                                        accumulate=accumulate, events=events)
    done.record()
    torch.cuda.synchronize()
    want_dx, want_dw = O.col_linear_bwd(synth.bf16_to_f64(Xb), synth.bf16_to_f64(Wb), synth.bf16_to_f64(dYb))
    assert np.array_equal(f64(dX), want_dx + (D0 if accumulate else 0))
    assert np.array_equal(f64(dW), want_dw)
    assert all(e.query() for e in events)
    for a, b in zip(events + [done], events[1:] + [done]):
        assert a.elapsed_time(b) >= 0.0


def test_chunked_col_bwd_split_chunks_and_no_dw():
    # 256-row chunks of a 2048-column output over K = 4096: 8 tiles each,
    # split along K; dW not requested
    N, k, n, nchunks = 1024, 2048, 4096, 4
    assert T.workspace_size("tp_col_linear_bwd_chunked", N, k, n, nchunks) > 0
    Xb, Wb, dYb = synth.int_inputs(87, (N, k)), synth.int_inputs(88, (k, n)), synth.int_inputs(89, (N, n))
    dX, dW = T.tp_col_linear_bwd_chunked(to_dev(Xb), to_dev(Wb), to_dev(dYb), nchunks, want_dw=False)
    torch.cuda.synchronize()
    assert dW is None
    want_dx, _ = O.col_linear_bwd(synth.bf16_to_f64(Xb), synth.bf16_to_f64(Wb), synth.bf16_to_f64(dYb))
    assert np.array_equal(f64(dX), want_dx)


def test_chunked_llama_mlp_dx_against_oracle():
    w = synth.WORKLOADS["llama70b_swiglu_t8"]
    rng = np.random.default_rng(10)
    n_w = 2 * w.f
    Xb = synth.draw(rng, (w.N, w.h))
    Wb = synth.draw(rng, (w.h, n_w), fan_in=w.h)
    dHb = synth.draw(rng, (w.N, n_w))
    X, W, dH = to_dev(Xb), to_dev(Wb), to_dev(dHb)
    want, _ = O.col_linear_bwd(synth.bf16_to_f64(Xb), synth.bf16_to_f64(Wb), synth.bf16_to_f64(dHb))
    errs = {}
    for nchunks in (2, 4, 8):
        dX, _ = T.tp_col_linear_bwd_chunked(X, W, dH, nchunks, want_dw=False)
        torch.cuda.synchronize()
        errs[f"dX_part, {nchunks} chunks"] = err(f64(dX), want)
        del dX
    check_errs(errs, "llama70b MLP dX chunked (every element)")


@pytest.mark.parametrize("which", ["row_partial", "col_bwd"])
def test_chunk_events_gate_a_consumer_stream(which):
    # The use the events are for: a second stream (the exchange) waits for
    # chunk c's event, then reads chunk c's rows while later chunks are
    # still computed. Here the reading is a copy; every copied chunk must be
    # the finished one.
    N, k, n, nchunks = 2048, 1024, 2048, 4
    A, Bm = synth.int_inputs(96, (N, k)), synth.int_inputs(97, (k, n))
    events = [torch.cuda.Event() for _ in range(nchunks)]
    # (filled before the call, so every event follows the fill)
    copy = torch.full((N, n), float("nan"), dtype=torch.float32, device="cuda:0")
    if which == "row_partial":
        out = T.tp_row_linear_partial_chunked(to_dev(A), to_dev(Bm), nchunks, events=events)
        want = O.row_linear_partial(synth.bf16_to_f64(A), synth.bf16_to_f64(Bm))
    else:
        X = torch.empty((N, n), dtype=torch.bfloat16, device="cuda:0")   # dX only: X not read
        out, _ = T.tp_col_linear_bwd_chunked(X, to_dev(Bm.T.copy()), to_dev(A), nchunks, want_dw=False,
                                             events=events)
        want, _ = O.col_linear_bwd(np.zeros((N, n)), synth.bf16_to_f64(Bm.T.copy()), synth.bf16_to_f64(A))
    rows = ((N + nchunks - 1) // nchunks + 15) // 16 * 16   # the calls' chunk height
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for c in range(nchunks):
            side.wait_event(events[c])
            copy[c * rows:(c + 1) * rows].copy_(out[c * rows:(c + 1) * rows])
    torch.cuda.synchronize()
    assert np.array_equal(f64(copy), want)


def test_chunked_col_bwd_no_tokens():
    # N = 0: every chunk is empty; dW contracts over no tokens and is zero
    k, n = 512, 640
    X = torch.empty((0, k), dtype=torch.bfloat16, device="cuda:0")
    dY = torch.empty((0, n), dtype=torch.bfloat16, device="cuda:0")
    dW = torch.full((k, n), 7.0, dtype=torch.float32, device="cuda:0")
    events = [torch.cuda.Event() for _ in range(3)]
    dX, dW = T.tp_col_linear_bwd_chunked(X, to_dev(synth.int_inputs(98, (k, n))), dY, 3, dW=dW, events=events)
    torch.cuda.synchronize()
    assert dX.shape == (0, k)
    assert bool(torch.all(dW == 0.0))
    assert all(e.query() for e in events)
