"""Operands and outputs larger than 2 and 4 GiB: a token matrix X[N, 8192] of
4.4 GB (rows past byte offsets 2^31 and 2^32, and a ragged last tile) through
the column-parallel forward, the row-parallel partial and the column-parallel
backward (dX_part of 8.9 GB; dW contracting 270k tokens with split-K).
Integer inputs keep every f32 sum exact, so sampled rows and columns must
equal the fp64 oracle exactly (bf16 outputs: its round-to-nearest-even)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import bits, f64

pytestmark = pytest.mark.gpu

N, K, NOUT = 270373, 8192, 128          # X is N * K * 2 B = 4.43 GB
ROW_BYTES = K * 2


def _sample_rows():
    edges = [0, 1, 255, 256]
    for b in (1 << 31, 1 << 32):         # rows around the byte offsets 2^31, 2^32 of X
        r = b // ROW_BYTES
        edges += [r - 1, r, r + 1]
    edges += [N - 38, N - 2, N - 1]
    rng = np.random.default_rng(11)
    return np.unique(np.concatenate([edges, rng.choice(N, 16, replace=False)]))


@pytest.fixture(scope="module")
def big():
    X = synth.int_inputs_device(90, (N, K), "cuda:0")
    W = synth.int_inputs_device(91, (K, NOUT), "cuda:0")
    dY = synth.int_inputs_device(92, (N, NOUT), "cuda:0")
    torch.cuda.synchronize()
    yield X, W, dY
    del X, W, dY
    torch.cuda.empty_cache()


def test_forward_products_past_4gib(big):
    X, W, _ = big
    rows = _sample_rows()
    ridx = torch.from_numpy(rows).cuda()
    X_rows, W64 = f64(X[ridx]), f64(W)
    want = O.col_linear(X_rows, W64)                   # exact integers (|sum| <= 73728)

    Y, _ = T.tp_col_linear(X, W, "none")
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y[ridx]), synth.bf16_round(want.astype(np.float32)))

    P = torch.full((N, NOUT), 0.5, dtype=torch.float32, device="cuda:0")
    T.tp_row_linear_partial(X, W, P=P, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(f64(P[ridx]), want + 0.5)
    del Y, P


def test_backward_past_4gib(big):
    X, W, dY = big
    rows = _sample_rows()
    rng = np.random.default_rng(12)
    cols = np.unique(np.concatenate([[0, 1, 4095, K - 1], rng.choice(K, 12, replace=False)]))
    cidx = torch.from_numpy(cols).cuda()
    X_cols = f64(X[:, cidx])                           # [N, 16]
    want_dx_cols, want_dw_rows = O.col_linear_bwd(X_cols, f64(W[cidx]), f64(dY))

    dX, dW = T.tp_col_linear_bwd(X, W, dY)             # dX_part: 8.9 GB; dW: K = 270373 tokens
    torch.cuda.synchronize()
    assert np.array_equal(f64(dW[cidx]), want_dw_rows)   # |sum| <= 2.4e6: exact in f32
    assert np.array_equal(f64(dX[:, cidx]), want_dx_cols)
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(f64(dX[ridx]), O.col_linear_bwd(f64(X[ridx]), f64(W), f64(dY[ridx]))[0])
    del dX, dW


def test_weight_window_past_2gib():
    # W[16384, 65600] bf16 = 2.15 GB: its K rows times its pitch reach 2^31
    # bytes, so the kernel moves its descriptor along K stage by stage;
    # ragged last column tile (65600 = 256 * 256 + 64)
    k, n = 16384, 65600
    X = synth.int_inputs_device(93, (64, k), "cuda:0")
    W = synth.int_inputs_device(94, (k, n), "cuda:0")
    rng = np.random.default_rng(13)
    cols = np.unique(np.concatenate([[0, 1, 255, 256, n - 65, n - 64, n - 1], rng.choice(n, 16, replace=False)]))
    cidx = torch.from_numpy(cols).cuda()
    want = O.col_linear(f64(X), f64(W[:, cidx]))      # exact integers (|sum| <= 147456)
    Y, _ = T.tp_col_linear(X, W, "none")
    P = T.tp_row_linear_partial(X, W)
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y[:, cidx]), synth.bf16_round(want.astype(np.float32)))
    assert np.array_equal(f64(P[:, cidx]), want)
    del X, W, Y, P
    torch.cuda.empty_cache()
