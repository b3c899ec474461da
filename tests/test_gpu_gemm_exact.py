"""Integer-exact parity of every GEMM layout through the C ABI.

Entries in {-2..2} are exact in bf16; with K <= 4096 every partial sum is an
integer below 2^24, so f32 accumulation is exact in any order. f32 outputs
must therefore equal the fp64 oracle bit for bit, and bf16 outputs must equal
the oracle rounded to nearest even. Shapes span several tiles with ragged
tails in every dimension the kernels allow to be ragged (the token count N,
which is the K dimension of the weight-gradient products). Bytes past each
output must stay untouched (canary)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import bits, f64, rne_bf16_bits, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def _ints(seed, shape):
    b = synth.int_inputs(seed, shape)
    return b, synth.bf16_to_f64(b)


def _canary_f32(shape):
    n = int(np.prod(shape))
    big = torch.full((n + 64,), SENTINEL, dtype=torch.float32, device="cuda:0")
    return big, big[:n].view(*shape)


def _canary_bf16(shape):
    n = int(np.prod(shape))
    big = torch.full((n + 64,), SENTINEL, dtype=torch.bfloat16, device="cuda:0")
    return big, big[:n].view(*shape)


SHAPES_NN = [(300, 256, 320), (16, 512, 128), (1, 64, 64), (257, 128, 512), (64, 64, 64),
             (600, 1024, 768)]


@pytest.mark.parametrize("N,k,n", SHAPES_NN)
def test_row_partial_nn_exact(N, k, n):
    Zb, Z = _ints(1, (N, k))
    Wb, W = _ints(2, (k, n))
    big, P = _canary_f32((N, n))
    T.tp_row_linear_partial(to_dev(Zb), to_dev(Wb), P=P)
    torch.cuda.synchronize()
    assert np.array_equal(f64(P), O.row_linear_partial(Z, W))
    assert torch.all(big[N * n:] == SENTINEL)


@pytest.mark.parametrize("N,k,n", [(300, 256, 320), (16, 128, 64)])
def test_row_partial_accumulate_exact(N, k, n):
    Zb, Z = _ints(3, (N, k))
    Wb, W = _ints(4, (k, n))
    P0b, P0 = _ints(5, (N, n))
    P = torch.from_numpy(P0.astype(np.float32)).to("cuda:0")
    T.tp_row_linear_partial(to_dev(Zb), to_dev(Wb), P=P, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(f64(P), P0 + O.row_linear_partial(Z, W))


@pytest.mark.parametrize("N,k,n", SHAPES_NN)
def test_col_linear_nn_bf16_exact(N, k, n):
    Xb, X = _ints(6, (N, k))
    Wb, W = _ints(7, (k, n))
    big, Y = _canary_bf16((N, n))
    T.tp_col_linear(to_dev(Xb), to_dev(Wb), "none", Y=Y)
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y), rne_bf16_bits(O.col_linear(X, W)))
    assert torch.all(big[N * n:] == SENTINEL)


# Products whose K is split over workgroups: decode sizes (N <= 64; ragged
# last chunk, many chunks, 16 / 32 / 64-row tiles) and large products with
# too few output tiles for the CUs (300 and 520 rows); accumulate into the
# partial.
SHAPES_SPLIT = [(16, 4160, 256), (40, 4160, 128), (64, 8192, 64), (3, 1024, 1280), (24, 2048, 384),
                (16, 8192, 1280), (300, 4096, 320), (520, 6208, 640),
                # token counts that end inside a lane's 4 rows of the fp32 store
                (301, 4096, 320), (777, 2048, 576)]


@pytest.mark.parametrize("N,k,n", SHAPES_SPLIT)
def test_split_k_exact(N, k, n):
    Xb, X = _ints(20, (N, k))
    Wb, W = _ints(21, (k, n))
    P0b, P0 = _ints(22, (N, n))
    big, Y = _canary_bf16((N, n))
    T.tp_col_linear(to_dev(Xb), to_dev(Wb), "none", Y=Y)
    P = torch.from_numpy(P0.astype(np.float32)).to("cuda:0")
    T.tp_row_linear_partial(to_dev(Xb), to_dev(Wb), P=P, accumulate=True)
    torch.cuda.synchronize()
    want = O.col_linear(X, W)
    assert np.array_equal(bits(Y), rne_bf16_bits(want))
    assert torch.all(big[N * n:] == SENTINEL)
    assert np.array_equal(f64(P), P0 + O.row_linear_partial(X, W))


def test_split_k_caller_workspace():
    # one caller workspace for three calls whose split products need small,
    # large and small workspaces (the largest size): results exact; a buffer
    # one byte too small is refused before anything runs
    shapes = [(16, 2048, 128), (64, 8192, 256), (8, 1024, 64)]
    need = [T.workspace_size("tp_row_linear_partial", *s) for s in shapes]
    assert all(x > 0 for x in need) and need[1] > max(need[0], need[2])
    ws = torch.empty(max(need), dtype=torch.uint8, device="cuda:0")
    for i, (N, k, n) in enumerate(shapes):
        Xb, X = _ints(30 + i, (N, k))
        Wb, W = _ints(40 + i, (k, n))
        big, P = _canary_f32((N, n))
        T.tp_row_linear_partial(to_dev(Xb), to_dev(Wb), P=P, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(f64(P), O.row_linear_partial(X, W)), (N, k, n)
        assert torch.all(big[N * n:] == SENTINEL)
    Xb, _ = _ints(33, shapes[1][:2])
    Wb, _ = _ints(43, shapes[1][1:])
    P = torch.full(shapes[1][::2], SENTINEL, dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError, match="bytes of workspace"):
        T.tp_row_linear_partial(to_dev(Xb), to_dev(Wb), P=P, workspace=ws[: need[1] - 1])
    torch.cuda.synchronize()
    assert torch.all(P == SENTINEL)


# (300, 320, 4096): the NT products split K = 4096; (2500, 320, 192): the TN
# products split K = 2500 tokens (ragged last chunk)
SHAPES_BWD = [(300, 320, 256), (16, 128, 192), (1, 64, 64), (513, 256, 128), (1000, 64, 512),
              (300, 320, 4096), (2500, 320, 192)]


@pytest.mark.parametrize("N,k,n", SHAPES_BWD)
def test_col_linear_bwd_nt_tn_exact(N, k, n):
    Xb, X = _ints(8, (N, k))
    Wb, W = _ints(9, (k, n))
    dYb, dY = _ints(10, (N, n))
    bx, dX = _canary_f32((N, k))
    bw, dW = _canary_f32((k, n))
    T.tp_col_linear_bwd(to_dev(Xb), to_dev(Wb), to_dev(dYb), dX_part=dX, dW=dW)
    torch.cuda.synchronize()
    want_dx, want_dw = O.col_linear_bwd(X, W, dY)
    assert np.array_equal(f64(dX), want_dx)
    assert np.array_equal(f64(dW), want_dw)
    assert torch.all(bx[N * k:] == SENTINEL) and torch.all(bw[k * n:] == SENTINEL)


@pytest.mark.parametrize("N,k,n", SHAPES_BWD)
def test_row_linear_bwd_exact(N, k, n):
    Zb, Z = _ints(11, (N, k))
    Wb, W = _ints(12, (k, n))
    dYb, dY = _ints(13, (N, n))
    bz, dZ = _canary_bf16((N, k))
    bw, dW = _canary_f32((k, n))
    T.tp_row_linear_bwd(to_dev(Zb), to_dev(Wb), to_dev(dYb), dZ=dZ, dW=dW)
    torch.cuda.synchronize()
    want_dz, want_dw = O.row_linear_bwd(Z, W, dY)
    assert np.array_equal(bits(dZ), rne_bf16_bits(want_dz))
    assert np.array_equal(f64(dW), want_dw)
    assert torch.all(bz[N * k:] == SENTINEL) and torch.all(bw[k * n:] == SENTINEL)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("N,h", [(1, 256), (300, 256), (16, 2048), (300, 4096)])
def test_pre_activation_save_is_exact(act, N, h):
    # H_save is X W_in rounded once to bf16, including the SwiGLU gate/up
    # interleave (N <= 64 runs the split-K reduction's epilogue)
    f = 192
    n_w = 2 * f if act == "swiglu" else f
    Xb, X = _ints(14, (N, h))
    Wb, W = _ints(15, (h, n_w))
    Y, H = T.tp_col_linear(to_dev(Xb), to_dev(Wb), act, want_h=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(H), rne_bf16_bits(O.col_linear(X, W)))


def test_empty_token_count_is_a_noop():
    W = to_dev(synth.int_inputs(16, (64, 64)))
    Z = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0")
    P = T.tp_row_linear_partial(Z, W)
    torch.cuda.synchronize()
    assert P.shape == (0, 64)


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        N = int(rng.choice([1, 7, 16, 33, 64, 100, 255, 256, 257, 700, 1500]))
        k = 64 * int(rng.integers(1, 40))
        n = 64 * int(rng.integers(1, 40))
        out.append((N, k, n))
    return out


@pytest.mark.parametrize("N,k,n", _random_shapes(2024, 12))
def test_random_shapes_every_layout_exact(N, k, n):
    # seeded random shapes: NN (forward, incl. split-K and decode tiles), NT and TN
    Xb, X = _ints(100, (N, k))
    Wb, W = _ints(101, (k, n))
    dYb, dY = _ints(102, (N, n))
    P = T.tp_row_linear_partial(to_dev(Xb), to_dev(Wb))
    dX, dW = T.tp_col_linear_bwd(to_dev(Xb), to_dev(Wb), to_dev(dYb))
    torch.cuda.synchronize()
    assert np.array_equal(f64(P), O.row_linear_partial(X, W))
    want_dx, want_dw = O.col_linear_bwd(X, W, dY)
    assert np.array_equal(f64(dX), want_dx)
    assert np.array_equal(f64(dW), want_dw)
