"""Whole-output parity, element by element, for every (layout, epilogue, tile)
the Llama-3-70B MLP step and the attention projections launch, at shapes
whose tile counts select exactly those kernels.

The tile of a product is chosen from its output shape (the fewest waves of
workgroups over the 256 CUs times the tile area, 256 x 256 against 256 x 224
and 224 x 256; always 256 x 256 for the SwiGLU forward); the contraction
length enters only for products with few output tiles (a K split, or the
mid tiles below, from K = 2048 on). So each case of the MLP step keeps the
step's output shape (or one with the same choice) and shortens K where that
keeps the oracle fast:

  kernel launched by the step          case here (M x N output, K)      tiles
  NN 256x256, SwiGLU (+H)              X W_gu   4096 x 3584 (2f=7168), 256   448 (2 waves)
  NN 256x256, fp32 store (GEMM2)       Z W_d    4096 x 8192, 256             512
  NN 256x256, GeLU (+H)                X A      4096 x 8192, 256             512
  NT 256x224, SwiGLU' from H (dZ)      dY W_d^T 4096 x 3584, 256             256 (1 wave)
  NT 256x256, fp32 store (dX)          dH W^T   4096 x 8192, 256             512
  TN 256x224, fp32 store (dW_gate|up)  X^T dH   8192 x 7168, 500 tokens      1024 (4 waves)
  TN 224x256, fp32 store (dW_down)     Z^T dY   3584 x 8192, 300 tokens      512

and the attention projections run at their own sizes (below), which also
select the TN 128 x 256 mid tile (dW_O); a ragged case covers that tile on
every edge.

Integer-valued inputs (small integers, times a power of two where an
activation should see values of order one) make every product exact in f32
in any summation order, so fp32 outputs and the saved pre-activation H must
equal the fp64 oracle bit for bit; activation outputs (rounded once to bf16
after an f32 evaluation of SiLU / GeLU) must be within one bf16 rounding of
the oracle, element by element. Bytes past each output stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import assert_elementwise, bits, f64, rne_bf16_bits, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def _ints(seed, shape, scale=1.0):
    b = synth.int_inputs(seed, shape, scale=scale)
    return b, synth.bf16_to_f64(b)


def _canary(shape, dtype):
    n = int(np.prod(shape))
    big = torch.full((n + 256,), SENTINEL, dtype=dtype, device="cuda:0")
    return big, big[:n].view(*shape)


def _untouched(big, n):
    return bool(torch.all(big[n:] == SENTINEL))


def test_gemm1_swiglu_nn_256x256():
    N, h, f = 4096, 256, 3584
    Xb, X = _ints(201, (N, h), scale=1 / 16)      # G, U = integers / 16: SiLU sees O(1)
    Wb, W = _ints(202, (h, 2 * f))
    bz, Z = _canary((N, f), torch.bfloat16)
    bh, H = _canary((N, 2 * f), torch.bfloat16)
    T.tp_col_linear(to_dev(Xb), to_dev(Wb), "swiglu", Y=Z, H_save=H)
    torch.cuda.synchronize()
    oZ, oH = O.col_linear_act(X, W, "swiglu")
    assert np.array_equal(bits(H), rne_bf16_bits(oH))
    assert_elementwise(f64(Z), oZ, "Z")
    assert _untouched(bz, N * f) and _untouched(bh, N * 2 * f)


def test_gemm2_nn_256x256_fp32_partial():
    N, f, h = 4096, 256, 8192
    Zb, Z = _ints(203, (N, f))
    Wb, W = _ints(204, (f, h))
    P0b, P0 = _ints(205, (N, h))
    big, P = _canary((N, h), torch.float32)
    P.copy_(torch.from_numpy(P0.astype(np.float32)))
    T.tp_row_linear_partial(to_dev(Zb), to_dev(Wb), P=P, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(f64(P), P0 + O.row_linear_partial(Z, W))
    assert _untouched(big, N * h)
    T.tp_row_linear_partial(to_dev(Zb), to_dev(Wb), P=P)
    torch.cuda.synchronize()
    assert np.array_equal(f64(P), O.row_linear_partial(Z, W))


def test_gelu_nn_256x256_with_saved_pre_activation():
    N, h, n = 4096, 256, 8192
    Xb, X = _ints(206, (N, h), scale=1 / 16)
    Wb, W = _ints(207, (h, n))
    bz, Z = _canary((N, n), torch.bfloat16)
    bh, H = _canary((N, n), torch.bfloat16)
    T.tp_col_linear(to_dev(Xb), to_dev(Wb), "gelu", Y=Z, H_save=H)
    torch.cuda.synchronize()
    oZ, oH = O.col_linear_act(X, W, "gelu")
    assert np.array_equal(bits(H), rne_bf16_bits(oH))
    assert_elementwise(f64(Z), oZ, "GeLU")
    assert _untouched(bz, N * n) and _untouched(bh, N * n)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_dz_activation_backward_nt_256x224(act):
    # tp_mlp_shard_bwd with no gradient requested runs the dZ product with
    # the activation backward in its epilogue alone (dH written)
    N, h, f = 4096, 256, 3584
    n_w = 2 * f if act == "swiglu" else f
    dYb, dY = _ints(208, (N, h), scale=1 / 16)
    Woutb, W_out = _ints(209, (f, h))
    Hb, H = _ints(210, (N, n_w), scale=1 / 2)         # saved pre-activation in {-1 .. 1}
    X = torch.empty((N, h), dtype=torch.bfloat16, device="cuda:0")
    W_in = torch.empty((h, n_w), dtype=torch.bfloat16, device="cuda:0")
    Z = torch.empty((N, f), dtype=torch.bfloat16, device="cuda:0")
    bd, dH = _canary((N, n_w), torch.bfloat16)
    out = T.tp_mlp_shard_bwd(X, W_in, to_dev(Woutb), to_dev(Hb), Z, to_dev(dYb), act, dH=dH, want=())
    torch.cuda.synchronize()
    assert out[1] is None and out[2] is None and out[3] is None
    # dH depends on dY, W_out and H only (X, W_in and Z enter other outputs)
    want = O.mlp_shard_bwd_saved(np.zeros((N, h)), np.zeros((h, n_w)), W_out, H, np.zeros((N, f)), dY, act)["dH"]
    assert_elementwise(f64(dH), want, f"dH ({act})")
    assert _untouched(bd, N * n_w)


def test_dx_nt_256x256_fp32_partial():
    N, k, n = 4096, 8192, 256
    Xd = torch.empty((N, k), dtype=torch.bfloat16, device="cuda:0")
    Wb, W = _ints(211, (k, n))
    dYb, dY = _ints(212, (N, n))
    big, dX = _canary((N, k), torch.float32)
    T.tp_col_linear_bwd(Xd, to_dev(Wb), to_dev(dYb), dX_part=dX, want_dw=False)
    torch.cuda.synchronize()
    assert np.array_equal(f64(dX), dY @ W.T)
    assert _untouched(big, N * k)


def test_dw_gate_up_tn_256x224_fp32():
    N, k, n = 500, 8192, 7168                         # ragged token count (the contraction)
    Xb, X = _ints(213, (N, k))
    W = torch.empty((k, n), dtype=torch.bfloat16, device="cuda:0")
    dYb, dY = _ints(214, (N, n))
    big, dW = _canary((k, n), torch.float32)
    T.tp_col_linear_bwd(to_dev(Xb), W, to_dev(dYb), dW=dW, want_dx=False)
    torch.cuda.synchronize()
    assert np.array_equal(f64(dW), X.T @ dY)
    assert _untouched(big, k * n)


def test_dw_down_tn_224x256_fp32():
    N, k_loc, n = 300, 3584, 8192
    Zb, Z = _ints(215, (N, k_loc))
    W = torch.empty((k_loc, n), dtype=torch.bfloat16, device="cuda:0")
    dYb, dY = _ints(216, (N, n))
    big, dW = _canary((k_loc, n), torch.float32)
    T.tp_row_linear_bwd(to_dev(Zb), W, to_dev(dYb), dW=dW, want_dz=False)
    torch.cuda.synchronize()
    assert np.array_equal(f64(dW), Z.T @ dY)
    assert _untouched(big, k_loc * n)


# The attention projections of one Llama-3-70B rank at t = 8 (h = 8192,
# W_r 1280 wide, W_O 1024 rows), prefill N = 4096 and decode N = 16, every
# product of the forward and backward: split-K (the QKV forward and dO at
# 4096 tokens, dO and dW_O at 16), the decode kernel (both forward products
# at 16), the TN mid tile (dW_O at 4096) and the large tiles.
@pytest.mark.parametrize("N", [4096, 16])
def test_attention_projection_products_exact(N):
    h, wq, wo = 8192, 1280, 1024
    Xb, X = _ints(230, (N, h))
    Wrb, Wr = _ints(231, (h, wq))
    Ob, Oa = _ints(232, (N, wo))
    WOb, WO = _ints(233, (wo, h))
    dQb, dQ = _ints(234, (N, wq))
    dYb, dY = _ints(235, (N, h))
    Xd, Wrd, Od, WOd = to_dev(Xb), to_dev(Wrb), to_dev(Ob), to_dev(WOb)
    Y, _ = T.tp_col_linear(Xd, Wrd, "none")
    P = T.tp_row_linear_partial(Od, WOd)
    dX, dW = T.tp_col_linear_bwd(Xd, Wrd, to_dev(dQb))
    dO, dWO = T.tp_row_linear_bwd(Od, WOd, to_dev(dYb))
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y), rne_bf16_bits(X @ Wr))
    assert np.array_equal(f64(P), Oa @ WO)
    assert np.array_equal(f64(dX), dQ @ Wr.T)
    assert np.array_equal(f64(dW), X.T @ dQ)
    assert np.array_equal(bits(dO), rne_bf16_bits(dY @ WO.T))
    assert np.array_equal(f64(dWO), Oa.T @ dY)


# The TN mid tile (128 x 256): a weight gradient whose 256 x 256 tiles would
# fill at most half of the 256 CUs but whose mid tiles fill more than half,
# with K >= 2048 tokens, runs one wave of mid tiles over the whole K (no
# split, no workspace). Ragged on every edge: 2112 weight rows (16.5 tiles
# of 128), 1984 columns (7.75 tiles of 256), 3000 tokens (not a multiple of
# 32). dZ of the same call (K = 1984) takes the large tiles without a split.
def test_mid_tile_tn_ragged_exact():
    N, k_loc, n = 3000, 2112, 1984
    assert T.workspace_size("tp_row_linear_bwd", N, k_loc, n) == 0
    Zb, Z = _ints(240, (N, k_loc))
    Wb, W = _ints(241, (k_loc, n))
    dYb, dY = _ints(242, (N, n))
    bz, dZ = _canary((N, k_loc), torch.bfloat16)
    bw, dW = _canary((k_loc, n), torch.float32)
    T.tp_row_linear_bwd(to_dev(Zb), to_dev(Wb), to_dev(dYb), dZ=dZ, dW=dW)
    torch.cuda.synchronize()
    assert np.array_equal(f64(dW), Z.T @ dY)
    assert np.array_equal(bits(dZ), rne_bf16_bits(dY @ W.T))
    assert _untouched(bz, N * k_loc) and _untouched(bw, k_loc * n)
