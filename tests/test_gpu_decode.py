"""Decode-sized forward products (at most 32 token rows): the weight is
streamed in slabs of 32 product columns, with K split over workgroups when the
slabs alone do not fill the CUs. Every element of every output is compared
with the fp64 oracle on integer-valued inputs (exact in f32 in any summation
order), for each epilogue, both token tiles (16 and 32 rows), split and
unsplit plans, and K shorter than one block per wave. Bytes past each output
stay untouched.

  case (M, K, n)       plan
  16, 8192, 1280       QKV at t = 8: 20 slabs of 64 columns x 12 K splits,
                       and the split reduction
  16, 1024, 8192       W_O at t = 8: 256 slabs of 32 columns (XCD pairs), no split
  1 / 5, 64, 512       2 k-blocks, 16 slabs of 32, no split: six of the eight
                       waves have no block
  17 / 32, 1024, 8192  32-row token tile, 256 slabs of 32, no split
  32, 2048, 1280       32-row token tile, 20 slabs of 64 x 8 K splits
  16, 256, 1408        44 slabs of 32, no split: two groups of 16 paired
                       slabs and a tail of 12 in plain order
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
CASES = [(16, 8192, 1280), (16, 1024, 8192), (1, 64, 512), (5, 64, 512), (17, 1024, 8192), (32, 1024, 8192),
         (32, 2048, 1280), (16, 256, 1408)]


def _ints(seed, shape, scale=1.0):
    b = synth.int_inputs(seed, shape, scale=scale)
    return b, synth.bf16_to_f64(b)


def _canary(shape, dtype):
    n = int(np.prod(shape))
    big = torch.full((n + 256,), SENTINEL, dtype=dtype, device="cuda:0")
    return big, big[:n].view(*shape)


def _untouched(big, n):
    return bool(torch.all(big[n:] == SENTINEL))


@pytest.mark.parametrize("M,K,n", CASES)
def test_decode_bf16_and_f32_outputs_exact(M, K, n):
    print(f"decode bf16/f32 M={M} K={K} n={n}", flush=True)
    Xb, X = _ints(300 + M, (M, K))
    Wb, W = _ints(301 + K, (K, n))
    Xd, Wd = to_dev(Xb), to_dev(Wb)
    by, Y = _canary((M, n), torch.bfloat16)
    T.tp_col_linear(Xd, Wd, "none", Y=Y)
    bp, P = _canary((M, n), torch.float32)
    T.tp_row_linear_partial(Xd, Wd, P=P)
    torch.cuda.synchronize()
    want = X @ W
    assert np.array_equal(bits(Y), rne_bf16_bits(want))
    assert np.array_equal(f64(P), want)
    assert _untouched(by, M * n) and _untouched(bp, M * n)
    # accumulate into an existing partial
    P0b, P0 = _ints(302, (M, n))
    P.copy_(torch.from_numpy(P0.astype(np.float32)))
    T.tp_row_linear_partial(Xd, Wd, P=P, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(f64(P), P0 + want)
    assert _untouched(bp, M * n)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("M,K,n", CASES)
def test_decode_activation_epilogues(M, K, n, act):
    print(f"decode {act} M={M} K={K} n_out={n // 2 if act == 'swiglu' else n}", flush=True)
    n_out = n // 2 if act == "swiglu" else n
    Xb, X = _ints(310 + M, (M, K), scale=1 / 16)   # pre-activations of order 1 to 10
    Wb, W = _ints(311 + K, (K, n))
    bz, Z = _canary((M, n_out), torch.bfloat16)
    bh, H = _canary((M, n), torch.bfloat16)
    T.tp_col_linear(to_dev(Xb), to_dev(Wb), act, Y=Z, H_save=H)
    torch.cuda.synchronize()
    oZ, oH = O.col_linear_act(X, W, act)
    assert np.array_equal(bits(H), rne_bf16_bits(oH))
    assert_elementwise(f64(Z), oZ, f"{act} Z")
    assert _untouched(bz, M * n_out) and _untouched(bh, M * n)


def test_decode_split_reuses_a_caller_workspace():
    # the split plan's partials live in the caller's workspace: further
    # calls (other values, same buffer) must not see the earlier partials
    M, K, n = 16, 8192, 1280
    need = T.workspace_size("tp_col_linear", M, K, n, 0)
    assert need > 0 and need % (M * n * 4) == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    Wb, W = _ints(320, (K, n))
    Wd = to_dev(Wb)
    for seed in (321, 322, 323):
        Xb, X = _ints(seed, (M, K))
        Y, _ = T.tp_col_linear(to_dev(Xb), Wd, "none", workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(Y), rne_bf16_bits(X @ W)), seed
