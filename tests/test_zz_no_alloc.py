"""tp_col_linear_noalloc through the C ABI: the same outputs as tp_col_linear
(the same kernels, its workspace replaced by the library's device scratch)
and as the fp64 oracle, bit for bit on integer inputs, on two calls in a row
(the second smaller, its split reusing the scratch the first left), for the
plain and the SwiGLU (+H) products; a product whose split needs more scratch
than the library holds is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import bits, rne_bf16_bits, to_dev

pytestmark = pytest.mark.gpu

SCRATCH = 16 << 20


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _ints(seed, shape, scale=1.0):
    b = synth.int_inputs(seed, shape, scale=scale)
    return b, synth.bf16_to_f64(b)


def _with_workspace(X, W, N, k, n_out, act, Y, H):
    lib = T.load()
    need = T.workspace_size("tp_col_linear", N, k, n_out, act)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda:0")
    st = lib.tp_col_linear(_p(X), _p(W), _p(Y), N, k, n_out, act, _p(H), _p(ws), need, _stream())
    assert st == 0, T.tp_last_error()
    return need


def _noalloc(X, W, N, k, n_out, act, Y, H):
    st = T.load().tp_col_linear_noalloc(_p(X), _p(W), _p(Y), N, k, n_out, act, _p(H), _stream())
    assert st == 0, T.tp_last_error()


@pytest.mark.parametrize("act", [0, 2])   # NONE, SWIGLU (with the saved pre-activation)
def test_noalloc_matches_the_workspace_call_twice_in_a_row(act):
    # decode-sized products (split K); the second call is smaller in every size
    for i, (N, k, n_out) in enumerate([(48, 8192, 1280), (16, 4096, 640)]):
        n_w = 2 * n_out if act == 2 else n_out
        Xb, X = _ints(300 + i, (N, k), scale=1 / 16 if act == 2 else 1.0)
        Wb, W = _ints(310 + i, (k, n_w))
        Xd, Wd = to_dev(Xb), to_dev(Wb)
        Y1 = torch.full((N, n_out), 3.0, dtype=torch.bfloat16, device="cuda:0")
        Y2 = torch.full((N, n_out), 5.0, dtype=torch.bfloat16, device="cuda:0")
        H1 = torch.zeros((N, n_w), dtype=torch.bfloat16, device="cuda:0") if act == 2 else None
        H2 = torch.ones((N, n_w), dtype=torch.bfloat16, device="cuda:0") if act == 2 else None
        need = _with_workspace(Xd, Wd, N, k, n_out, act, Y1, H1)
        assert 0 < need <= SCRATCH, need                 # the product is split
        _noalloc(Xd, Wd, N, k, n_out, act, Y2, H2)
        torch.cuda.synchronize()
        assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16)), (act, i)
        oZ, oH = O.col_linear_act(X, W, "swiglu" if act == 2 else "none")
        if act == 2:
            assert torch.equal(H1.view(torch.int16), H2.view(torch.int16)), i
            assert np.array_equal(bits(H2), rne_bf16_bits(oH)), i
            z = synth.bf16_to_f64(bits(Y2))
            assert np.all(np.abs(z - oZ) <= 2.0 ** -8 * np.abs(oZ) + 1e-6 * np.max(np.abs(oZ))), i
        else:
            assert np.array_equal(bits(Y2), rne_bf16_bits(oZ)), i


def test_noalloc_refuses_a_split_larger_than_its_scratch():
    N, k, n_out = 4096, 8192, 1280           # the attention QKV product at prefill size
    need = T.workspace_size("tp_col_linear", N, k, n_out, 0)
    if need <= SCRATCH:
        pytest.skip(f"this device splits the product into {need} bytes, within the scratch")
    X = torch.zeros((N, k), dtype=torch.bfloat16, device="cuda:0")
    W = torch.zeros((k, n_out), dtype=torch.bfloat16, device="cuda:0")
    Y = torch.full((N, n_out), 3.0, dtype=torch.bfloat16, device="cuda:0")
    st = T.load().tp_col_linear_noalloc(_p(X), _p(W), _p(Y), N, k, n_out, 0, _p(None), _stream())
    assert st == 3 and "scratch" in T.tp_last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 3.0))
