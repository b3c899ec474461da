"""Random-value parity of the MLP shard (forward and backward), the tiny
t-shard workload and the QKV / W_O projections at small sizes, against the
fp64 oracle, within max|gpu - oracle| / max|oracle| <= 2e-2 per tensor."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import TOL, check_errs, err, f64, to_dev

pytestmark = pytest.mark.gpu


def _mlp(seed, N, h, F, t, act):
    d = synth.mlp_inputs(seed, N, h, F, t, act)
    return d, {k: synth.bf16_to_f64(v) for k, v in d.items()}


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("N,h,F,t", [(300, 256, 768, 4), (1, 128, 512, 8), (16, 512, 1024, 4),
                                     (513, 384, 2048, 8)])
def test_mlp_shard_fwd_bwd_parity(act, N, h, F, t):
    d, o = _mlp(20 + N, N, h, F, t, act)
    dYb = synth.mlp_bwd_inputs(21 + N, N, h)["dY"]
    dY = synth.bf16_to_f64(dYb)
    X, W_in, W_out = to_dev(d["X"]), to_dev(d["W_in"]), to_dev(d["W_out"])
    Z, H, P = T.tp_mlp_shard_fwd(X, W_in, W_out, act)
    dH, dX, dWi, dWo = T.tp_mlp_shard_bwd(X, W_in, W_out, H, Z, to_dev(dYb), act)
    torch.cuda.synchronize()
    oZ, oH, oP = O.mlp_shard_fwd(o["X"], o["W_in"], o["W_out"], act)
    g = O.mlp_shard_bwd(o["X"], o["W_in"], o["W_out"], dY, act)
    errs = {"Z": err(f64(Z), oZ), "H": err(f64(H), oH), "P": err(f64(P), oP),
            "dH": err(f64(dH), g["dH"]), "dX_part": err(f64(dX), g["dX_part"]),
            "dW_in": err(f64(dWi), g["dW_in"]), "dW_out": err(f64(dWo), g["dW_out"])}
    check_errs(errs, f"{act} N={N} h={h} F={F} t={t}")


def test_tiny_gelu_four_shards_sum_to_unsharded():
    # t = 4 shards of GeLU(X A_i) B_i computed one after another into one buffer
    w = synth.WORKLOADS["tiny_gelu_t4"]
    d = synth.mlp_inputs(w.seed, w.N, w.h, w.F, w.t, "gelu", shard_only=False)
    o = {k: synth.bf16_to_f64(v) for k, v in d.items()}
    f = w.F // w.t
    X = to_dev(d["X"])
    P = torch.zeros((w.N, w.h), dtype=torch.float32, device="cuda:0")
    for r in range(w.t):
        A_r = to_dev(np.ascontiguousarray(d["W_in"][:, r * f:(r + 1) * f]))
        B_r = to_dev(np.ascontiguousarray(d["W_out"][r * f:(r + 1) * f]))
        T.tp_mlp_shard_fwd(X, A_r, B_r, "gelu", P=P, want_h=False, accumulate=True)
    torch.cuda.synchronize()
    full = O.gelu(o["X"] @ o["W_in"]) @ o["W_out"]
    e = err(f64(P), full)
    print("tiny t=4 sum of partials vs unsharded:", e)
    assert e <= TOL


def test_accumulate_into_dx_partial():
    d, o = _mlp(30, 64, 128, 512, 4, "swiglu")
    dYb = synth.mlp_bwd_inputs(31, 64, 128)["dY"]
    X, W_in, W_out = to_dev(d["X"]), to_dev(d["W_in"]), to_dev(d["W_out"])
    Z, H, _ = T.tp_mlp_shard_fwd(X, W_in, W_out, "swiglu")
    dX = torch.ones((64, 128), dtype=torch.float32, device="cuda:0")
    T.tp_mlp_shard_bwd(X, W_in, W_out, H, Z, to_dev(dYb), "swiglu", dX_part=dX, accumulate=True)
    torch.cuda.synchronize()
    g = O.mlp_shard_bwd(o["X"], o["W_in"], o["W_out"], synth.bf16_to_f64(dYb), "swiglu")
    assert err(f64(dX), 1.0 + g["dX_part"]) <= TOL


@pytest.mark.parametrize("N", [16, 300, 0])
def test_backward_outputs_skipped_when_not_requested(N):
    # each subset of {dX_part, dW_in, dW_out}: the requested outputs are the
    # ones the full call gives (bit for bit: same kernels, same order), the
    # others are not written
    d, o = _mlp(50 + N, N, 256, 1024, 4, "swiglu")
    dYb = synth.mlp_bwd_inputs(51 + N, N, 256)["dY"]
    X, W_in, W_out, dY = to_dev(d["X"]), to_dev(d["W_in"]), to_dev(d["W_out"]), to_dev(dYb)
    Z, H, _ = T.tp_mlp_shard_fwd(X, W_in, W_out, "swiglu")
    full = T.tp_mlp_shard_bwd(X, W_in, W_out, H, Z, dY, "swiglu")
    torch.cuda.synchronize()
    g = O.mlp_shard_bwd(o["X"], o["W_in"], o["W_out"], synth.bf16_to_f64(dYb), "swiglu")
    assert err(f64(full[0]), g["dH"]) <= TOL
    names = ("dX_part", "dW_in", "dW_out")
    for mask in range(8):
        want = tuple(n for i, n in enumerate(names) if mask >> i & 1)
        outs = {n: torch.full_like(full[1 + i], 7.0) for i, n in enumerate(names)}
        dH = torch.zeros_like(full[0])
        res = T.tp_mlp_shard_bwd(X, W_in, W_out, H, Z, dY, "swiglu", dH=dH, want=want,
                                 **{n: outs[n] for n in want})
        torch.cuda.synchronize()
        assert torch.equal(dH.view(torch.int16), full[0].view(torch.int16)), mask
        for i, n in enumerate(names):
            if n in want:
                assert res[1 + i] is outs[n]
                assert torch.equal(outs[n], full[1 + i]), (mask, n)
            else:
                assert res[1 + i] is None
                assert bool(torch.all(outs[n] == 7.0)), (mask, n)


@pytest.mark.parametrize("N", [16, 300])
def test_qkv_and_wo_shard_small(N):
    n_h, n_kv, d_h, t, h = 8, 4, 32, 4, 256
    d = synth.qkv_inputs(40, N, h, n_h, n_kv, d_h, t)
    o = {k: synth.bf16_to_f64(v) for k, v in d.items()}
    for r in range(t):
        W_r = T.tp_qkv_regroup(to_dev(d["W_qkv"]), n_h, n_kv, d_h, t, r)
        Wr_bits = O.qkv_regroup(d["W_qkv"], n_h, n_kv, d_h, t, r)
        torch.cuda.synchronize()
        assert np.array_equal(W_r.cpu().view(torch.int16).numpy().view(np.uint16), Wr_bits)
    W_r = to_dev(Wr_bits)
    Y, _ = T.tp_col_linear(to_dev(d["X"]), W_r, "none")
    P = T.tp_row_linear_partial(to_dev(d["O"]), to_dev(d["W_O"]))
    dX, dW = T.tp_col_linear_bwd(to_dev(d["X"]), W_r, to_dev(d["dQKV"]))
    dO, dWO = T.tp_row_linear_bwd(to_dev(d["O"]), to_dev(d["W_O"]), to_dev(d["dY"]))
    torch.cuda.synchronize()
    Wr = synth.bf16_to_f64(Wr_bits)
    assert err(f64(Y), O.col_linear(o["X"], Wr)) <= TOL
    assert err(f64(P), O.row_linear_partial(o["O"], o["W_O"])) <= TOL
    want_dx, want_dw = O.col_linear_bwd(o["X"], Wr, o["dQKV"])
    assert err(f64(dX), want_dx) <= TOL and err(f64(dW), want_dw) <= TOL
    want_do, want_dwo = O.row_linear_bwd(o["O"], o["W_O"], o["dY"])
    assert err(f64(dO), want_do) <= TOL and err(f64(dWO), want_dwo) <= TOL


def test_invalid_shapes_raise_value_error():
    X = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda:0")
    W = torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(NotImplementedError):
        T.tp_col_linear(X, W, "none")
    Wq = torch.zeros((64, (64 + 16) * 8), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError, match="multiple of tensor_model_parallel_size"):
        T.tp_qkv_regroup(Wq, 64, 8, 8, 7, 0)
