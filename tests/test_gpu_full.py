"""Parity at the full workload sizes, in the launch configuration the benchmark
times: every element of every output against the fp64 oracle (the Llama-3-70B
TP=8 SwiGLU MLP shard forward and backward, the GPT GeLU shard forward, the
Llama-3-70B attention projections at prefill and decode sizes), plus the
bit-exact fused-QKV regroup for every rank of Llama-3-70B at t = 8. The
oracle's backward runs from its own fp64 forward tensors, so the errors
include the bf16 roundings of Z, H and dH on the GPU path."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import check_errs, err, f64, to_dev

pytestmark = pytest.mark.gpu


def test_llama70b_swiglu_shard_fwd_bwd_full_size():
    w = synth.WORKLOADS["llama70b_swiglu_t8"]
    wb = synth.WORKLOADS["llama70b_swiglu_t8_bwd"]
    d = synth.mlp_inputs(w.seed, w.N, w.h, w.F, w.t, "swiglu")
    dYb = synth.mlp_bwd_inputs(wb.seed, w.N, w.h)["dY"]
    X, W_in, W_out, dY = to_dev(d["X"]), to_dev(d["W_in"]), to_dev(d["W_out"]), to_dev(dYb)
    Z, H, P = T.tp_mlp_shard_fwd(X, W_in, W_out, "swiglu")
    dH, dX, dWi, dWo = T.tp_mlp_shard_bwd(X, W_in, W_out, H, Z, dY, "swiglu")
    torch.cuda.synchronize()
    o = {k: synth.bf16_to_f64(v) for k, v in d.items()}
    oZ, oH, oP = O.mlp_shard_fwd(o["X"], o["W_in"], o["W_out"], "swiglu")
    g = O.mlp_shard_bwd_saved(o["X"], o["W_in"], o["W_out"], oH, oZ, synth.bf16_to_f64(dYb), "swiglu")
    errs = {"Z": err(f64(Z), oZ), "H": err(f64(H), oH), "P": err(f64(P), oP), "dH": err(f64(dH), g["dH"]),
            "dX_part": err(f64(dX), g["dX_part"]), "dW_in": err(f64(dWi), g["dW_in"]),
            "dW_out": err(f64(dWo), g["dW_out"])}
    check_errs(errs, "llama70b swiglu t8 (every element)")


def test_gpt_gelu_shard_fwd_full_size():
    w = synth.WORKLOADS["gpt_gelu_t4"]
    d = synth.mlp_inputs(w.seed, w.N, w.h, w.F, w.t, "gelu")
    Z, H, P = T.tp_mlp_shard_fwd(to_dev(d["X"]), to_dev(d["W_in"]), to_dev(d["W_out"]), "gelu")
    torch.cuda.synchronize()
    o = {k: synth.bf16_to_f64(v) for k, v in d.items()}
    oZ, oH, oP = O.mlp_shard_fwd(o["X"], o["W_in"], o["W_out"], "gelu")
    check_errs({"Z": err(f64(Z), oZ), "H": err(f64(H), oH), "P": err(f64(P), oP)},
               "gpt gelu t4 (every element)")


@pytest.fixture(scope="module")
def llama_qkv():
    q = synth.WORKLOADS["llama70b_qkv_t8"]
    return q, synth.qkv_inputs(q.seed, q.N, q.h, q.n_h, q.n_kv, q.d_h, q.t)


def test_llama70b_qkv_regroup_every_rank_exact(llama_qkv):
    q, d = llama_qkv
    W = to_dev(d["W_qkv"])
    for r in range(q.t):
        got = T.tp_qkv_regroup(W, q.n_h, q.n_kv, q.d_h, q.t, r)
        want = O.qkv_regroup(d["W_qkv"], q.n_h, q.n_kv, q.d_h, q.t, r)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), want), r


@pytest.mark.parametrize("N", [4096, 16])
def test_llama70b_attention_projections_full_size(llama_qkv, N):
    q, d = llama_qkv
    r = 3
    Wr_bits = O.qkv_regroup(d["W_qkv"], q.n_h, q.n_kv, q.d_h, q.t, r)
    Xb, Ob = d["X"][:N], d["O"][:N]
    W_r = T.tp_qkv_regroup(to_dev(d["W_qkv"]), q.n_h, q.n_kv, q.d_h, q.t, r)
    X, O_, W_O = to_dev(Xb), to_dev(Ob), to_dev(d["W_O"])
    dQKV, dY = to_dev(d["dQKV"][:N]), to_dev(d["dY"][:N])
    Y, _ = T.tp_col_linear(X, W_r, "none")
    P = T.tp_row_linear_partial(O_, W_O)
    dX, dW = T.tp_col_linear_bwd(X, W_r, dQKV)
    dO, dWO = T.tp_row_linear_bwd(O_, W_O, dY)
    torch.cuda.synchronize()
    X64, O64 = synth.bf16_to_f64(Xb), synth.bf16_to_f64(Ob)
    Wr64, WO64 = synth.bf16_to_f64(Wr_bits), synth.bf16_to_f64(d["W_O"])
    dQ64, dY64 = synth.bf16_to_f64(d["dQKV"][:N]), synth.bf16_to_f64(d["dY"][:N])
    want_dx, want_dw = O.col_linear_bwd(X64, Wr64, dQ64)
    want_do, want_dwo = O.row_linear_bwd(O64, WO64, dY64)
    errs = {
        "Y": err(f64(Y), O.col_linear(X64, Wr64)), "P": err(f64(P), O.row_linear_partial(O64, WO64)),
        "dX": err(f64(dX), want_dx), "dW": err(f64(dW), want_dw),
        "dO": err(f64(dO), want_do), "dWO": err(f64(dWO), want_dwo),
    }
    check_errs(errs, f"llama70b attention projections N={N} (every element)")
