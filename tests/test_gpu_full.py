"""Parity at the full workload sizes, in the launch configuration the benchmark
times, on sampled outputs the oracle computes one by one (token rows of the
forward outputs and of dX; columns of the weight gradients), plus the
bit-exact fused-QKV regroup for every rank of Llama-3-70B at t = 8."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import TOL, err, f64, to_dev

pytestmark = pytest.mark.gpu


def _rows(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=k, replace=False)]))


@pytest.fixture(scope="module")
def llama_mlp():
    w = synth.WORKLOADS["llama70b_swiglu_t8"]
    wb = synth.WORKLOADS["llama70b_swiglu_t8_bwd"]
    d = synth.mlp_inputs(w.seed, w.N, w.h, w.F, w.t, "swiglu")
    dY = synth.mlp_bwd_inputs(wb.seed, w.N, w.h)["dY"]
    return w, d, dY


def test_llama70b_swiglu_shard_fwd_bwd_full_size(llama_mlp):
    w, d, dYb = llama_mlp
    N, h, f = w.N, w.h, w.f
    X, W_in, W_out, dY = to_dev(d["X"]), to_dev(d["W_in"]), to_dev(d["W_out"]), to_dev(dYb)
    Z, H, P = T.tp_mlp_shard_fwd(X, W_in, W_out, "swiglu")
    dH, dX, dWi, dWo = T.tp_mlp_shard_bwd(X, W_in, W_out, H, Z, dY, "swiglu")
    torch.cuda.synchronize()
    o = {k: synth.bf16_to_f64(v) for k, v in d.items()}
    dY64 = synth.bf16_to_f64(dYb)
    rows = _rows(N, 40, 1)
    oZ, oH, oP = O.mlp_shard_fwd_rows(o["X"], o["W_in"], o["W_out"], "swiglu", rows)
    br = O.mlp_shard_bwd_rows(o["X"], o["W_in"], o["W_out"], dY64, "swiglu", rows)
    cols = _rows(f, 22, 2)
    bc = O.mlp_shard_bwd_cols(o["X"], o["W_in"], o["W_out"], dY64, "swiglu", cols)
    sel = np.concatenate([cols, f + cols])
    errs = {
        "Z": err(f64(Z[rows]), oZ), "H": err(f64(H[rows]), oH), "P": err(f64(P[rows]), oP),
        "dH": err(f64(dH[rows]), br["dH"]), "dX_part": err(f64(dX[rows]), br["dX_part"]),
        "dW_in": err(f64(dWi[:, sel]), bc["dW_in_cols"]),
        "dW_out": err(f64(dWo[cols]), bc["dW_out_rows"]),
    }
    print({k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    assert torch.isfinite(P).all() and torch.isfinite(dWi).all() and torch.isfinite(dWo).all()


def test_gpt_gelu_shard_fwd_full_size():
    w = synth.WORKLOADS["gpt_gelu_t4"]
    d = synth.mlp_inputs(w.seed, w.N, w.h, w.F, w.t, "gelu")
    Z, H, P = T.tp_mlp_shard_fwd(to_dev(d["X"]), to_dev(d["W_in"]), to_dev(d["W_out"]), "gelu")
    torch.cuda.synchronize()
    o = {k: synth.bf16_to_f64(v) for k, v in d.items()}
    rows = _rows(w.N, 40, 3)
    oZ, oH, oP = O.mlp_shard_fwd_rows(o["X"], o["W_in"], o["W_out"], "gelu", rows)
    for name, got, want in (("Z", Z, oZ), ("H", H, oH), ("P", P, oP)):
        e = err(f64(got[rows]), want)
        print(name, f"{e:.2e}")
        assert e <= TOL


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
    rows = _rows(N, min(N - 2, 40), 4)
    cols = _rows(Wr64.shape[1], 20, 5)
    ocols = _rows(WO64.shape[0], 20, 6)
    errs = {
        "Y": err(f64(Y[rows]), O.col_linear(X64[rows], Wr64)),
        "P": err(f64(P[rows]), O.row_linear_partial(O64[rows], WO64)),
        "dX": err(f64(dX[rows]), O.col_linear_bwd(X64[rows], Wr64, dQ64[rows])[0]),
        "dW": err(f64(dW[:, cols]), O.col_linear_bwd(X64, Wr64[:, cols], dQ64[:, cols])[1]),
        "dO": err(f64(dO[rows]), O.row_linear_bwd(O64[rows], WO64, dY64[rows])[0]),
        "dWO": err(f64(dWO[ocols]), O.row_linear_bwd(O64[:, ocols], WO64[ocols], dY64)[1]),
    }
    print(N, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
