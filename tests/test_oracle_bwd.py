"""Pins of the oracle's backward: central finite differences of L = sum(dY * out),
the shard-vs-full gradient identity (dX = sum_i dX_part,i) and the sampled
(row / column restricted) forms against the full computation."""
import numpy as np
import pytest

import oracle as O


def _fd_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        hi = f()
        x[i] = old - eps
        lo = f()
        x[i] = old
        g[i] = (hi - lo) / (2 * eps)
    return g


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_mlp_shard_bwd_finite_differences(act):
    rng = np.random.default_rng(3)
    N, h, f = 3, 4, 3
    n_w = 2 * f if act == "swiglu" else f
    X = rng.standard_normal((N, h))
    W_in = rng.standard_normal((h, n_w))
    W_out = rng.standard_normal((f, h))
    dY = rng.standard_normal((N, h))

    def loss():
        return float(np.sum(dY * O.mlp_shard_fwd(X, W_in, W_out, act)[2]))

    g = O.mlp_shard_bwd(X, W_in, W_out, dY, act)
    assert np.allclose(g["dX_part"], _fd_grad(loss, X), rtol=1e-6, atol=1e-7)
    assert np.allclose(g["dW_in"], _fd_grad(loss, W_in), rtol=1e-6, atol=1e-7)
    assert np.allclose(g["dW_out"], _fd_grad(loss, W_out), rtol=1e-6, atol=1e-7)


def test_linear_bwd_finite_differences():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3, 5))
    W = rng.standard_normal((5, 4))
    dY = rng.standard_normal((3, 4))

    def loss():
        return float(np.sum(dY * O.col_linear(X, W)))

    dX, dW = O.col_linear_bwd(X, W, dY)
    assert np.allclose(dX, _fd_grad(loss, X), rtol=1e-7, atol=1e-8)
    assert np.allclose(dW, _fd_grad(loss, W), rtol=1e-7, atol=1e-8)
    dX2, dW2 = O.row_linear_bwd(X, W, dY)
    assert np.allclose(dX2, dX) and np.allclose(dW2, dW)


def test_column_parallel_dx_partials_sum_to_full():
    # dX = sum_i dY_i W_i^T over the t column shards
    rng = np.random.default_rng(5)
    X = rng.standard_normal((6, 8))
    W = rng.standard_normal((8, 12))
    dY = rng.standard_normal((6, 12))
    full_dX, full_dW = O.col_linear_bwd(X, W, dY)
    t = 4
    acc = np.zeros_like(full_dX)
    dWs = []
    for Wi, dYi in zip(np.split(W, t, axis=1), np.split(dY, t, axis=1)):
        dXi, dWi = O.col_linear_bwd(X, Wi, dYi)
        acc += dXi
        dWs.append(dWi)
    assert np.allclose(acc, full_dX, rtol=1e-13, atol=1e-13)
    assert np.allclose(np.concatenate(dWs, axis=1), full_dW, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_sampled_forms_match_full(act):
    rng = np.random.default_rng(6)
    N, h, f = 20, 16, 12
    n_w = 2 * f if act == "swiglu" else f
    X = rng.standard_normal((N, h))
    W_in = rng.standard_normal((h, n_w)) / 4
    W_out = rng.standard_normal((f, h)) / 4
    dY = rng.standard_normal((N, h))
    Z, H, P = O.mlp_shard_fwd(X, W_in, W_out, act)
    g = O.mlp_shard_bwd(X, W_in, W_out, dY, act)
    rows = np.array([0, 3, 19, 7])
    Zr, Hr, Pr = O.mlp_shard_fwd_rows(X, W_in, W_out, act, rows)
    assert np.allclose(Pr, P[rows]) and np.allclose(Zr, Z[rows]) and np.allclose(Hr, H[rows])
    br = O.mlp_shard_bwd_rows(X, W_in, W_out, dY, act, rows)
    assert np.allclose(br["dH"], g["dH"][rows])
    assert np.allclose(br["dX_part"], g["dX_part"][rows])
    cols = np.array([1, 5, 11])
    bc = O.mlp_shard_bwd_cols(X, W_in, W_out, dY, act, cols)
    sel = np.concatenate([cols, f + cols]) if act == "swiglu" else cols
    assert np.allclose(bc["dW_in_cols"], g["dW_in"][:, sel])
    assert np.allclose(bc["dW_out_rows"], g["dW_out"][cols])


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_bwd_from_saved_tensors_is_the_recomputing_bwd(act):
    # mlp_shard_bwd recomputes H, Z; mlp_shard_bwd_saved takes the forward's:
    # the same gradients (and a planted swap of Z for H fails)
    rng = np.random.default_rng(11)
    N, h, f = 5, 6, 4
    n_w = 2 * f if act == "swiglu" else f
    X = rng.standard_normal((N, h))
    W_in = rng.standard_normal((h, n_w))
    W_out = rng.standard_normal((f, h))
    dY = rng.standard_normal((N, h))
    Z, H, _ = O.mlp_shard_fwd(X, W_in, W_out, act)
    g = O.mlp_shard_bwd(X, W_in, W_out, dY, act)
    s = O.mlp_shard_bwd_saved(X, W_in, W_out, H, Z, dY, act)
    for k in ("dZ", "dH", "dX_part", "dW_in", "dW_out"):
        assert np.array_equal(g[k], s[k]), k
    if act == "gelu":
        wrong = O.mlp_shard_bwd_saved(X, W_in, W_out, Z, Z, dY, act)
        assert not np.allclose(wrong["dX_part"], g["dX_part"])
