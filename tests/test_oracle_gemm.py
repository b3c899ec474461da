"""Pins of the oracle's products and sharding identities (CPU only).

The identities are the two block-matmul identities of [TPSP] "矩阵乘法的两种切法"
(also [REVISIT] "Tensor Parallel"); the negative cases are the statements of
[TPSP] "MLP：先列后行，只通信一次" that a row split before GeLU, or gate/up
columns from different F segments, give the wrong result.
"""
import numpy as np
import pytest

import oracle as O
import synth


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 2), (4, 8, 16), (7, 3, 9)])
def test_products_match_brute_force(shape):
    n, k, m = shape
    rng = np.random.default_rng(11)
    X, W = _rand(rng, n, k), _rand(rng, k, m)
    ref = O.matmul_loops(X, W)
    assert np.allclose(O.col_linear(X, W), ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(O.row_linear_partial(X, W), ref, rtol=1e-13, atol=1e-13)


def test_brute_force_transposition_detects_swapped_operands():
    # a plausible slip (operands swapped / transposed) must not pass the pin above
    rng = np.random.default_rng(12)
    X, W = _rand(rng, 4, 4), _rand(rng, 4, 4)
    ref = O.matmul_loops(X, W)
    assert not np.allclose(O.col_linear(W, X), ref)
    assert not np.allclose(O.col_linear(X, W.T), ref)


def test_integer_products_are_exact():
    X = synth.bf16_to_f64(synth.int_inputs(1, (16, 64)))
    W = synth.bf16_to_f64(synth.int_inputs(2, (64, 24)))
    assert np.array_equal(O.col_linear(X, W), O.matmul_loops(X, W))


@pytest.mark.parametrize("t", [1, 2, 4])
def test_column_identity(t):
    # X [W_1 ... W_t] = [X W_1 ... X W_t]
    X = synth.bf16_to_f64(synth.int_inputs(3, (8, 32)))
    W = synth.bf16_to_f64(synth.int_inputs(4, (32, 16)))
    parts = [O.col_linear(X, Wi) for Wi in np.split(W, t, axis=1)]
    assert np.array_equal(np.concatenate(parts, axis=1), O.col_linear(X, W))


@pytest.mark.parametrize("t", [1, 2, 4])
def test_row_identity(t):
    # [X_1 ... X_t][W_1; ...; W_t] = sum_i X_i W_i, shards run one after another
    X = synth.bf16_to_f64(synth.int_inputs(5, (8, 32)))
    W = synth.bf16_to_f64(synth.int_inputs(6, (32, 16)))
    acc = np.zeros((8, 16))
    for Xi, Wi in zip(np.split(X, t, axis=1), np.split(W, t, axis=0)):
        acc += O.row_linear_partial(Xi, Wi)
    assert np.array_equal(acc, O.col_linear(X, W))


def _tiny_gelu():
    w = synth.WORKLOADS["tiny_gelu_t4"]
    d = synth.mlp_inputs(w.seed, w.N, w.h, w.F, w.t, "gelu", shard_only=False)
    return w, {k: synth.bf16_to_f64(v) for k, v in d.items()}


def test_tiny_gelu_sum_of_shard_partials_equals_unsharded():
    # the tiny workload: t=4 shards of GeLU(X A_i) B_i summed equal GeLU(X A) B
    w, d = _tiny_gelu()
    X, A, B = d["X"], d["W_in"], d["W_out"]
    full = O.gelu(X @ A) @ B
    acc = np.zeros_like(full)
    for Ai, Bi in zip(np.split(A, w.t, axis=1), np.split(B, w.t, axis=0)):
        _, _, P = O.mlp_shard_fwd(X, Ai, Bi, "gelu")
        acc += P
    assert O.rel_err(acc, full) <= 1e-12


def test_gelu_forbids_row_split_before_activation():
    # GeLU(X A_1 + X A_2) != GeLU(X A_1) + GeLU(X A_2): row-splitting A first fails
    w, d = _tiny_gelu()
    X, A = d["X"], d["W_in"]
    full = O.gelu(X @ A)
    wrong = sum(O.gelu(Xi @ Ai) for Xi, Ai in zip(np.split(X, w.t, axis=1),
                                                   np.split(A, w.t, axis=0)))
    assert O.rel_err(wrong, full) > 0.1


def _swiglu_full(seed=7, N=32, h=64, F=128):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, h))
    Wg = rng.standard_normal((h, F)) / np.sqrt(h)
    Wu = rng.standard_normal((h, F)) / np.sqrt(h)
    Wd = rng.standard_normal((F, h)) / np.sqrt(F)
    return X, Wg, Wu, Wd


@pytest.mark.parametrize("t", [1, 2, 4, 8])
def test_swiglu_shards_sum_to_full_mlp(t):
    X, Wg, Wu, Wd = _swiglu_full()
    F = Wg.shape[1]
    f = F // t
    full = (O.silu(X @ Wg) * (X @ Wu)) @ Wd
    acc = np.zeros_like(full)
    for r in range(t):
        seg = slice(r * f, (r + 1) * f)
        W_gu = np.concatenate([Wg[:, seg], Wu[:, seg]], axis=1)
        _, _, P = O.mlp_shard_fwd(X, W_gu, Wd[seg], "swiglu")
        acc += P
    assert O.rel_err(acc, full) <= 1e-12


def test_swiglu_misaligned_gate_up_segments_fail():
    X, Wg, Wu, Wd = _swiglu_full()
    t = 4
    f = Wg.shape[1] // t
    full = (O.silu(X @ Wg) * (X @ Wu)) @ Wd
    acc = np.zeros_like(full)
    for r in range(t):
        g = slice(r * f, (r + 1) * f)
        u = slice(((r + 1) % t) * f, ((r + 1) % t + 1) * f)   # up from another segment
        W_gu = np.concatenate([Wg[:, g], Wu[:, u]], axis=1)
        _, _, P = O.mlp_shard_fwd(X, W_gu, Wd[g], "swiglu")
        acc += P
    assert O.rel_err(acc, full) > 0.1


def test_swiglu_shard_layout_is_gate_then_up():
    # H = X [W_gate,i | W_up,i]; Z = SiLU(H[:, :f]) * H[:, f:]
    rng = np.random.default_rng(8)
    X = rng.standard_normal((5, 6))
    W = rng.standard_normal((6, 8))
    Z, H = O.col_linear_act(X, W, "swiglu")
    G = O.matmul_loops(X, W[:, :4])
    U = O.matmul_loops(X, W[:, 4:])
    silu_g = [[g / (1.0 + np.exp(-g)) for g in row] for row in G]
    assert np.allclose(H, O.matmul_loops(X, W), rtol=1e-13, atol=1e-13)
    assert np.allclose(Z, np.array(silu_g) * U, rtol=1e-13, atol=1e-13)
    Zg, Hg = O.col_linear_act(X, W, "gelu")
    assert np.allclose(Hg, O.matmul_loops(X, W), rtol=1e-13, atol=1e-13)
    assert Zg.shape == (5, 8) and Z.shape == (5, 4)


def test_rel_err_is_max_abs_diff_over_max_abs_reference():
    # the parity metric, max|got - want| / max|want|, on values where the
    # plausible slips (mean instead of max, the denominator taken from
    # `got`, a signed instead of absolute difference) give other numbers
    got = np.array([[1.0, 2.0], [3.0, -4.0]])
    want = np.array([[1.0, 2.5], [5.0, -4.0]])
    assert O.rel_err(got, want) == pytest.approx(2.0 / 5.0)
    assert O.rel_err(want, got) == pytest.approx(2.0 / 4.0)          # not symmetric
    assert O.rel_err(-got, -want) == pytest.approx(0.4)
    assert np.mean(np.abs(got - want)) / np.mean(np.abs(want)) != pytest.approx(0.4)
    assert O.rel_err(np.array([1.0, 3.0]), np.array([2.0, 1.0])) == pytest.approx(2.0 / 2.0)
    # a reference of zeros: the plain maximum error; empty: 0
    assert O.rel_err(np.array([0.5, -1.5]), np.zeros(2)) == pytest.approx(1.5)
    assert O.rel_err(np.zeros(0), np.zeros(0)) == 0.0
    # NaN in the result is never within any tolerance
    assert not O.rel_err(np.array([np.nan, 1.0]), np.array([1.0, 1.0])) <= 1.0
