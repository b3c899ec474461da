"""Pins of the oracle's vocab-parallel cross-entropy ([TPSP] "LM head 与交叉熵")
against what the mathematics fixes: the unsharded cross-entropy (scipy's
logsumexp on the concatenated logits), uniform logits (loss = log V), the
rescaled merge of per-shard statistics, gradient rows that sum to zero, and
central differences of the sharded loss."""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle as O


def _problem(seed, N=7, h=5, V=24, t=4):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, h))
    W = rng.standard_normal((h, V)) * 1.5
    y = rng.integers(0, V, size=N)
    shards = np.split(W, t, axis=1)
    return X, W, y, shards


@pytest.mark.parametrize("t", [1, 2, 4])
def test_sharded_loss_is_the_unsharded_cross_entropy(t):
    X, W, y, _ = _problem(1, t=t)
    loss, m, S = O.vocab_ce_loss(X, np.split(W, t, axis=1), y)
    z = X @ W
    want = logsumexp(z, axis=1) - z[np.arange(len(y)), y]
    assert np.allclose(loss, want, rtol=0, atol=1e-12)
    assert np.allclose(np.log(S) + m, logsumexp(z, axis=1), atol=1e-12)


def test_uniform_logits_give_log_v():
    X, W, y, _ = _problem(2)
    loss, m, S = O.vocab_ce_loss(X, np.split(np.zeros_like(W), 4, axis=1), y)
    assert np.allclose(loss, np.log(W.shape[1]), atol=1e-14)
    assert np.all(m == 0) and np.allclose(S, W.shape[1])


def test_local_statistics_merge_to_the_global_ones():
    # the single-device merge: m = max m_i, S = sum_i s_i exp(m_i - m), z_y = sum_i z_y,i
    X, W, y, shards = _problem(3)
    loss, m, S = O.vocab_ce_loss(X, shards, y)
    starts = np.cumsum([0] + [s.shape[1] for s in shards[:-1]])
    stats = [O.vocab_ce_local(X, Wi, y, st) for Wi, st in zip(shards, starts)]
    mm = np.max([st[0] for st in stats], axis=0)
    SS = np.sum([st[1] * np.exp(st[0] - mm) for st in stats], axis=0)
    zy = np.sum([st[2] for st in stats], axis=0)
    assert np.allclose(mm, m) and np.allclose(SS, S, rtol=1e-13)
    assert np.allclose(np.log(SS) + mm - zy, loss, atol=1e-12)
    # exactly one shard holds each token's target
    held = np.sum([(y >= st) & (y < st + Wi.shape[1]) for Wi, st in zip(shards, starts)], axis=0)
    assert np.all(held == 1)


def test_gradient_rows_sum_to_zero():
    X, W, y, shards = _problem(4)
    loss, m, S = O.vocab_ce_loss(X, shards, y)
    dloss = np.linspace(0.5, 2.0, len(y))
    starts = np.cumsum([0] + [s.shape[1] for s in shards[:-1]])
    dZ = np.concatenate([O.vocab_ce_bwd(X, Wi, y, st, m, S, dloss)[0] for Wi, st in zip(shards, starts)],
                        axis=1)
    assert np.allclose(dZ.sum(axis=1), 0.0, atol=1e-12)
    assert np.all(dZ[np.arange(len(y)), y] < 0)


def test_backward_matches_central_differences():
    X, W, y, shards = _problem(5, N=4, h=3, V=8, t=2)
    dloss = np.array([1.0, 0.5, 2.0, 1.5])

    def L(Xv, Ws):
        return float(np.sum(dloss * O.vocab_ce_loss(Xv, Ws, y)[0]))

    loss, m, S = O.vocab_ce_loss(X, shards, y)
    starts = [0, shards[0].shape[1]]
    outs = [O.vocab_ce_bwd(X, Wi, y, st, m, S, dloss) for Wi, st in zip(shards, starts)]
    dX = sum(o[1] for o in outs)                       # the f all-reduce of dX_part
    eps = 1e-5
    fdX = np.zeros_like(X)
    for a in range(X.shape[0]):
        for b in range(X.shape[1]):
            Xp, Xm = X.copy(), X.copy()
            Xp[a, b] += eps
            Xm[a, b] -= eps
            fdX[a, b] = (L(Xp, shards) - L(Xm, shards)) / (2 * eps)
    assert np.allclose(dX, fdX, atol=1e-7)
    for i in range(2):
        fdW = np.zeros_like(shards[i])
        for a in range(fdW.shape[0]):
            for b in range(fdW.shape[1]):
                Wp = [s.copy() for s in shards]
                Wm = [s.copy() for s in shards]
                Wp[i][a, b] += eps
                Wm[i][a, b] -= eps
                fdW[a, b] = (L(X, Wp) - L(X, Wm)) / (2 * eps)
        assert np.allclose(outs[i][2], fdW, atol=1e-7)


def test_masked_lookups_sum_to_the_one_hot_product():
    # [TPSP] "输入 embedding": the lookup is the one-hot [N, V] times the table
    # [V, h], split on the contraction dim V (a row-parallel layer); each
    # token gets a non-zero row from exactly one rank
    rng = np.random.default_rng(6)
    N, V, h, t = 11, 20, 3, 4
    E = rng.standard_normal((V, h))
    ids = rng.integers(0, V, size=N)
    ids[:2] = [0, V - 1]
    onehot = np.zeros((N, V))
    onehot[np.arange(N), ids] = 1.0
    parts = [O.vocab_embed_fwd(ids, E[i * V // t:(i + 1) * V // t], i * V // t) for i in range(t)]
    assert np.array_equal(sum(parts), onehot @ E)
    nonzero = np.sum([np.any(p != 0, axis=1) for p in parts], axis=0)
    assert np.all(nonzero == 1)
    # backward: dE = onehot^T dY, per rank its own rows
    dY = rng.standard_normal((N, h))
    full = onehot.T @ dY
    for i in range(t):
        got = O.vocab_embed_bwd(ids, dY, i * V // t, V // t)
        assert np.allclose(got, full[i * V // t:(i + 1) * V // t], atol=1e-12)
