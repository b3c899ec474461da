"""Pins of the fused-QKV regroup, the shard arithmetic and the Llama-3 accounting
against what the pages print (tests/golden/*.json carry the citations)."""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)




def test_regroup_rank_contents_llama70b():
    # rank r: Q heads 8r..8r+7, K head r, V head r, in that order
    n_h, n_kv, d_h, t = 64, 8, 128, 8
    for r in range(t):
        idx = O.qkv_regroup_index(n_h, n_kv, d_h, t, r)
        assert idx.shape == (1280,)
        q, k, v = idx[:1024], idx[1024:1152], idx[1152:]
        assert np.array_equal(q, np.arange(r * 1024, (r + 1) * 1024))
        assert np.array_equal(k, 8192 + np.arange(r * 128, (r + 1) * 128))
        assert np.array_equal(v, 8192 + 1024 + np.arange(r * 128, (r + 1) * 128))


@pytest.mark.parametrize("n_h,n_kv,d_h,t", [(64, 8, 128, 8), (64, 8, 128, 4), (32, 8, 16, 2),
                                            (4, 4, 8, 4), (8, 2, 4, 1), (8, 2, 4, 2)])
def test_regroup_is_a_partition_and_groups_match(n_h, n_kv, d_h, t):
    width = (n_h + 2 * n_kv) * d_h
    allidx = np.concatenate([O.qkv_regroup_index(n_h, n_kv, d_h, t, r) for r in range(t)])
    assert np.array_equal(np.sort(allidx), np.arange(width))
    group = n_h // n_kv
    for r in range(t):
        idx = O.qkv_regroup_index(n_h, n_kv, d_h, t, r)
        q_heads = sorted(set(int(c) // d_h for c in idx[: n_h // t * d_h]))
        kv_heads = sorted(set((int(c) - n_h * d_h) // d_h
                              for c in idx[n_h // t * d_h: (n_h // t + n_kv // t) * d_h]))
        # every query head on this rank uses a KV head on this rank
        assert all(qh // group in kv_heads for qh in q_heads)


def test_naive_equal_split_is_wrong_as_the_page_says():
    # first card gets only Q heads, last card gets all of V
    n_h, n_kv, d_h, t = 64, 8, 128, 8
    first = O.naive_split_index(n_h, n_kv, d_h, t, 0)
    last = O.naive_split_index(n_h, n_kv, d_h, t, t - 1)
    assert first.max() < n_h * d_h
    v_cols = np.arange((n_h + n_kv) * d_h, (n_h + 2 * n_kv) * d_h)
    assert np.isin(v_cols, last).all()
    assert not np.array_equal(first, O.qkv_regroup_index(n_h, n_kv, d_h, t, 0))


def test_regroup_copies_columns_exactly():
    # n_h=2, n_kv=2, d_h=5, t=2: source [Q0 Q1 | K0 K1 | V0 V1], each 5 columns
    W = np.arange(6 * 30, dtype=np.uint16).reshape(6, 30)
    for r in range(2):
        Wr = O.qkv_regroup(W, 2, 2, 5, 2, r)
        assert Wr.dtype == np.uint16 and Wr.shape == (6, 15)
        assert np.array_equal(Wr[:, 0:5], W[:, 5 * r: 5 * r + 5])            # Q head r
        assert np.array_equal(Wr[:, 5:10], W[:, 10 + 5 * r: 15 + 5 * r])     # K head r
        assert np.array_equal(Wr[:, 10:15], W[:, 20 + 5 * r: 25 + 5 * r])    # V head r


def test_regroup_divisibility_errors():
    with pytest.raises(ValueError, match="must be a multiple of"):
        O.qkv_regroup_index(64, 8, 128, 7, 0)
    with pytest.raises(ValueError):
        O.qkv_regroup_index(48, 8, 128, 12, 0)    # n_kv < t but KV heads cannot be replicated evenly
    with pytest.raises(ValueError):
        O.qkv_regroup_index(32, 8, 128, 64, 0)    # more ranks than query heads
    with pytest.raises(ValueError):
        O.qkv_regroup_index(64, 8, 128, 8, 8)


@pytest.mark.parametrize("t", [16, 32])
def test_replicated_kv_heads_llama3_8b(t):
    # [TPSP] "GQA：KV 头比 query 头少": Llama-3 8B has 32 query and 8 KV heads; TP can
    # go to 32, and past 8 every KV head is copied to t / 8 cards, each serving its
    # own query heads with it
    n_h, n_kv, d_h = 32, 8, 128
    qh, group = n_h // t, n_h // n_kv
    q_cols, kv_count = [], np.zeros(2 * n_kv, dtype=int)
    for r in range(t):
        idx = O.qkv_regroup_index(n_h, n_kv, d_h, t, r)
        assert idx.shape == ((qh + 2) * d_h,)
        q, k, v = idx[: qh * d_h], idx[qh * d_h: (qh + 1) * d_h], idx[(qh + 1) * d_h:]
        q_cols.append(q)
        kh = (int(k[0]) - n_h * d_h) // d_h
        vh = (int(v[0]) - (n_h + n_kv) * d_h) // d_h
        assert kh == vh == r // (t // n_kv)
        assert np.array_equal(k, n_h * d_h + kh * d_h + np.arange(d_h))
        assert np.array_equal(v, (n_h + n_kv) * d_h + vh * d_h + np.arange(d_h))
        # every query head on this rank uses the KV head on this rank
        assert all(int(c) // d_h // group == kh for c in q)
        kv_count[kh] += 1
        kv_count[n_kv + vh] += 1
        assert r in O.kv_replica_ranks(n_kv, t, kh)
    assert np.array_equal(np.sort(np.concatenate(q_cols)), np.arange(n_h * d_h))
    assert np.all(kv_count == t // n_kv)


def test_replica_kv_gradients_sum_to_the_full_gradient():
    # With replicated KV heads each replica's K/V weight gradient is a partial
    # sum ([TPSP] "GQA：KV 头比 query 头少"). Loss L = sum_r <G_r, X W_qkv[:, idx_r]>
    # (rank r's projection with upstream gradient G_r); its gradient with respect
    # to W_qkv, by central differences, must equal each rank's own Q columns of
    # X^T G_r and, for each KV head, the replicas' K|V columns summed.
    rng = np.random.default_rng(11)
    n_h, n_kv, d_h, t, h, N = 4, 2, 2, 4, 3, 5
    width = (n_h + 2 * n_kv) * d_h
    X = rng.standard_normal((N, h))
    W = rng.standard_normal((h, width))
    idxs = [O.qkv_regroup_index(n_h, n_kv, d_h, t, r) for r in range(t)]
    G = [rng.standard_normal((N, len(i))) for i in idxs]

    def loss(Wq):
        return sum(float(np.sum(G[r] * (X @ Wq[:, idxs[r]]))) for r in range(t))

    fd = np.zeros_like(W)
    eps = 1e-3
    for a in range(h):
        for b in range(width):
            Wp, Wm = W.copy(), W.copy()
            Wp[a, b] += eps
            Wm[a, b] -= eps
            fd[a, b] = (loss(Wp) - loss(Wm)) / (2 * eps)
    dWs = [O.col_linear_bwd(X, W[:, idxs[r]], G[r])[1] for r in range(t)]
    qw = (n_h // t) * d_h
    for r in range(t):
        assert np.allclose(dWs[r][:, :qw], fd[:, idxs[r][:qw]], atol=1e-8)
    sums = O.kv_replica_grad_sum(dWs, n_h, n_kv, d_h, t)
    for g in range(n_kv):
        k_cols = n_h * d_h + g * d_h + np.arange(d_h)
        v_cols = (n_h + n_kv) * d_h + g * d_h + np.arange(d_h)
        assert np.allclose(sums[g], fd[:, np.concatenate([k_cols, v_cols])], atol=1e-8)
        # the pairwise accumulate, in rank order, gives the same sum; Q untouched
        ranks = O.kv_replica_ranks(n_kv, t, g)
        acc = dWs[ranks[0]]
        for r in ranks[1:]:
            acc = O.kv_grad_accumulate(acc, dWs[r], n_h, n_kv, d_h, t)
        assert np.array_equal(acc[:, qw:], sums[g])
        assert np.array_equal(acc[:, :qw], dWs[ranks[0]][:, :qw])
    with pytest.raises(ValueError):
        O.kv_grad_accumulate(dWs[0], dWs[1], 8, 8, 2, 4)       # no replicas when t <= n_kv


def test_shard_shape_pop_quiz():
    g = _gold("shard_quiz.json")
    mesh = dict((a, s) for a, s in g["mesh"])
    spec = [tuple(x) for x in g["spec"]]
    shape, local_bytes, total = O.shard_shape(g["shape"], g["elem_bytes"], mesh, spec)
    assert list(shape) == g["local_shape"]
    assert local_bytes == g["local_bytes"]
    assert total == g["total_bytes"]
    with pytest.raises(O.ShardError):
        O.shard_shape(g["shape"], 1, mesh, [tuple(x) for x in g["illegal_same_axis_spec"]])


def test_shard_shape_more_cases():
    mesh = {"X": 4, "Y": 2}
    assert O.shard_shape((8, 6), 2, mesh, [("X",), ("Y",)]) == ((2, 3), 12, 96)
    assert O.shard_shape((8, 6), 2, mesh, [("Y", "X"), ()]) == ((1, 6), 12, 96)
    with pytest.raises(O.ShardError):
        O.shard_shape((6, 6), 2, mesh, [("X",), ()])          # 6 not divisible by 4
    with pytest.raises(O.ShardError):
        O.shard_shape((8, 8), 2, mesh, [("X", "X"), ()])      # axis twice in one dim


def test_llama3_param_counts_match_printed():
    g = _gold("llama3_printed.json")
    c, p = g["llama3_70b"], g["printed"]
    layer = O.llama_layer_params(c["h"], c["n_h"], c["n_kv"], c["d_h"], c["F"])
    per_card = O.llama_layer_params(c["h"], c["n_h"], c["n_kv"], c["d_h"], c["F"], t=c["t"])
    assert layer == 855_638_016 and per_card == 106_954_752
    assert round(layer / 1e8, 2) == p["layer_params_1e8"]
    assert round(per_card / 1e8, 2) == p["layer_params_per_card_1e8"]
    model = O.llama_model_params(c["h"], c["n_h"], c["n_kv"], c["d_h"], c["F"], c["L"], c["V"])
    assert round(model / 1e8) == p["model_params_1e8"]
    assert round(model / c["t"] / 1e8) == p["model_params_per_card_1e8"]
    s8 = g["llama3_8b"]
    emb = 2 * s8["V"] * s8["h"]
    m8 = O.llama_model_params(s8["h"], s8["n_h"], s8["n_kv"], s8["d_h"], s8["F"], s8["L"], s8["V"])
    assert round(emb / 1e8, 1) == p["llama3_8b_embed_plus_head_1e8"]
    assert round(100 * emb / m8) == p["llama3_8b_embed_share_percent"]


def test_llama3_shard_shapes_and_flops_match_printed():
    g = _gold("llama3_printed.json")
    c, p = g["llama3_70b"], g["printed"]
    shapes = O.llama_shard_weight_shapes(c["h"], c["n_h"], c["n_kv"], c["d_h"], c["F"], c["t"])
    assert shapes["W_down"] == (3584, 8192)
    assert int(np.prod(shapes["W_down"]) * 2 / 1e6) == p["mlp_weight_shard_mb"]
    b, s = 1, 4096
    layer = O.llama_layer_params(c["h"], c["n_h"], c["n_kv"], c["d_h"], c["F"])
    lin = 2 * b * s * layer
    attn = 2 * b * s * s * c["h"]
    assert round(lin / 1e12, 1) == p["fwd_tflop_linear_b1_s4096"]
    assert round(attn / 1e12, 2) == p["fwd_tflop_causal_attention_b1_s4096"]
    assert round((lin + attn) / 1e12, 1) == p["fwd_tflop_layer_b1_s4096"]
    per_card = 3 * (lin + attn) / c["t"]
    assert round(per_card / 1e12, 2) == p["per_card_fwd_bwd_tflop"]
    assert round(per_card / 990e12 * 1e3, 2) == p["per_card_ms_at_990_tflops"]
    # the MLP share of that linear count equals our GEMM accounting of one shard
    N, h, f = b * s, c["h"], c["F"] // c["t"]
    mlp_params_card = sum(int(np.prod(shapes[k])) for k in ("W_gate", "W_up", "W_down"))
    assert O.mlp_shard_flops(N, h, f, "swiglu") == 2 * N * mlp_params_card
    assert O.mlp_shard_flops(N, h, f, "swiglu", backward=True) == 2 * O.mlp_shard_flops(
        N, h, f, "swiglu")
