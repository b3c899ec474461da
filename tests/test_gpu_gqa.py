"""GQA with fewer KV heads than ranks (n_kv < t): the regroup replicates each KV
head on t / n_kv ranks, bit for bit against the oracle's index definition, and
the replicas' K|V weight gradients (tp_col_linear_bwd's dW of each rank, then
tp_kv_grad_accumulate in rank order) equal the oracle's replica sum exactly on
integer inputs."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import bits, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("h,n_h,n_kv,d_h,t", [(4096, 32, 8, 128, 16), (4096, 32, 8, 128, 32),
                                              (8192, 64, 8, 128, 16), (520, 16, 2, 8, 8)])
def test_regroup_replicated_kv_every_rank_exact(h, n_h, n_kv, d_h, t):
    W = synth.int_inputs(60, (h, (n_h + 2 * n_kv) * d_h), lo=-30000, hi=30000)
    Wd = to_dev(W)
    for r in range(t):
        got = T.tp_qkv_regroup(Wd, n_h, n_kv, d_h, t, r)
        torch.cuda.synchronize()
        want = O.qkv_regroup(W, n_h, n_kv, d_h, t, r)
        assert got.shape == want.shape, r
        assert np.array_equal(bits(got), want), r


def test_kv_grad_accumulate_exact():
    h, n_h, n_kv, d_h, t = 1000, 64, 8, 128, 16
    w = (n_h // t + 2) * d_h
    rng = np.random.default_rng(3)
    a = rng.standard_normal((h, w)).astype(np.float32)
    b = rng.standard_normal((h, w)).astype(np.float32)
    dst = torch.from_numpy(a).to("cuda:0")
    src = torch.from_numpy(b).to("cuda:0")
    T.tp_kv_grad_accumulate(dst, src, n_h, n_kv, d_h, t)
    torch.cuda.synchronize()
    want = O.kv_grad_accumulate(a, b, n_h, n_kv, d_h, t).astype(np.float32)  # f32 sum, rounded once
    assert np.array_equal(dst.cpu().numpy(), want)


def test_replica_weight_gradients_sum_exact():
    # integer entries: every GEMM and every sum below is exact in f32
    N, h, n_h, n_kv, d_h, t = 300, 256, 32, 8, 16, 16
    width = (n_h + 2 * n_kv) * d_h
    X = synth.int_inputs(61, (N, h))
    W = synth.int_inputs(62, (h, width))
    Xd = to_dev(X)
    dWs_gpu, dWs_ref = [], []
    for r in range(t):
        W_r = O.qkv_regroup(W, n_h, n_kv, d_h, t, r)
        G = synth.int_inputs(70 + r, (N, W_r.shape[1]))
        _, dW = T.tp_col_linear_bwd(Xd, to_dev(W_r), to_dev(G), want_dx=False)
        dWs_gpu.append(dW)
        dWs_ref.append(O.col_linear_bwd(synth.bf16_to_f64(X), synth.bf16_to_f64(W_r), synth.bf16_to_f64(G))[1])
    want = O.kv_replica_grad_sum(dWs_ref, n_h, n_kv, d_h, t)
    q = (n_h // t) * d_h
    for g in range(n_kv):
        ranks = O.kv_replica_ranks(n_kv, t, g)
        acc = dWs_gpu[ranks[0]].clone()
        for r in ranks[1:]:
            T.tp_kv_grad_accumulate(acc, dWs_gpu[r], n_h, n_kv, d_h, t)
        torch.cuda.synchronize()
        got = f64(acc)
        assert np.array_equal(got[:, q:], want[g]), g
        assert np.array_equal(got[:, :q], dWs_ref[ranks[0]][:, :q]), g
