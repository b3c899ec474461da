"""Vocab-parallel embedding through the C ABI: each rank's masked lookup is a
bit-exact copy of the oracle's, the t ranks accumulated on one buffer give the
full lookup (equal in value), and the table gradient equals the oracle's
(exact on integer gradients; repeated ids summed in token order)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_sharded_matmul_amd as T
from gpu_util import TOL, bits, err, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,V,h,t", [(300, 1000, 256, 4), (4096, 16128 * 2, 8192, 2), (5, 64, 64, 1)])
def test_embedding_forward_backward(N, V, h, t):
    rng = np.random.default_rng(N + V)
    v_loc = V // t
    E = synth.draw(rng, (V, h))
    ids = rng.integers(0, V, size=N).astype(np.int32)
    ids[: min(N, 4)] = [0, V - 1, v_loc - 1, v_loc][: min(N, 4)]
    ids[N // 2:] = ids[: N - N // 2]                 # repeated ids
    idd = torch.from_numpy(ids).to("cuda:0")
    acc = torch.zeros((N, h), dtype=torch.bfloat16, device="cuda:0")
    for i in range(t):
        Ei = E[i * v_loc:(i + 1) * v_loc]
        out = T.tp_vocab_embed_fwd(idd, to_dev(Ei), i * v_loc)
        T.tp_vocab_embed_fwd(idd, to_dev(Ei), i * v_loc, out=acc, accumulate=True)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), O.vocab_embed_fwd(ids, Ei, i * v_loc))
    # the sum over ranks equals the full lookup in value (a -0.0 entry of the
    # table plus the other ranks' +0.0 is +0.0, as any summing exchange gives)
    assert np.array_equal(f64(acc), synth.bf16_to_f64(E[ids]))

    dY = synth.bf16_to_f64(synth.int_inputs(90, (N, h))).astype(np.float32)   # exact sums
    dYd = torch.from_numpy(dY).to("cuda:0")
    for i in range(t):
        dE = T.tp_vocab_embed_bwd(idd, dYd, i * v_loc, v_loc)
        torch.cuda.synchronize()
        assert np.array_equal(f64(dE), O.vocab_embed_bwd(ids, dY, i * v_loc, v_loc)), i


def test_table_gradient_calls_in_a_row_and_graph_replays():
    # Rows used by an earlier call (or marked by bits other calls leave in a
    # shared workspace) must come out as exactly what this call's ids give:
    # successive calls into one buffer with different ids and one workspace,
    # a split-K product between them that rewrites that workspace, no tokens
    # at all, then graph replays (captured on a fresh stream) with the ids
    # rewritten in place between replays.
    N, V, h = 512, 4096, 512
    v_loc = V // 2
    rng = np.random.default_rng(77)
    dY = synth.bf16_to_f64(synth.int_inputs(91, (N, h))).astype(np.float32)
    dYd = torch.from_numpy(dY).to("cuda:0")
    dE = torch.full((v_loc, h), 7.0, dtype=torch.float32, device="cuda:0")
    X = to_dev(synth.draw(rng, (16, 2048)))
    W = to_dev(synth.draw(rng, (2048, 384), fan_in=2048))
    need = max(T.workspace_size("tp_vocab_embed_bwd", N, v_loc, h),
               T.workspace_size("tp_col_linear", 16, 2048, 384, 0))
    assert T.workspace_size("tp_col_linear", 16, 2048, 384, 0) > 0   # the product below is split
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    for rnd in range(3):
        ids = rng.integers(0, V, size=N).astype(np.int32)
        ids[:8] = rnd * 97 + np.arange(8)            # rows that move from call to call
        T.tp_vocab_embed_bwd(torch.from_numpy(ids).to("cuda:0"), dYd, 0, v_loc, dE_i=dE, workspace=ws)
        T.tp_col_linear(X, W, "none", workspace=ws)  # a split-K product rewrites the workspace
        torch.cuda.synchronize()
        assert np.array_equal(f64(dE), O.vocab_embed_bwd(ids, dY, 0, v_loc)), rnd
    empty = torch.empty((0,), dtype=torch.int32, device="cuda:0")
    T.tp_vocab_embed_bwd(empty, dYd[:0], 0, v_loc, dE_i=dE, workspace=ws)
    torch.cuda.synchronize()
    assert not torch.any(dE).item()

    idd = torch.from_numpy(rng.integers(0, V, size=N).astype(np.int32)).to("cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        T.tp_vocab_embed_bwd(idd, dYd, 0, v_loc, dE_i=dE)
    torch.cuda.synchronize()
    for rnd in range(3):
        ids = rng.integers(0, V, size=N).astype(np.int32)
        ids[:8] = 1000 + rnd * 13 + np.arange(8)
        idd.copy_(torch.from_numpy(ids))
        dE.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(f64(dE), O.vocab_embed_bwd(ids, dY, 0, v_loc)), ("replay", rnd)
    del graph
