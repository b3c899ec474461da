"""Vocab-parallel LM head with fused cross-entropy through the C ABI against the
fp64 oracle: each rank's local statistics, the single-device exchange
(tp_vocab_ce_combine) giving the loss, and the backward (dZ, dX_part summed
over ranks with accumulate, dW_i); small shapes with ragged vocab tiles, a
2^20-column shard, then Llama-3-70B's shard at full size, every element."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_util import TOL, check_errs, err, f64, to_dev
import tensor_sharded_matmul_amd as T

pytestmark = pytest.mark.gpu


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


@pytest.mark.parametrize("N,h,v_loc,t", [(300, 512, 1344, 4), (77, 256, 1280, 3), (16, 1024, 448, 2)])
def test_vocab_ce_forward_backward_small(N, h, v_loc, t):
    V = v_loc * t
    rng = np.random.default_rng(N + v_loc)
    X = synth.draw(rng, (N, h))
    Ws = [synth.draw(rng, (h, v_loc), fan_in=h) for _ in range(t)]
    # a few logits well above the rest, so that the max is not flat
    y = rng.integers(0, V, size=N).astype(np.int32)
    y[:4] = [0, v_loc - 1, v_loc, V - 1][:4]          # shard edges
    X64, W64 = synth.bf16_to_f64(X), [synth.bf16_to_f64(W) for W in Ws]
    Xd, Wd, yd = to_dev(X), [to_dev(W) for W in Ws], _dev_i32(y)

    stats = [T.tp_vocab_ce_fwd(Xd, Wd[i], yd, i * v_loc) for i in range(t)]
    torch.cuda.synchronize()
    for i in range(t):
        m_i, s_i, zy_i = O.vocab_ce_local(X64, W64[i], y, i * v_loc)
        assert err(f64(stats[i][0]), m_i) <= TOL, ("m", i)
        assert err(f64(stats[i][1]), s_i) <= TOL, ("s", i)
        assert err(f64(stats[i][2]), zy_i) <= TOL, ("zy", i)
        # z_y is zero exactly where the target is on another rank
        inside = (y >= i * v_loc) & (y < (i + 1) * v_loc)
        assert np.all(f64(stats[i][2])[~inside] == 0.0)

    loss, m, S = T.tp_vocab_ce_combine(*(torch.stack([st[k] for st in stats]) for k in range(3)))
    torch.cuda.synchronize()
    want_loss, want_m, want_S = O.vocab_ce_loss(X64, W64, y)
    assert err(f64(loss), want_loss) <= TOL
    assert err(f64(m), want_m) <= TOL and err(f64(S), want_S) <= TOL

    dloss = np.linspace(0.5, 1.5, N).astype(np.float32)
    dld = _dev_f32(dloss)
    dX = torch.zeros((N, h), dtype=torch.float32, device="cuda:0")
    for i in range(t):
        dZ, _, dW = T.tp_vocab_ce_bwd(Xd, Wd[i], yd, i * v_loc, m, S, dld, dX_part=dX, accumulate=True)
        torch.cuda.synchronize()
        wz, _, ww = O.vocab_ce_bwd(X64, W64[i], y, i * v_loc, want_m, want_S, dloss)
        assert err(f64(dZ), wz) <= TOL, ("dZ", i)
        assert err(f64(dW), ww) <= TOL, ("dW", i)
    want_dx = sum(O.vocab_ce_bwd(X64, W64[i], y, i * v_loc, want_m, want_S, dloss)[1] for i in range(t))
    assert err(f64(dX), want_dx) <= TOL


def test_vocab_ce_forward_wide_weight_window():
    # a vocabulary shard so wide that the weight's window ((h + 512) rows of
    # its pitch) reaches 2^31 bytes: the statistics GEMM then runs 256 x 224
    # tiles with the WIDE descriptor walk (one record per 112 columns). The
    # widest shard the library takes (2^20 columns) over h = 512.
    N, h, v_loc = 16, 512, 1 << 20
    assert (h + 512) * v_loc * 2 >= 1 << 31
    assert T.workspace_size("tp_vocab_ce_fwd", N, h, v_loc) == N * 2 * -(-v_loc // 224) * 12
    rng = np.random.default_rng(4242)
    X = synth.draw(rng, (N, h))
    W = synth.draw(rng, (h, v_loc), fan_in=h)
    y = rng.integers(0, v_loc, size=N).astype(np.int32)
    y[:3] = [0, v_loc - 1, v_loc // 2]
    print(f"ce wide window: N={N} h={h} v_loc={v_loc}", flush=True)
    m_i, s_i, zy_i = T.tp_vocab_ce_fwd(to_dev(X), to_dev(W), _dev_i32(y), 0)
    torch.cuda.synchronize()
    wm, ws, wz = O.vocab_ce_local(synth.bf16_to_f64(X), synth.bf16_to_f64(W), y, 0)
    assert err(f64(m_i), wm) <= TOL and err(f64(s_i), ws) <= TOL and err(f64(zy_i), wz) <= TOL


def test_llama70b_lm_head_shard_full_size():
    # every element of every output at Llama-3-70B's shard size (4096 tokens,
    # h = 8192, 16128 vocab columns): the fp64 oracle takes a few seconds
    w = synth.WORKLOADS["llama70b_lm_head_t8"]
    v_loc = w.extra["V_pad"] // w.t
    d = synth.vocab_ce_inputs(w.seed, w.N, w.h, v_loc, w.extra["V"])
    rank = 0
    Xd, Wd, yd = to_dev(d["X"]), to_dev(d["W_i"]), _dev_i32(d["targets"])
    m_i, s_i, zy_i = T.tp_vocab_ce_fwd(Xd, Wd, yd, rank * v_loc)
    torch.cuda.synchronize()
    X64, W64 = synth.bf16_to_f64(d["X"]), synth.bf16_to_f64(d["W_i"])
    want = O.vocab_ce_local(X64, W64, d["targets"], rank * v_loc)
    errs = {name: err(f64(got), wnt) for got, wnt, name in zip((m_i, s_i, zy_i), want, ("m", "s", "zy"))}
    # backward with this rank's statistics standing for the global ones (t = 1)
    loss, m, S = T.tp_vocab_ce_combine(m_i[None], s_i[None], zy_i[None])
    dld = _dev_f32(d["dloss"])
    dZ, dX, dW = T.tp_vocab_ce_bwd(Xd, Wd, yd, rank * v_loc, m, S, dld)
    torch.cuda.synchronize()
    wz, wx, ww = O.vocab_ce_bwd(X64, W64, d["targets"], rank * v_loc, f64(m), f64(S), d["dloss"])
    errs.update({"dZ": err(f64(dZ), wz), "dX": err(f64(dX), wx), "dW": err(f64(dW), ww)})
    check_errs(errs, "Llama-3-70B LM head shard")
