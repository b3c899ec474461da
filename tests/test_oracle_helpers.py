"""Direct pins of the oracle's small helpers (each also reached through the
functions that use them): the SwiGLU gate at points where SiLU has a closed
value, the head-count rules of [TPSP] "注意力：按头切，以及 GQA 的约束" / "GQA：KV
头比 query 头少" on the Llama-3-70B head counts, which KV heads a rank holds
with and without replication, and the multiply-add count of a product
against a brute-force count."""
import math

import numpy as np
import pytest

import oracle as O


def test_swiglu_at_closed_values():
    # SiLU(0) = 0; sigmoid(ln 3) = 3/4, so SiLU(ln 3) = (3/4) ln 3; SiLU(-ln 3) = -(1/4) ln 3
    G = np.array([0.0, math.log(3.0), -math.log(3.0)])
    U = np.array([5.0, 2.0, -4.0])
    want = np.array([0.0, 1.5 * math.log(3.0), math.log(3.0)])
    assert np.allclose(O.swiglu(G, U), want, rtol=1e-15, atol=0)
    # the gate multiplies U: linear in U, zero at U = 0
    assert np.allclose(O.swiglu(G, 2 * U), 2 * O.swiglu(G, U), rtol=1e-15, atol=0)
    assert np.all(O.swiglu(G, np.zeros(3)) == 0.0)
    # large positive gate: SiLU(g) -> g; large negative: -> 0
    assert math.isclose(float(O.swiglu(np.array([40.0]), np.array([3.0]))[0]), 120.0, rel_tol=1e-15)
    assert abs(float(O.swiglu(np.array([-40.0]), np.array([3.0]))[0])) < 1e-15


@pytest.mark.parametrize("n_h,n_kv,t,ok", [
    (64, 8, 8, True),     # Llama-3-70B at t = 8: one KV head per rank
    (64, 8, 4, True),     # two KV heads per rank
    (64, 8, 16, True),    # every KV head on two ranks
    (64, 8, 64, True),    # one query head per rank, each KV head on 8 ranks
    (64, 8, 7, False),    # 7 does not divide the 64 query heads
    (48, 8, 12, False),   # n_kv < t, but 8 does not divide 12: no even replication
    (64, 8, 128, False),  # more ranks than query heads
    (64, 8, 0, False),
])
def test_head_count_rules(n_h, n_kv, t, ok):
    if ok:
        O.check_heads_divisible(n_h, n_kv, t)
    else:
        with pytest.raises(ValueError):
            O.check_heads_divisible(n_h, n_kv, t)


def test_kv_heads_of_rank():
    assert [O.kv_heads_of_rank(8, 8, r) for r in range(8)] == [[r] for r in range(8)]
    assert [O.kv_heads_of_rank(8, 4, r) for r in range(4)] == [[2 * r, 2 * r + 1] for r in range(4)]
    # replicated: ranks 2j and 2j + 1 share KV head j; every head is held
    got = [O.kv_heads_of_rank(8, 16, r) for r in range(16)]
    assert got == [[r // 2] for r in range(16)]
    assert sorted({h for hs in got for h in hs}) == list(range(8))


def test_gemm_flops_counts_multiply_adds():
    M, N, K = 3, 5, 7
    count = sum(2 for _ in range(M) for _ in range(N) for _ in range(K))  # one multiply and one add each
    assert O.gemm_flops(M, N, K) == count == 210
