"""fp64 CPU oracle for one GPU's share of a tensor-parallel layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package. The product (the HIP library and
its Python binding) never imports, links or calls it, and it never imports the
product. The two share nothing but the seeded input generators in ``synth``.

Everything here is the plain mathematical definition of what a tensor-parallel
shard computes, in numpy float64, on the same bfloat16-rounded inputs the GPU
receives (widened exactly), with no intermediate rounding. A library matmul
(``numpy.matmul``, OpenBLAS dgemm) is used as a step; there is no blocking,
fusion or reordering beyond the definitions.

Sources (pages, by title and section):
  [TPSP]    hs-black, "张量并行与序列并行" (scaling-tensor-parallel):
            "矩阵乘法的两种切法" (the two block-matmul identities and their
            backward), "MLP：先列后行，只通信一次" (GeLU and SwiGLU MLPs),
            "注意力：按头切，以及 GQA 的约束" (head-aligned split, fused-QKV
            layout), "GQA：KV 头比 query 头少", "精确的通信量" (FLOP count).
  [REVISIT] pufanyi, "ml-revisit-infra", section "Tensor Parallel" (column-wise
            and row-wise identities with their gradients; head-count check).
  [SB6]     r00kie-liu, "Scaling Book 入门第 6 章：分片矩阵乘法", §6.1
            "什么是分片" (sharding notation and its Pop Quiz).

Pins: every function is checked in ``tests/test_oracle_*.py`` against values
the pages print, closed forms, finite differences and brute force; none is
"parity unpinned".
"""
from .tp_oracle import *  # noqa: F401,F403
from .tp_oracle import __all__  # noqa: F401
