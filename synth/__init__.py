"""Seeded synthetic inputs for the tensor-parallel shard workloads.

This module only draws random numbers and rounds them to bfloat16. It holds
none of the arithmetic of the method (no products, activations or layouts),
so both the fp64 oracle and the HIP path may consume what it produces.

Recipe (the same for every workload):
  * ``rng = numpy.random.default_rng(seed)``;
  * each tensor is drawn in a fixed order with
    ``rng.standard_normal(shape, dtype=float32)``;
  * weights are multiplied, in fp32, by ``1/sqrt(fan_in)`` where ``fan_in``
    is the width of the *unsharded* contraction (h for the first matrix of
    the MLP and for the QKV / output projections, F for the second MLP
    matrix);
  * the fp32 values are rounded to bfloat16 with round-to-nearest-even.

Tensors are returned as ``uint16`` arrays holding the bfloat16 bit patterns;
``bf16_to_f64`` widens them exactly (every bfloat16 is an fp64).

The shapes are Llama-3-70B's (h=8192, n_h=64, n_kv=8, d_h=128, F=28672) at
TP degree 8, a GPT-style layer (h=4096, F=16384) at TP degree 4, and a tiny
layer for exhaustive checks (the WORKLOADS table below).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import math

import numpy as np

__all__ = [
    "bf16_round", "bf16_to_f64", "bf16_to_f32", "draw", "Workload",
    "WORKLOADS", "mlp_inputs", "qkv_inputs", "mlp_bwd_inputs", "digest",
    "int_inputs",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round-to-nearest-even, NaN kept."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_to_f32(b).astype(np.float64)


def draw(rng: np.random.Generator, shape, fan_in: int | None = None) -> np.ndarray:
    """One N(0,1) fp32 draw, scaled by 1/sqrt(fan_in) in fp32, rounded to bf16."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if fan_in is not None:
        x *= np.float32(1.0 / np.sqrt(fan_in))
    return bf16_round(x)


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


@dataclass(frozen=True)
class Workload:
    """A named workload: shapes, TP degree and seed (no arithmetic)."""
    name: str
    kind: str           # "mlp" | "qkv" | "mlp_bwd" | "vocab_ce"
    seed: int
    N: int              # tokens (b*s)
    h: int
    F: int = 0          # unsharded MLP width
    t: int = 1          # TP degree
    act: str = "gelu"   # "gelu" | "swiglu"
    n_h: int = 0
    n_kv: int = 0
    d_h: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def f(self) -> int:
        return self.F // self.t


WORKLOADS = {
    # tiny GeLU MLP, 4 shards run one after another on one device
    "tiny_gelu_t4": Workload("tiny_gelu_t4", "mlp", 0, N=64, h=256, F=1024, t=4, act="gelu"),
    # GPT-style GeLU MLP, one shard of four
    "gpt_gelu_t4": Workload("gpt_gelu_t4", "mlp", 1, N=8192, h=4096, F=16384, t=4, act="gelu"),
    # Llama-3-70B SwiGLU MLP, one shard of eight
    "llama70b_swiglu_t8": Workload("llama70b_swiglu_t8", "mlp", 2, N=4096, h=8192, F=28672, t=8,
                                   act="swiglu"),
    # Llama-3-70B attention projections, one shard of eight
    "llama70b_qkv_t8": Workload("llama70b_qkv_t8", "qkv", 3, N=4096, h=8192, t=8,
                                n_h=64, n_kv=8, d_h=128),
    # backward of the Llama-3-70B SwiGLU MLP shard
    "llama70b_swiglu_t8_bwd": Workload("llama70b_swiglu_t8_bwd", "mlp_bwd", 4, N=4096, h=8192,
                                       F=28672, t=8, act="swiglu"),
    # Llama-3-70B vocab-parallel LM head, one shard of eight: V = 128256 padded
    # to a multiple of 128 t = 1024 (129024), 16128 vocab ids per rank
    "llama70b_lm_head_t8": Workload("llama70b_lm_head_t8", "vocab_ce", 5, N=4096, h=8192, t=8,
                                    extra={"V": 128256, "V_pad": 129024}),
}


def mlp_inputs(seed: int, N: int, h: int, F: int, t: int, act: str, shard_only: bool = True):
    """Inputs of one MLP shard.

    GeLU: X[N,h], A_i[h,F/t] (fan_in h), B_i[F/t,h] (fan_in F).
    SwiGLU: X[N,h], W_gu[h,2F/t] = [gate | up] drawn as one array (fan_in h),
    W_down[F/t,h] (fan_in F).
    With ``shard_only=False`` (GeLU, used by the tiny t-shard workload) the
    full A[h,F] and B[F,h] are drawn instead and the caller slices shards.
    """
    rng = np.random.default_rng(seed)
    f = F // t
    X = draw(rng, (N, h))
    if act == "gelu":
        if shard_only:
            W_in = draw(rng, (h, f), fan_in=h)
            W_out = draw(rng, (f, h), fan_in=F)
        else:
            W_in = draw(rng, (h, F), fan_in=h)
            W_out = draw(rng, (F, h), fan_in=F)
    elif act == "swiglu":
        W_in = draw(rng, (h, 2 * f), fan_in=h)
        W_out = draw(rng, (f, h), fan_in=F)
    else:
        raise ValueError(act)
    return {"X": X, "W_in": W_in, "W_out": W_out}


def mlp_bwd_inputs(seed: int, N: int, h: int):
    """Upstream gradient dY[N,h] ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    return {"dY": draw(rng, (N, h))}


def qkv_inputs(seed: int, N: int, h: int, n_h: int, n_kv: int, d_h: int, t: int):
    """Attention-projection inputs of one shard.

    X[N,h], the full fused W_qkv[h,(n_h+2n_kv)d_h] (fan_in h), the rank's
    output-projection rows W_O,r[n_h d_h/t, h] (fan_in n_h d_h), a synthetic
    attention output O_r[N, n_h d_h/t] and upstream gradients dQKV[N, width/t],
    dY[N,h], all N(0,1) apart from the weight scaling.
    """
    rng = np.random.default_rng(seed)
    width = (n_h + 2 * n_kv) * d_h
    X = draw(rng, (N, h))
    W_qkv = draw(rng, (h, width), fan_in=h)
    W_O = draw(rng, (n_h * d_h // t, h), fan_in=n_h * d_h)
    O = draw(rng, (N, n_h * d_h // t))
    dQKV = draw(rng, (N, width // t))
    dY = draw(rng, (N, h))
    return {"X": X, "W_qkv": W_qkv, "W_O": W_O, "O": O, "dQKV": dQKV, "dY": dY}


def vocab_ce_inputs(seed: int, N: int, h: int, v_loc: int, V: int):
    """One rank's LM-head inputs: X[N,h] ~ N(0,1), its weight shard
    W_i[h,v_loc] (fan_in h), the token targets (uniform over the V real vocab
    ids, int32; padded ids never occur) and the upstream gradient of each
    token's loss (1/N: the mean loss)."""
    rng = np.random.default_rng(seed)
    X = draw(rng, (N, h))
    W_i = draw(rng, (h, v_loc), fan_in=h)
    targets = rng.integers(0, V, size=N).astype(np.int32)
    dloss = np.full(N, 1.0 / N, dtype=np.float32)
    return {"X": X, "W_i": W_i, "targets": targets, "dloss": dloss}


def int_inputs(seed: int, shape, lo: int = -2, hi: int = 2, scale: float = 1.0) -> np.ndarray:
    """Small integers in [lo, hi], times `scale` (a power of two), as bf16 bit
    patterns (exact in bfloat16)."""
    assert scale > 0 and math.frexp(scale)[0] == 0.5, "scale must be a power of two"
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32) * np.float32(scale)
    return bf16_round(x)


def int_inputs_device(seed: int, shape, device, lo: int = -3, hi: int = 3):
    """Small integers in [lo, hi] as a bf16 torch tensor drawn on `device` by
    torch's seeded generator: inputs of several GiB that a host draw would take
    minutes to produce. Host checks copy the rows or columns they need."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device, dtype=torch.int8)
    return x.to(torch.bfloat16)
