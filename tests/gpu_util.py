"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch

import synth

# max|gpu - oracle| / max|oracle| per output tensor, bf16 inputs, f32 accumulation
TOL = 2e-2


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> a bf16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def f64(t: torch.Tensor) -> np.ndarray:
    """A GPU tensor (bf16 or f32) -> float64 numpy (exact widening)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)


def rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values (exact in f32) to bf16 bit patterns, nearest even."""
    return synth.bf16_round(np.asarray(x, dtype=np.float32))


def err(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.max(np.abs(want)) if want.size else 0.0
    return float(np.max(np.abs(got - want)) / den) if den > 0 else float(np.max(np.abs(got - want)))
