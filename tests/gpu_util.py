"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import warnings

import numpy as np
import torch

import oracle as O
import synth

# max|gpu - oracle| / max|oracle| per output tensor, bf16 inputs, f32 accumulation
TOL = 2e-2
# The error expected from the bf16 roundings on the path (Z, H, dH stored in
# bf16: 2^-9 relative) is about 1e-3 to 3e-3; a tensor above this still
# passes but is reported as drift, the sign of a regression.
DRIFT = 5e-3


class ParityDriftWarning(UserWarning):
    """An output within tolerance but above the error the bf16 roundings explain."""


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
    """The parity metric, the oracle's rel_err."""
    return O.rel_err(got, want)


def check_errs(errs: dict, label="", tol=TOL):
    """Print the per-tensor errors, warn about drift above DRIFT, assert <= tol."""
    print(label, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        if v > DRIFT and v <= tol:
            warnings.warn(ParityDriftWarning(f"{label} {k}: {v:.2e} above {DRIFT:.0e}"))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (label, bad)


def bf16_ulps(got_bits: np.ndarray, want: np.ndarray) -> int:
    """Largest distance in bf16 units in the last place between GPU bf16 outputs
    and the oracle's values rounded to bf16 (finite values; sign-magnitude
    patterns mapped to a monotone integer line)."""
    w = rne_bf16_bits(want).astype(np.int32)
    g = np.asarray(got_bits).astype(np.int32)

    def line(b):
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)

    return int(np.max(np.abs(line(g) - line(w)))) if g.size else 0


def assert_elementwise(got, want, label, rel=2.0 ** -8, abs_frac=1e-6):
    """|got - want| <= rel |want| + abs_frac max|want| for every element: one
    bf16 rounding (2^-9 relative) plus the f32 evaluation of the activation;
    the absolute part covers tails where f32 flushes what bf16 could hold."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    tol = rel * np.abs(want) + abs_frac * np.max(np.abs(want))
    bad = ~(np.abs(got - want) <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} elements off, first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r}, want {want[tuple(i)]!r}")
