"""The seeded input generators: determinism and bfloat16 rounding."""
import numpy as np
import torch

import synth


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 37,
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38, -3.0e38, 1e-40, np.inf, -np.inf],
                                 dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_round(x), ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert synth.bf16_round(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80
    assert synth.bf16_round(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82
    assert np.isnan(synth.bf16_to_f32(synth.bf16_round(np.array([np.nan], np.float32))))[0]


def test_widening_is_exact():
    b = np.arange(0, 65536, 7, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen with an FP flag
        f = synth.bf16_to_f64(b)
    finite = np.isfinite(f)
    assert np.array_equal(synth.bf16_round(f[finite].astype(np.float32)), b[finite])


def test_generators_are_deterministic():
    a = synth.mlp_inputs(2, 16, 64, 256, 8, "swiglu")
    b = synth.mlp_inputs(2, 16, 64, 256, 8, "swiglu")
    for k in a:
        assert synth.digest(a[k]) == synth.digest(b[k])
    assert a["W_in"].shape == (64, 64) and a["W_out"].shape == (32, 64)
    c = synth.mlp_inputs(3, 16, 64, 256, 8, "swiglu")
    assert synth.digest(a["X"]) != synth.digest(c["X"])


def test_weight_scaling_uses_unsharded_fan_in():
    d = synth.mlp_inputs(5, 8, 1024, 4096, 4, "gelu")
    w_in = synth.bf16_to_f64(d["W_in"])
    w_out = synth.bf16_to_f64(d["W_out"])
    assert abs(w_in.std() - 1 / np.sqrt(1024)) < 2e-3 / np.sqrt(1024) * 10
    assert abs(w_out.std() - 1 / np.sqrt(4096)) < 2e-3 / np.sqrt(4096) * 10


def test_int_inputs_are_exact_small_integers():
    v = synth.bf16_to_f64(synth.int_inputs(0, (100, 100)))
    assert set(np.unique(v)) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
