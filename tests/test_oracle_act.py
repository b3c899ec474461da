"""Pins of the oracle's activations: closed forms, limits, textbook values and a
library cross-check (torch CPU, float64)."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def test_gelu_closed_forms():
    x = np.linspace(-6, 6, 241)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    # GeLU(x) - GeLU(-x) = x  (Phi(x) + Phi(-x) = 1)
    assert np.allclose(O.gelu(x) - O.gelu(-x), x, rtol=0, atol=1e-14)
    # GeLU(1) = Phi(1) (standard normal CDF at 1, textbook value)
    assert abs(O.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    # large-|x| limits: x and 0
    assert abs(O.gelu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.gelu(np.array([-40.0]))[0]) < 1e-12


def test_gelu_is_not_the_tanh_approximation():
    x = np.array([1.5])
    tanh_form = 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
    assert abs(O.gelu(x)[0] - tanh_form[0]) > 1e-5


def test_silu_closed_forms():
    x = np.linspace(-30, 30, 601)
    assert O.silu(np.array([0.0]))[0] == 0.0
    # SiLU(x) - SiLU(-x) = x  (sigmoid(x) + sigmoid(-x) = 1)
    assert np.allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-12)
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert np.all(np.isfinite(O.silu(np.array([-1000.0, 1000.0]))))


@pytest.mark.parametrize("fn,tfn", [(O.gelu, torch.nn.functional.gelu),
                                    (O.silu, torch.nn.functional.silu)])
def test_activations_match_torch_fp64(fn, tfn):
    x = np.random.default_rng(0).standard_normal(10000) * 4
    ref = tfn(torch.from_numpy(x)).numpy()
    assert np.allclose(fn(x), ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("fn,grad", [(O.gelu, O.gelu_grad), (O.silu, O.silu_grad)])
def test_activation_gradients(fn, grad):
    x = np.linspace(-8, 8, 161)
    eps = 1e-6
    fd = (fn(x + eps) - fn(x - eps)) / (2 * eps)
    assert np.allclose(grad(x), fd, rtol=1e-7, atol=1e-8)
    # value at 0 is 1/2 for both
    assert abs(grad(np.array([0.0]))[0] - 0.5) < 1e-15


def test_activation_gradients_match_torch_autograd():
    x = torch.from_numpy(np.random.default_rng(1).standard_normal(1000) * 3).requires_grad_()
    for fn, grad, tfn in [(O.gelu, O.gelu_grad, torch.nn.functional.gelu),
                          (O.silu, O.silu_grad, torch.nn.functional.silu)]:
        x.grad = None
        tfn(x).sum().backward()
        assert np.allclose(grad(x.detach().numpy()), x.grad.numpy(), rtol=1e-13, atol=1e-14)
