"""Pins for the oracle's fused-epilogue reference (oracle.activation,
oracle.epilogue): torch's own float64 SiLU and tanh-GELU (library routines),
ReLU and the odd-part identities act(x) - act(-x) = x of SiLU and tanh-GELU
(closed forms), zero at zero, the bias added exactly, and the slope bound
the parity tolerance uses.  The fused epilogue is the roadmap item "GEMM
尾部融合" of "PyTorch 接上 FlyDSL" (5ulink.com, closing paragraph)."""
import numpy as np
import pytest
import torch

import oracle

X = np.concatenate([np.linspace(-30, 30, 60001), [0.0, -0.0, 1e-30, -1e-30, 700.0, -700.0]])


def test_silu_matches_torch():
    ref = torch.nn.functional.silu(torch.tensor(X, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(oracle.activation(oracle.ACT_SILU, X), ref, rtol=1e-14, atol=1e-300)


def test_gelu_tanh_matches_torch():
    ref = torch.nn.functional.gelu(torch.tensor(X, dtype=torch.float64), approximate="tanh").numpy()
    # far left both are cancellations near 0 (1 + tanh -> 0): absolute 1e-15 there
    np.testing.assert_allclose(oracle.activation(oracle.ACT_GELU_TANH, X), ref, rtol=1e-13, atol=1e-15)


def test_relu_closed_form():
    y = oracle.activation(oracle.ACT_RELU, X)
    assert np.array_equal(y, np.where(X > 0, X, 0.0))
    assert np.array_equal(oracle.activation(oracle.ACT_NONE, X), X)


@pytest.mark.parametrize("act", [oracle.ACT_SILU, oracle.ACT_GELU_TANH])
def test_odd_part_identity_and_zero(act):
    x = np.linspace(-8, 8, 1601)
    d = oracle.activation(act, x) - oracle.activation(act, -x)
    np.testing.assert_allclose(d, x, rtol=0, atol=1e-14)
    assert oracle.activation(act, np.array([0.0]))[0] == 0.0


def test_bias_is_added_exactly():
    rng = np.random.default_rng(1)
    c = rng.integers(-1000, 1000, size=(7, 16)).astype(np.float64) / 8
    bias = torch.tensor(rng.integers(-64, 64, size=16) / 4.0, dtype=torch.float32).to(torch.bfloat16)
    bits = bias.view(torch.int16).numpy().view(np.uint16)
    y, slope = oracle.epilogue(c, bits, oracle.ACT_NONE)
    assert np.array_equal(y, c + bias.double().numpy()[None, :])
    assert np.all(slope == 1.0)


@pytest.mark.parametrize("act", [oracle.ACT_RELU, oracle.ACT_SILU, oracle.ACT_GELU_TANH])
def test_slope_bound_holds(act):
    x = np.linspace(-20, 20, 400001)
    h = 1e-5
    fd = np.abs(oracle.activation(act, x + h) - oracle.activation(act, x - h)) / (2 * h)
    _, slope = oracle.epilogue(x[None, :], None, act)
    away = np.abs(x) > h          # ReLU's kink: the difference quotient straddles it
    assert np.all(fd[away] <= slope[0][away] + 1e-6)
