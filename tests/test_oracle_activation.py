"""Pins for the oracle's SiLU-and-mul (SwiGLU) activation."""

from decimal import Decimal, getcontext

import numpy as np
import torch

from oracle import activation as A


def test_silu_vs_torch_float64():
    rng = np.random.default_rng(40)
    g = np.concatenate([rng.standard_normal(100000) * 4, [-700.0, -50.0, -1e-300, 0.0, 1e-300, 50.0, 700.0]])
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    np.testing.assert_allclose(A.silu(g), ref, rtol=1e-15, atol=1e-300)


def test_silu_closed_forms():
    assert A.silu(np.array([0.0]))[0] == 0.0
    g = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(A.silu(g) - A.silu(-g), g, rtol=1e-14, atol=1e-14)  # g(s(g) + s(-g)) = g
    assert A.silu(np.array([60.0]))[0] == 60.0  # sigmoid rounds to 1
    assert abs(A.silu(np.array([-60.0]))[0]) < 1e-24
    assert np.all(np.isfinite(A.silu(np.array([-1e308, 1e308]))))


def test_silu_decimal_reference():
    getcontext().prec = 40
    for g in (-8.5, -3.25, -1.0, -0.125, 0.0078125, 0.5, 2.0, 6.75, 13.0):
        d = Decimal(g)
        exact = d / (1 + (-d).exp())
        got = Decimal(float(A.silu(np.array([g]))[0]))
        assert abs(got - exact) <= abs(exact) * Decimal("1e-15") + Decimal("1e-300"), g


def test_silu_mul_rows_halves():
    rng = np.random.default_rng(41)
    d = 96
    x = rng.standard_normal((5, 2 * d))
    y = A.silu_mul_rows(x, d)
    for r in range(5):
        for i in range(0, d, 7):
            g, u = x[r, i], x[r, d + i]
            assert y[r, i] == A.silu(np.array([g]))[0] * u
    # the gate and up halves are not interchangeable
    assert not np.allclose(A.silu_mul_rows(np.concatenate([x[:, d:], x[:, :d]], axis=1), d), y)
