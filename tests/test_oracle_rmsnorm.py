"""Pins for the oracle's RMSNorm rows and per-head QK-norm.

Every check here compares ``oracle.rmsnorm_rows`` / ``oracle.qknorm`` with
something other than itself: hand-derived closed forms (tests/golden/),
exact rational arithmetic, invariants of the definition, or torch's float64
``rms_norm`` as an independent library routine.  The ``check_*`` helpers
take the implementation as an argument so that tests/test_oracle_mutations.py
can run the same pins against deliberately broken copies of the oracle and
show that each plausible mistake is caught.
"""

import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import rownorm as O


# ---------------------------------------------------------------------------
# checks, parameterized by the implementation under test
# ---------------------------------------------------------------------------

def load_closed_forms(golden_dir):
    cases = []
    with open(os.path.join(golden_dir, "rmsnorm_closed_forms.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, ws, ys = line.split("|")
            parts = head.split()
            name, H, b, eps = parts[0], int(parts[1]), float(parts[2]), float(parts[3])
            x = [float(t) for t in parts[4:]]
            w = [float(t) for t in ws.split()]
            y = [float(t) for t in ys.split()]
            assert len(x) == len(w) == len(y) == H, name
            cases.append((name, H, b, eps, np.array([x]), np.array(w), np.array([y])))
    return cases


def check_closed_forms(impl, golden_dir):
    for name, H, b, eps, x, w, y in load_closed_forms(golden_dir):
        got = impl(x, w, eps, b)["y"]
        np.testing.assert_allclose(got, y, rtol=1e-15, atol=0, err_msg=name)


def check_constant_rows(impl):
    rng = np.random.default_rng(10)
    for H in (1, 7, 64, 1000):
        for b in (0.0, 1.0):
            c = rng.standard_normal()
            eps = float(np.float32(10.0 ** rng.uniform(-7, -1)))
            w = rng.standard_normal(H)
            x = np.full((1, H), c)
            got = impl(x, w, eps, b)["y"][0]
            expect = (w + b) * c / math.sqrt(c * c + eps)
            np.testing.assert_allclose(got, expect, rtol=1e-14, atol=0)


def check_zero_row(impl):
    for b in (0.0, 1.0):
        got = impl(np.zeros((2, 16)), np.linspace(-1, 1, 16), 1e-6, b)["y"]
        assert np.all(got == 0)


def check_unit_weight_rms(impl):
    rng = np.random.default_rng(11)
    for eps in (0.0, float(np.float32(1e-6)), 0.5):
        x = rng.standard_normal((8, 333)) * 3
        y = impl(x, np.ones(333), eps, 0.0)["y"]
        ms = np.mean(x * x, axis=1)
        rms_y = np.sqrt(np.mean(y * y, axis=1))
        np.testing.assert_allclose(rms_y, np.sqrt(ms / (ms + eps)), rtol=1e-14)


def check_scale_invariance(impl):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 96))
    w = rng.standard_normal(96)
    y0 = impl(x, w, 0.0, 0.0)["y"]
    for k in (-20, -3, 5, 30):
        yk = impl(x * 2.0 ** k, w, 0.0, 0.0)["y"]
        assert np.array_equal(yk, y0), k


def check_brute_force_rational(impl):
    """Tiny bf16 rows: exact rational sum of squares, 50-digit decimal sqrt."""
    getcontext().prec = 50
    rng = np.random.default_rng(13)
    for H in (1, 2, 3, 5, 8, 13, 16):
        for _ in range(20):
            bits = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(torch.bfloat16)
            x = bits.to(torch.float64).numpy()
            w = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(torch.bfloat16)
            w = w.to(torch.float64).numpy()
            b = float(rng.integers(0, 2))
            eps = float(np.float32(1e-5))
            got = impl(x[None, :], w, eps, b)["y"][0]
            ss = sum(Fraction(v) * Fraction(v) for v in x)
            ms = ss / H + Fraction(eps)
            root = Decimal(ms.numerator).sqrt() / Decimal(ms.denominator).sqrt()
            for i in range(H):
                exact = (Decimal(Fraction(w[i]).numerator) / Decimal(Fraction(w[i]).denominator) + Decimal(b)) \
                    * (Decimal(Fraction(x[i]).numerator) / Decimal(Fraction(x[i]).denominator)) / root
                assert abs(Decimal(got[i]) - exact) <= abs(exact) * Decimal("1e-15") + Decimal("1e-300")


def check_torch_rms_norm(impl):
    """torch.nn.functional.rms_norm in float64 computes the same definition."""
    rng = np.random.default_rng(14)
    for H in (8, 128, 1000, 4096):
        x = rng.standard_normal((16, H)) * rng.uniform(0.1, 10)
        w = rng.standard_normal(H)
        for b in (0.0, 1.0):
            eps = float(np.float32(1e-6))
            got = impl(x, w, eps, b)["y"]
            ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (H,), weight=torch.from_numpy(w + b),
                                               eps=eps).numpy()
            np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-300)


def check_weight_bias_equivalence(impl):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((5, 256))
    w = torch.from_numpy((rng.standard_normal(256) * 0.02).astype(np.float32)).to(torch.bfloat16)
    w = w.to(torch.float64).numpy()
    a = impl(x, w, 1e-5, 1.0)["y"]
    b = impl(x, w + 1.0, 1e-5, 0.0)["y"]  # w + 1 is exact for bf16 w of this size
    assert np.array_equal(a, b)


def check_residual_cases(impl):
    rng = np.random.default_rng(16)
    xb = torch.from_numpy(rng.standard_normal((6, 512)).astype(np.float32)).to(torch.bfloat16)
    rb = torch.from_numpy(rng.standard_normal((6, 512)).astype(np.float32)).to(torch.bfloat16)
    x = xb.to(torch.float64).numpy()
    r = rb.to(torch.float64).numpy()
    w = rng.standard_normal(512)
    plain = impl(x, w, 1e-6, 0.0)
    zero_res = impl(x, w, 1e-6, 0.0, residual=np.zeros_like(x), res_dtype="bf16")
    assert np.array_equal(zero_res["h"], x)
    assert np.array_equal(zero_res["y"], plain["y"])
    swapped = impl(r, w, 1e-6, 0.0, residual=x, res_dtype="bf16")
    direct = impl(x, w, 1e-6, 0.0, residual=r, res_dtype="bf16")
    assert np.array_equal(swapped["h"], direct["h"])
    assert np.array_equal(swapped["y"], direct["y"])
    # the norm is taken over the rounded residual: out == RMSNorm(res_out)
    again = impl(direct["h"], w, 1e-6, 0.0)
    assert np.array_equal(again["y"], direct["y"])
    # the updated residual is the once-rounded sum (torch bf16 add rounds once, see codec pins)
    ref_h = (xb + rb).to(torch.float64).numpy()
    assert np.array_equal(direct["h"], ref_h)


def check_eps_is_float32(impl):
    # the library receives eps as a C float: 1e-6 is used as float32(1e-6)
    x = np.full((1, 4), 1e-3)
    y = impl(x, np.ones(4), 1e-6, 0.0)["y"][0, 0]
    e32 = float(np.float32(1e-6))
    assert y == pytest.approx(1e-3 / math.sqrt(1e-6 + e32), rel=1e-15)
    assert abs(y - 1e-3 / math.sqrt(1e-6 + 1e-6)) > 1e-15


ALL_CHECKS = [
    check_closed_forms, check_constant_rows, check_zero_row, check_unit_weight_rms,
    check_scale_invariance, check_brute_force_rational, check_torch_rms_norm,
    check_weight_bias_equivalence, check_residual_cases, check_eps_is_float32,
]


# ---------------------------------------------------------------------------
# the oracle itself must pass every check
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check, golden_dir):
    if check is check_closed_forms:
        check(O.rmsnorm_rows, golden_dir)
    else:
        check(O.rmsnorm_rows)


def test_qknorm_matches_head_loop():
    """Every (token, head) pair is its own row; Q rows use q_weight, K rows k_weight."""
    rng = np.random.default_rng(17)
    T, nq, nk, D = 5, 3, 2, 64
    q = rng.standard_normal((T, nq, D))
    k = rng.standard_normal((T, nk, D)) * 3
    qw, kw = rng.standard_normal(D), rng.standard_normal(D)
    eps = float(np.float32(1e-6))
    qy, ky = O.qknorm(q, k, qw, kw, eps, 1.0)
    for t in range(T):
        for hh in range(nq + nk):  # the page's order: heads of Q first, then heads of K
            src, w, dst, j = (q, qw, qy, hh) if hh < nq else (k, kw, ky, hh - nq)
            row = src[t, j]
            ms = sum(float(v) * float(v) for v in row) / D
            expect = [(w[i] + 1.0) * row[i] / math.sqrt(ms + eps) for i in range(D)]
            np.testing.assert_allclose(dst[t, j], expect, rtol=1e-14)
    qy2, ky2 = O.qknorm(q, None, qw, None, eps, 1.0)
    assert ky2 is None and np.array_equal(qy2, qy)
