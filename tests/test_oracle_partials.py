"""Pins of the oracle's partial-input sum (``exact_sum``, ``rmsnorm_rows_partials``).

The reference values come from outside the oracle: exact rational arithmetic
(``fractions.Fraction``) with an independent round-to-nearest-even written
over rationals, IEEE signed-zero rules, torch's float32 sum where the recipe
makes it exact, and the single-input oracle (already pinned) for one partial.
The mutants at the end plant plausible slips in CPU copies of ``exact_sum``;
each must fail one of the checks.
"""

from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import rownorm as O


# ---------------------------------------------------------------------------
# Independent references over the rationals.
# ---------------------------------------------------------------------------

def rne_rational(q: Fraction, precision: int, emin: int) -> Fraction:
    """Round a rational to a binary format with ``precision`` significant bits and
    minimum normal exponent ``emin`` (no overflow handling), ties to even."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - precision + 1)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def exact(terms) -> Fraction:
    return sum((Fraction(float(t)) for t in terms), Fraction(0))


def _random_terms(rng, k):
    """Doubles of mixed magnitude: f32 values, bf16 values and full doubles,
    exponents over about +-60 binades, some exact cancellations."""
    out = []
    for _ in range(k):
        kind = rng.integers(4)
        mag = math.ldexp(1.0, int(rng.integers(-60, 60)))
        v = float(rng.standard_normal()) * mag
        if kind == 0:
            v = float(np.float32(v))
        elif kind == 1:
            v = float(O.bf16_decode(O.bf16_encode(np.array([v])))[0])
        elif kind == 2 and out:
            v = -out[int(rng.integers(len(out)))]
        out.append(v)
    return out


# ---------------------------------------------------------------------------
# Checks (each takes an exact_sum implementation, so mutants can be run).
# ---------------------------------------------------------------------------

def check_matches_rational_sum(exact_sum):
    rng = np.random.default_rng(11)
    for _ in range(400):
        k = int(rng.integers(1, 10))
        cols = [_random_terms(rng, k) for _ in range(3)]
        terms = [np.array([c[i] for c in cols]) for i in range(k)]
        s, e = exact_sum(terms)
        for j in range(3):
            q = exact([t[j] for t in terms])
            assert Fraction(float(s[j])) == Fraction(float(q)), (cols[j], s[j], float(q))
            assert float(e[j]) == float(q - Fraction(float(s[j])))


def check_remainder_decides_ties(exact_sum):
    one = 1.0
    cases = [  # (terms, format, expected single rounding of the exact sum)
        ([one, 2.0 ** -8], O.BF16, one),                               # exact tie -> even
        ([one, 2.0 ** -8, 2.0 ** -60], O.BF16, one + 2.0 ** -7),       # just above the tie
        ([one, 2.0 ** -8, -2.0 ** -60], O.BF16, one),                  # just below
        ([one, 2.0 ** -24, 2.0 ** -80], O.F32, one + 2.0 ** -23),      # f32 tie broken below double
        ([one + 2.0 ** -7, 2.0 ** -8], O.BF16, one + 2.0 ** -6),       # tie from an odd neighbour -> up
        ([2.0 ** 40, 1.0, -2.0 ** 40, 2.0 ** -70], O.F32, 1.0),
    ]
    for terms, fmt, expected in cases:
        s, e = exact_sum([np.array([t]) for t in terms])
        got = float(O.round_to_format(s, fmt, e)[0])
        ref = float(rne_rational(exact(terms), fmt.precision, fmt.emin))
        assert ref == expected
        assert got == expected, (terms, got, expected)


def check_rounded_sums_match_rational_rne(exact_sum):
    """Random sums rounded once to bf16 and f32, many near a tie."""
    rng = np.random.default_rng(5)
    for fmt in (O.BF16, O.F32):
        for _ in range(300):
            base = float(O.round_to_format(np.array([rng.standard_normal()]), fmt)[0])
            if base == 0.0:
                continue
            ulp = math.ldexp(1.0, math.frexp(abs(base))[1] - fmt.precision)
            terms = [base, ulp / 2 * float(rng.choice([-1, 1])),
                     math.ldexp(float(rng.standard_normal()), -90), -base / 3, base / 3]
            s, e = exact_sum([np.array([t]) for t in terms])
            got = float(O.round_to_format(s, fmt, e)[0])
            assert got == float(rne_rational(exact(terms), fmt.precision, fmt.emin)), terms


def check_signed_zeros(exact_sum):
    cases = [([-0.0, -0.0], True), ([-0.0], True), ([-0.0, 0.0], False), ([1.5, -1.5], False),
             ([0.0, -0.0, -0.0], False)]
    for terms, negative in cases:
        s, _ = exact_sum([np.array([t]) for t in terms])
        assert float(s[0]) == 0.0 and bool(np.signbit(s[0])) == negative, terms


def check_order_independent(exact_sum):
    rng = np.random.default_rng(3)
    for _ in range(50):
        k = int(rng.integers(2, 6))
        terms = [np.array(_random_terms(rng, 4)) for _ in range(k)]
        ref = exact_sum(terms)
        for perm in itertools.islice(itertools.permutations(range(k)), 6):
            s, e = exact_sum([terms[i] for i in perm])
            assert np.array_equal(s, ref[0]) and np.array_equal(e, ref[1])


ALL_CHECKS = [check_matches_rational_sum, check_remainder_decides_ties, check_rounded_sums_match_rational_rne,
              check_signed_zeros, check_order_independent]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_exact_sum(check):
    check(O.exact_sum)


# ---------------------------------------------------------------------------
# The workload recipe and the norm over the sum.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_exact_sum_recipe_makes_float32_sums_exact(x_dtype):
    """Under the exact-sum recipe every nonzero term lies in [2^-7, 2^5), every float32
    prefix sum in slot order is exact, and torch's float32 sum equals the oracle's."""
    wl = W.PartialsWorkload(name="t", rows=16, hidden=1024, num_partials=8, x_dtype=x_dtype, res_dtype=None,
                            w_dtype="bf16", out_dtype="bf16", part_dist=W.Dist(0.0, 0.5), res_dist=None,
                            w_dist=W.Dist(1.0, 0.1), weight_plus_one=False, eps=1e-6, exact_sum=True)
    inp = W.generate_partials(wl, seed=4)
    vals = [O.decode(p, x_dtype) for p in inp["partials"]]
    nz = np.abs(np.concatenate([v[v != 0] for v in vals]))
    assert nz.min() >= 2.0 ** -7 and nz.max() < 2.0 ** 5
    acc = torch.zeros(16, 1024, dtype=torch.float32)
    for v in vals:
        acc = acc + torch.from_numpy(v.astype(np.float32))
    s, e = O.exact_sum(vals)
    assert np.array_equal(acc.numpy().astype(np.float64), s) and not e.any()
    prefix = np.zeros_like(vals[0])
    for v in vals:
        prefix = prefix + v
        assert np.array_equal(prefix.astype(np.float32).astype(np.float64), prefix)


@pytest.mark.parametrize("res_dtype", ["f32", "bf16"])
def test_one_partial_is_the_single_input_oracle(res_dtype):
    rng = np.random.default_rng(9)
    x = O.decode(O.bf16_encode(rng.standard_normal((5, 256))), "bf16")
    r = rng.standard_normal((5, 256))
    r = O.decode(O.encode(r, res_dtype), res_dtype)
    w = 1.0 + 0.1 * rng.standard_normal(256)
    a = O.rmsnorm_rows_partials([x], w, 1e-6, 0.0, residual=r, res_dtype=res_dtype)
    b = O.rmsnorm_rows(x, w, 1e-6, 0.0, residual=r, res_dtype=res_dtype)
    for key in ("h", "inv", "y"):
        assert np.array_equal(a[key], b[key])


def test_partials_with_residual_round_the_rational_sum_once():
    rng = np.random.default_rng(21)
    parts = [O.decode(O.bf16_encode(rng.standard_normal((3, 64)) * 2.0 ** rng.integers(-30, 30)), "bf16")
             for _ in range(5)]
    res = rng.standard_normal((3, 64)).astype(np.float32).astype(np.float64)
    out = O.rmsnorm_rows_partials(parts, np.ones(64), 1e-6, 1.0, residual=res, res_dtype="bf16")
    for i in range(3):
        for j in range(64):
            q = exact([p[i, j] for p in parts] + [res[i, j]])
            assert out["h"][i, j] == float(rne_rational(q, O.BF16.precision, O.BF16.emin))
    ref = O.rmsnorm_rows(out["h"], np.ones(64), 1e-6, 1.0)
    assert np.array_equal(out["y"], ref["y"])


def test_partials_without_residual_normalize_the_exact_sum():
    parts = [np.array([[3.0, 0.0]]), np.array([[2.0 ** -60, 4.0]]), np.array([[-2.0 ** -60, 0.0]])]
    out = O.rmsnorm_rows_partials(parts, np.ones(2), 0.0, 0.0)
    # the row (3, 4): rms = sqrt(25 / 2)
    assert np.allclose(out["y"], np.array([[3.0, 4.0]]) / math.sqrt(12.5), rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# Mutants: plausible slips in exact_sum, each caught by some check.
# ---------------------------------------------------------------------------

def _naive_double(terms):
    s = np.zeros_like(np.asarray(terms[0], dtype=np.float64))
    for t in terms:
        s = s + t
    return s, np.zeros_like(s)


def _no_remainder(terms):
    s, _ = O.exact_sum(terms)
    return s, np.zeros_like(s)


def _negated_remainder(terms):
    s, e = O.exact_sum(terms)
    return s, -e


def _drop_last(terms):
    return O.exact_sum(terms[:-1]) if len(terms) > 1 else O.exact_sum(terms)


def _float32_accumulate(terms):
    s = np.zeros_like(np.asarray(terms[0], dtype=np.float32))
    for t in terms:
        s = (s + np.asarray(t, dtype=np.float32)).astype(np.float32)
    return s.astype(np.float64), np.zeros(s.shape)


def _fsum_signs_lost(terms):
    s, e = O.exact_sum(terms)
    return np.where(s == 0, 0.0, s), e


MUTANTS = {"naive_double": _naive_double, "no_remainder": _no_remainder, "negated_remainder": _negated_remainder,
           "drop_last": _drop_last, "float32_accumulate": _float32_accumulate, "signs_lost": _fsum_signs_lost}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    impl = MUTANTS[name]
    caught = None
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, OverflowError):
            caught = check.__name__
            break
    assert caught is not None, f"mutant {name} passed every check"
