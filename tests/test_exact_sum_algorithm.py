"""The partial-input kernels' summation algorithm, replayed on the CPU.

The kernels sum their terms (the partials and the residual) with float32
TwoSum additions, keep the rounding errors in a double, and round the result
once through round-to-odd (see ``csrc/device_common.h``).  This file restates
those steps in numpy's IEEE float32 / float64 arithmetic, operation for
operation, and checks them against the oracle's exact sum rounded once
(``oracle.rownorm.exact_sum`` + ``round_to_format``) on random terms across
wide magnitude spans and on hand-made rounding hazards.  It pins the
algorithm and its stated range on far more inputs than the GPU tests run;
the GPU tests check the kernels themselves against the oracle.
"""

import numpy as np
import pytest

from oracle import rownorm as O

f32, f64 = np.float32, np.float64


def _two_sum_err(a, b, t):
    bv = t - a
    return (a - (t - bv)) + (b - bv)


def _step(bits, step, away):
    return bits + np.where(step, np.where(away, 1, -1), 0)


def replay(terms, odd=False, wave_fast_path=True):
    """The kernels' sum of float32 terms, rounded once to float32 (nearest
    even), or to odd at float32 precision when ``odd`` (for bf16 targets).

    Every term but the last goes through float32 TwoSum with the error added
    to a double; the last term is added in float32, and where no earlier
    addition rounded, that sum (made odd with its own error for ``odd``) is
    the result.  Elsewhere the double path: a double TwoSum of the float32
    sum and all the errors, round-to-odd at double precision, then float32
    (and round-to-odd at float32 for ``odd``).  ``wave_fast_path=False``
    takes the double path for every element (the kernels take it for a whole
    wave when any of its lanes needs it); both give the same bits.
    """
    with np.errstate(over="ignore", invalid="ignore"):
        s = np.asarray(terms[0], dtype=f32).copy()
        c = np.zeros(s.shape, dtype=f64)
        for v in terms[1:-1]:
            v = np.asarray(v, dtype=f32)
            t = s + v
            c = c + _two_sum_err(s, v, t).astype(f64)
            s = t
        v = np.asarray(terms[-1], dtype=f32)
        t = s + v
        e = _two_sum_err(s, v, t)
        # fast path (no earlier rounding)
        fast = t.copy()
        if odd:
            tb = fast.view(np.uint32).astype(np.int64)
            fast = _step(tb, (e != 0) & ((tb & 1) == 0), (e > 0) == (t > 0)).astype(np.uint32).view(f32)
        # double path
        cc = c + e.astype(f64)
        sd = t.astype(f64)
        u = sd + cc
        r = _two_sum_err(sd, cc, u)
        u = np.where(cc == 0, sd, u)
        ub = u.view(np.int64).copy()
        u = _step(ub, (r != 0) & ((ub & 1) == 0), (r > 0) == (u > 0)).view(f64)
        slow = u.astype(f32)
        if odd:
            back = slow.astype(f64)
            fb = slow.view(np.uint32).astype(np.int64)
            slow = _step(fb, (back != u) & ((fb & 1) == 0), (u > back) == (slow > 0)).astype(np.uint32).view(f32)
        return np.where((c == 0) & wave_fast_path, fast, slow)


def expected(terms, fmt):
    s, e = O.exact_sum([np.asarray(t, dtype=f64) for t in terms])
    return O.round_to_format(s, fmt, e)


def bf16_of_f32(a):
    """Round float32 values to bfloat16 (nearest even), as float32 values."""
    return O.bf16_decode(O.bf16_encode(np.asarray(a, dtype=f64))).astype(f32)


def random_terms(rng, n, k, bf16, span):
    """k arrays of n terms: random signs, magnitudes 2^[-span/2, span/2], some zeros."""
    out = []
    for _ in range(k):
        mag = np.exp2(rng.uniform(-span / 2, span / 2, n)) * rng.uniform(1, 2, n)
        v = (mag * rng.choice([-1.0, 1.0], n)).astype(f32)
        v[rng.random(n) < 0.02] = 0.0
        v[rng.random(n) < 0.01] = -0.0
        out.append(bf16_of_f32(v) if bf16 else v)
    return out


@pytest.mark.parametrize("bf16_terms,span", [(True, 20), (True, 50), (True, 62), (False, 20), (False, 40), (False, 46)])
def test_random_terms_round_like_the_exact_sum(bf16_terms, span):
    """Random terms within the stated range (bf16 terms within 2^63 of one
    another, float32 terms within 2^47; magnitudes here span 2^(span+1)):
    float32 and bf16 targets, 2-9 terms."""
    rng = np.random.default_rng(span + 1000 * bf16_terms)
    for k in range(2, 10):
        terms = random_terms(rng, 20000, k, bf16_terms, span)
        want = expected(terms, O.F32).astype(f32).view(np.uint32)
        want16 = O.bf16_encode(expected(terms, O.BF16))
        for fast in (True, False):
            got = replay(terms, wave_fast_path=fast)
            assert np.array_equal(got.view(np.uint32), want), (k, fast)
            got16 = O.bf16_encode(replay(terms, odd=True, wave_fast_path=fast).astype(f64))
            assert np.array_equal(got16, want16), (k, fast)


def test_near_midpoints():
    """Terms built so that the exact sum lies on, just above or just below a
    float32 or bfloat16 rounding midpoint (a sum rounded twice would be off)."""
    rng = np.random.default_rng(5)
    n = 50000
    base = bf16_of_f32(rng.uniform(1, 2, n).astype(f32))
    half32 = np.ldexp(1.0, np.frexp(base.astype(f64))[1] - 25).astype(f32)   # half an f32 ulp of base
    half16 = np.ldexp(1.0, np.frexp(base.astype(f64))[1] - 9).astype(f32)    # half a bf16 ulp of base
    tiny = bf16_of_f32(np.ldexp(rng.uniform(1, 2, n), -rng.integers(30, 70, n)).astype(f32))
    sign = rng.choice([-1.0, 1.0, 0.0], n).astype(f32)
    for half in (half32, half16):
        terms = [base, half, (sign * tiny).astype(f32), -base * 0, np.full(n, -0.0, dtype=f32)]
        assert np.array_equal(replay(terms).view(np.uint32), expected(terms, O.F32).astype(f32).view(np.uint32))
        assert np.array_equal(O.bf16_encode(replay(terms, odd=True).astype(f64)),
                              O.bf16_encode(expected(terms, O.BF16)))


def test_cancellation_and_signed_zeros():
    cases = [
        [2.0 ** 60, 1.0, -(2.0 ** 60)],
        [2.0 ** 40, 3.0, -(2.0 ** 40), 2.0 ** -30],
        [2.0 ** 30, 2.0 ** -30, -(2.0 ** 30), 2.0 ** -36, 2.0 ** -37],
        [-0.0, -0.0, -0.0],
        [-0.0, 0.0, -0.0],
        [1.0, -1.0],
        [-1.0, 1.0, -0.0],
    ]
    for terms in cases:
        t = [np.array([v], dtype=f32) for v in terms]
        got = replay(t)
        want = expected(t, O.F32).astype(f32)
        assert got.view(np.uint32)[0] == want.view(np.uint32)[0], (terms, got, want)


def test_a_plain_float32_sum_would_fail_these():
    """The same hazards summed in float32 in slot order give other bits: the
    hazards are real, so the tests above do check the exact algorithm."""
    terms = [np.array([1.0], f32), np.array([2.0 ** -24], f32), np.array([2.0 ** -60], f32)]
    plain = (terms[0] + terms[1]) + terms[2]
    assert plain[0] != expected(terms, O.F32)[0]
    assert replay(terms)[0] == expected(terms, O.F32)[0]


def test_outside_the_stated_range_the_last_bit_can_be_off():
    """Terms spanning 2^150 (largest running sum 2^70, last bit 2^-80): the
    error sum no longer fits a double, and the rounding at a midpoint can be
    off by one unit -- the documented limit is a real one."""
    terms = [np.array([v], f32) for v in (2.0 ** 70, 1.0, 2.0 ** -24, 2.0 ** -80, -(2.0 ** 70))]
    assert expected(terms, O.F32)[0] == 1.0 + 2.0 ** -23
    assert replay(terms)[0] == 1.0
