"""The oracle's pins catch plausible mistakes.

Each mutant below is a copy of the oracle's RMSNorm with one plausible slip
(a dropped term, a wrong divisor, a transposed or reversed operand, a sign,
eps in the wrong place or precision, the norm over the unrounded residual
sum).  Every mutant must fail at least one of the pins that the real oracle
passes; a mutant that slipped through would mean the pins could not tell
that mistake from the definition.  The mistakes are planted here, in CPU
copies of the oracle, never in any GPU code.
"""

import numpy as np
import pytest

from oracle import rownorm as O
from tests.test_oracle_rmsnorm import ALL_CHECKS, check_closed_forms


def _mutant(*, drop_eps=False, eps_outside=False, sum_not_mean=False, divisor_minus_one=False,
            sqrt_not_rsqrt=False, drop_bias=False, bias_on_x=False, eps_double=False,
            unrounded_residual=False, wrong_axis=False, negate=False, reverse_weight=False,
            abs_not_square=False):
    def impl(x, weight, eps, weight_bias, residual=None, res_dtype=None):
        x = np.asarray(x, dtype=np.float64)
        H = x.shape[1]
        if residual is not None:
            s = x + np.asarray(residual, dtype=np.float64)
            h_out = O.round_to_format(s, O.FORMATS[res_dtype])
            h = s if unrounded_residual else h_out
        else:
            h = h_out = x
        e = eps if eps_double else float(np.float32(eps))
        sq = np.abs(h) if abs_not_square else h * h
        if wrong_axis:
            total = np.sum(sq, axis=0).mean() * np.ones(h.shape[0])
        else:
            total = np.sum(sq, axis=1)
        div = H - 1 if (divisor_minus_one and H > 1) else H
        ms = total if sum_not_mean else total / div
        if drop_eps:
            inv = 1.0 / np.sqrt(ms)
        elif eps_outside:
            inv = 1.0 / np.sqrt(ms) + e
        else:
            inv = 1.0 / np.sqrt(ms + e)
        if sqrt_not_rsqrt:
            inv = 1.0 / inv
        w = np.asarray(weight, dtype=np.float64)
        if reverse_weight:
            w = w[::-1]
        if bias_on_x:
            y = w[None, :] * (h + weight_bias) * inv[:, None]
        else:
            wb = w if drop_bias else w + weight_bias
            y = wb[None, :] * h * inv[:, None]
        if negate:
            y = -y
        with np.errstate(all="ignore"):
            return {"h": h_out, "inv": inv, "y": y}
    return impl


MUTANTS = {
    name: _mutant(**{name: True})
    for name in ["drop_eps", "eps_outside", "sum_not_mean", "divisor_minus_one", "sqrt_not_rsqrt",
                 "drop_bias", "bias_on_x", "eps_double", "unrounded_residual", "wrong_axis", "negate",
                 "reverse_weight", "abs_not_square"]
}


def _fails_some_check(impl, golden_dir):
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                if check is check_closed_forms:
                    check(impl, golden_dir)
                else:
                    check(impl)
        except (AssertionError, ZeroDivisionError, ValueError, FloatingPointError):
            return check.__name__
    return None


def test_unmutated_copy_passes(golden_dir):
    assert _fails_some_check(_mutant(), golden_dir) is None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, golden_dir):
    caught_by = _fails_some_check(MUTANTS[name], golden_dir)
    assert caught_by is not None, f"mutant {name} passed every pin"
