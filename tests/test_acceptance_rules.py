"""Pins for the acceptance rules themselves (oracle/compare.py): the rounding
discipline accepts a correctly rounded output with float32-sized evaluation
noise and rejects a truncating conversion or flips away from rounding
midpoints, which the one-step bounds alone would accept."""

import numpy as np

from oracle import blockquant as B
from oracle import compare as C
from oracle import rownorm as O


def _values(seed, n=20000, scale_exp=(-20, 20)):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n) * np.exp2(rng.integers(*scale_exp, n))


def test_bf16_noise_accepted_truncation_rejected():
    y = _values(60)
    noisy = y * (1.0 + np.random.default_rng(61).uniform(-3e-6, 3e-6, y.size))
    good = O.bf16_encode(noisy)  # correctly rounded from a slightly perturbed value
    rep = C.check_bf16(good, y)
    assert rep["ok"], rep
    # truncation toward zero: within one ulp everywhere, but not round-to-nearest
    trunc = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert C.check_bf16(trunc, y)["max_ulp"] <= 1.0
    rep = C.check_bf16(trunc, y)
    assert not rep["ok"] and rep["n_bad"] == 0 and rep["n_bad_rounding"] > 1000


def test_exact_midpoints_take_either_neighbour():
    # bf16 neighbours 1 and 1 + 2^-7: the midpoint 1 + 2^-8 may round either way
    y = np.array([1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20])
    lower = O.bf16_encode(np.array([1.0, 1.0]))
    assert C.check_bf16(lower, y)["ok"]  # both within 2^-15 relative of the midpoint
    y_far = np.array([1.0 + 2.0 ** -8 + 2.0 ** -12])
    assert not C.check_bf16(O.bf16_encode(np.array([1.0])), y_far)["ok"]


def test_fp8_and_fp4_codes_rounding_discipline():
    v = _values(62, scale_exp=(-8, 9))
    v = np.clip(v, -600, 600)
    ref8 = O.e4m3fn_decode(O.e4m3fn_encode(v))
    assert C.check_rounding(ref8, v, O.E4M3FN)["ok"]
    # one step toward zero everywhere: rejected
    codes = O.e4m3fn_encode(v)
    mag = codes & 0x7F
    down = np.where(mag > 0, codes - 1, codes).astype(np.uint8)
    rep = C.check_rounding(O.e4m3fn_decode(down), v, O.E4M3FN)
    assert not rep["ok"] and rep["n_bad"] > v.size // 2
    w = np.clip(_values(63, scale_exp=(-3, 3)), -8, 8)
    ref4 = B.e2m1_decode(B.e2m1_encode(w))
    assert C.check_rounding(ref4, w, B.E2M1)["ok"]
    # truncating E2M1 conversion (toward zero onto the grid): rejected
    grid = B.e2m1_decode(np.arange(8))
    t = np.sign(w) * grid[np.searchsorted(grid, np.minimum(np.abs(w), 6.0), side="right") - 1]
    assert not C.check_rounding(t, w, B.E2M1)["ok"]


def test_bf16_subnormal_window():
    # values far below float32's normal range: float32 intermediates carry absolute
    # errors of a few 2^-149, so the window there is absolute (2^-140)
    q = 2.0 ** -133  # bf16 subnormal quantum
    y = np.array([3.5 * q + 2.0 ** -148, -(5.5 * q) - 2.0 ** -148])  # just past midpoints
    other_side = O.bf16_encode(np.array([3.0 * q, -5.0 * q]))  # the neighbours below them
    rep = C.check_bf16(other_side, y)
    assert rep["ok"] and rep["n_near_midpoint_other_side"] == 2, rep
    far = np.array([3.2 * q])  # 0.3 quanta from the midpoint: must round to 3 quanta
    assert not C.check_bf16(O.bf16_encode(np.array([4.0 * q])), far)["ok"]
