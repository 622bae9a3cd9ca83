"""Pins for the oracle's per-row fp8 e4m3fn output quantization.

Checked against the format's own error bounds, numpy's IEEE float32 division
for the scale, and invariants of ``scale = amax / 448``.
"""

import numpy as np
import pytest

from oracle import rownorm as O


def _rows(seed, rows=32, H=7168, outliers=True):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((rows, H))
    if outliers:
        y[rng.random((rows, H)) < 0.01] *= 20
    return y * np.exp2(rng.integers(-10, 10, (rows, 1)))


def test_scale_is_float32_division_of_float32_amax():
    y = _rows(20)
    q = O.fp8_quantize_rows(y)
    amax32 = np.max(np.abs(y), axis=1).astype(np.float32)
    ref = amax32 / np.float32(448.0)  # numpy float32 division: IEEE, one rounding
    assert ref.dtype == np.float32
    assert np.array_equal(q["scale"], ref)


def test_every_nonzero_row_reaches_the_top_code():
    q = O.fp8_quantize_rows(_rows(21))
    assert np.all(np.max(q["codes"] & 0x7F, axis=1) == 0x7E)


def test_dequantized_error_within_format_bounds():
    y = _rows(22)
    q = O.fp8_quantize_rows(y)
    s = q["scale"].astype(np.float64)[:, None]
    deq = O.e4m3fn_decode(q["codes"]) * s
    v = np.abs(y / s)
    normal = v >= 2.0 ** -6
    err = np.abs(deq - y)
    # normal: at most half an ulp of 3 fraction bits = 2^-4 relative
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(y[normal]) * (1 + 1e-12))
    # subnormal: at most half the quantum 2^-9, in units of the scale
    assert np.all(err[~normal] <= 2.0 ** -10 * np.broadcast_to(s, y.shape)[~normal] * (1 + 1e-12))


def test_codes_use_the_given_scale():
    y = _rows(23, rows=4, H=512)
    own = O.fp8_quantize_rows(y)
    other = own["scale"] * np.float32(1.0 + 2.0 ** -20)
    q2 = O.fp8_quantize_rows(y, scale=other)
    expect = O.e4m3fn_encode(y / other.astype(np.float64)[:, None])
    assert np.array_equal(q2["codes"], expect)


def test_zero_row_gives_zero_scale_and_codes():
    y = np.zeros((3, 64))
    y[1] = np.linspace(-1, 1, 64)
    q = O.fp8_quantize_rows(y)
    assert q["scale"][0] == 0 and q["scale"][2] == 0 and q["scale"][1] > 0
    assert np.all(q["codes"][0] == 0) and np.all(q["codes"][2] == 0)


def test_sign_symmetry():
    y = _rows(24, rows=4, H=256)
    a = O.fp8_quantize_rows(y)
    b = O.fp8_quantize_rows(-y)
    assert np.array_equal(a["scale"], b["scale"])
    nz = (a["codes"] & 0x7F) != 0
    assert np.array_equal(a["codes"][nz] ^ 0x80, b["codes"][nz])


def test_end_to_end_quantized_norm_row():
    """A hand-checked row: x = (1, -1, 2, -2), w = 1, b = 0, eps = 0.

    mean square = 2.5, y = x / sqrt(2.5), amax = 2 / sqrt(2.5), codes of
    y / scale are +-224 and +-448 (exact e4m3fn values 0x76 and 0x7E), up to
    the float32 rounding of the scale.
    """
    x = np.array([[1.0, -1.0, 2.0, -2.0]])
    y = O.rmsnorm_rows(x, np.ones(4), 0.0, 0.0)["y"]
    q = O.fp8_quantize_rows(y)
    assert list(q["codes"][0]) == [0x76, 0xF6, 0x7E, 0xFE]
    assert q["scale"][0] == np.float32(np.float32(2 / np.sqrt(2.5)) / np.float32(448))


def test_f32_acceptance_rule_underflow_floor():
    from oracle import compare as C
    # relative 1e-5 in the normal range ...
    assert C.check_f32(np.array([1.0 + 2e-6]), np.array([1.0]))["ok"]
    assert not C.check_f32(np.array([1.0 + 2e-5]), np.array([1.0]))["ok"]
    # ... and four subnormal quanta (4 * 2^-149) absolute below it: an exact
    # value of 1e-67 rounds to 0 in float32, which must be accepted, and so
    # must a correctly rounded subnormal; 0 for a subnormal of 3e-40 must not
    # (about 2e5 quanta), nor 1e-30
    q = 2.0 ** -149
    assert C.check_f32(np.array([0.0]), np.array([1e-67]))["ok"]
    assert C.check_f32(np.array([0.0]), np.array([2.5 * q]))["ok"]
    assert C.check_f32(np.array([1234 * q]), np.array([1236.9 * q]))["ok"]
    assert not C.check_f32(np.array([1234 * q]), np.array([1239 * q]))["ok"]
    assert not C.check_f32(np.array([-0.0]), np.array([-3e-40]))["ok"]
    assert not C.check_f32(np.array([0.0]), np.array([1e-30]))["ok"]
    # the SwiGLU float32 output's wider floor, 2^-126, accepts 0 for that subnormal
    assert C.check_f32(np.array([-0.0]), np.array([-3e-40]), abs_floor=C.SILU_F32_ABS_FLOOR)["ok"]
    assert not C.check_f32(np.array([0.0]), np.array([1e-30]), abs_floor=C.SILU_F32_ABS_FLOOR)["ok"]
