"""Pins for the oracle's block-scaled outputs (FP8 groups, MXFP8, MXFP4).

Checked against the MX specification's value tables (tests/golden/), brute
force nearest-value search, closed forms and invariants, and the separately
pinned per-row fp8 scheme.
"""

import os

import numpy as np
import pytest

from oracle import blockquant as B
from oracle import rownorm as O


def _golden(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "mx_landmarks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_e2m1_and_e8m0_tables_from_spec(golden_dir):
    n = 0
    for kind, code, val in _golden(golden_dir):
        if kind == "e2m1":
            c = int(code, 16)
            got = B.e2m1_decode(np.array([c]))[0]
            assert got == float(val) and np.signbit(got) == np.signbit(float(val)), code
            assert B.e2m1_encode(np.array([float(val)]))[0] == c, code
            n += 1
        elif kind == "e8m0":
            got = B.e8m0_decode(np.array([int(code)]))[0]
            if val == "nan":
                assert np.isnan(got)
            else:
                assert got == float(val), code
            n += 1
        elif kind == "emax":
            assert B.EMAX_ELEM[code] == int(val)
    assert n == 22


def test_e2m1_encode_is_nearest_with_ties_to_even_code():
    rng = np.random.default_rng(30)
    v = np.concatenate([rng.uniform(-8, 8, 20000),
                        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 6.0, 6.5, 100.0, -7.0, 1e-9]])
    got = B.e2m1_encode(v)
    table = B.e2m1_decode(np.arange(16))
    for x, c in zip(v, got):
        xs = min(max(x, -6.0), 6.0)  # saturation
        d = np.abs(table - xs)
        best = np.flatnonzero(d == d.min())
        best = [b for b in best if np.signbit(table[b]) == np.signbit(xs) or table[b] != 0] or list(best)
        if len(best) > 1:  # exact tie: the even code (mantissa bit 0)
            best = [b for b in best if b % 2 == 0]
        assert B.e2m1_decode(np.array([c]))[0] == table[best[0]], (x, c, best)


def test_pack_unpack_fp4_roundtrip():
    c = np.random.default_rng(31).integers(0, 16, (3, 64)).astype(np.uint8)
    p = B.pack_fp4(c)
    assert p.shape == (3, 32)
    assert np.array_equal(B.unpack_fp4(p), c)
    assert p[0, 0] == (c[0, 0] | (c[0, 1] << 4))


@pytest.mark.parametrize("elem", ["fp8_e4m3fn", "fp4_e2m1"])
def test_mx_power_of_two_block_max(elem):
    """A block whose max is exactly 2^k: shared exponent k - emax, and that
    element encodes to exactly 2^emax (E4M3 256 = 0x78, E2M1 4.0 = 0x6)."""
    for k in (-20, -3, 0, 5, 17):
        y = np.zeros((1, 32))
        y[0, 7] = -(2.0 ** k)
        y[0, 3] = 2.0 ** (k - 2) * 1.5
        q = B.mx_quantize(y, elem)
        assert q["shared_exp"][0, 0] == k - B.EMAX_ELEM[elem]
        assert q["scale_codes"][0, 0] == k - B.EMAX_ELEM[elem] + 127
        top = 0xF8 if elem == "fp8_e4m3fn" else 0xE  # negative 2^emax
        assert q["codes"][0, 7] == top


@pytest.mark.parametrize("elem", ["fp8_e4m3fn", "fp4_e2m1"])
def test_mx_top_binade_and_error_bounds(elem):
    rng = np.random.default_rng(32)
    y = rng.standard_normal((16, 256)) * np.exp2(rng.integers(-12, 12, (16, 1)))
    y[rng.random(y.shape) < 0.02] *= 20
    q = B.mx_quantize(y, elem)
    blocks = y.reshape(16, -1, 32)
    X = np.ldexp(1.0, q["shared_exp"])[:, :, None]
    scaled = np.abs(blocks) / X
    emax = B.EMAX_ELEM[elem]
    # the block maximum lands in the element format's top binade [2^emax, 2^(emax+1))
    m = scaled.max(axis=2)
    assert np.all((m >= 2.0 ** emax) & (m < 2.0 ** (emax + 1)))
    dec = (O.e4m3fn_decode(q["codes"]) if elem == "fp8_e4m3fn" else B.e2m1_decode(q["codes"])).reshape(blocks.shape)
    deq = dec * X
    maxv = 448.0 if elem == "fp8_e4m3fn" else 6.0
    mant_bits = 3 if elem == "fp8_e4m3fn" else 1
    emin = -6 if elem == "fp8_e4m3fn" else 0
    sat = scaled > maxv
    assert np.all(np.abs(dec[sat]) == maxv)
    ok = ~sat
    normal = scaled >= 2.0 ** emin
    tol_rel = 2.0 ** -(mant_bits + 1)
    err = np.abs(np.abs(deq) - np.abs(blocks))
    assert np.all(err[ok & normal] <= tol_rel * np.abs(blocks[ok & normal]) * (1 + 1e-12))
    half_quantum = 2.0 ** (emin - mant_bits - 1)
    assert np.all(err[ok & ~normal] <= (half_quantum * X + 0 * blocks)[ok & ~normal] * (1 + 1e-12))


def test_mx_all_zero_block_and_given_exponent():
    y = np.zeros((2, 64))
    y[1, 40] = 3.0
    q = B.mx_quantize(y, "fp8_e4m3fn")
    assert list(q["scale_codes"][0]) == [0, 0] and q["scale_codes"][1, 0] == 0
    assert q["shared_exp"][1, 1] == 1 - 8
    assert np.all(q["codes"][0] == 0)
    # codes judged with another exponent follow it exactly
    se = q["shared_exp"].copy()
    se[1, 1] -= 1
    q2 = B.mx_quantize(y, "fp8_e4m3fn", shared_exp=se)
    assert q2["codes"][1, 40] == O.e4m3fn_encode(np.array([3.0 * 2.0 ** 8]))[0]  # 768 saturates to 448


def test_group_fp8_one_group_per_row_is_the_row_scheme():
    rng = np.random.default_rng(33)
    y = rng.standard_normal((8, 512)) * 3
    g = B.fp8_quantize_groups(y, group=512)
    r = O.fp8_quantize_rows(y)
    assert np.array_equal(g["scale"][:, 0], r["scale"])
    assert np.array_equal(g["codes"], r["codes"])


def test_group_fp8_groups_are_independent():
    rng = np.random.default_rng(34)
    y = rng.standard_normal((4, 1024))
    y[:, 128:256] *= 50  # one loud group must not change the others
    g = B.fp8_quantize_groups(y, group=128)
    for j in range(8):
        part = O.fp8_quantize_rows(y[:, 128 * j:128 * (j + 1)])
        assert np.array_equal(g["scale"][:, j], part["scale"])
        assert np.array_equal(g["codes"][:, 128 * j:128 * (j + 1)], part["codes"])
    assert np.all(np.max(g["codes"].reshape(4, 8, 128) & 0x7F, axis=2) == 0x7E)
