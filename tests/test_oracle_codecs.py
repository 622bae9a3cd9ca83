"""Pins for the oracle's number formats: bf16, f32 and OCP e4m3fn rounding.

Each check compares the oracle's own encoder/decoder (written from the
format definitions) with something independent of it: torch's CPU casts,
numpy's IEEE float32 arithmetic, exact rational arithmetic, or the OCP FP8
specification's landmark table in tests/golden/.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import rownorm as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _torch_bf16_bits_from_f32(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_encode_random_vs_torch():
    rng = np.random.default_rng(1)
    # every binade from the subnormals to overflow, random fraction bits
    u = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = O.bf16_encode(f.astype(np.float64))
    ref = _torch_bf16_bits_from_f32(f)
    assert np.array_equal(ours, ref)


def test_bf16_encode_exact_ties_go_to_even():
    hi = np.arange(0, 0x7F7F, 7, dtype=np.uint32)  # finite bf16 patterns (positive)
    mid = ((hi << 16) | 0x8000).view(np.float32)  # exactly halfway between hi and hi + 1
    ours = O.bf16_encode(mid.astype(np.float64))
    expect = np.where(hi % 2 == 0, hi, hi + 1).astype(np.uint16)
    assert np.array_equal(ours, expect)
    assert np.array_equal(ours, _torch_bf16_bits_from_f32(mid))


def test_f32_round_vs_numpy_cast():
    rng = np.random.default_rng(2)
    d = rng.standard_normal(1 << 18) * np.exp2(rng.integers(-160, 140, size=1 << 18))
    ours = O.round_to_format(d, O.F32)
    with np.errstate(over="ignore"):
        ref = d.astype(np.float32).astype(np.float64)  # IEEE round to nearest even
    assert np.array_equal(ours, ref)


def test_round_to_format_sticky_tie_break_vs_fractions():
    # v on an exact f32 midpoint: the true value v + err decides the direction.
    one = 1.0
    mid = one + 2.0 ** -24
    assert O.round_to_format(np.array([mid]), O.F32)[0] == one  # tie -> even
    assert O.round_to_format(np.array([mid]), O.F32, np.array([1e-30]))[0] == one + 2.0 ** -23
    assert O.round_to_format(np.array([mid]), O.F32, np.array([-1e-30]))[0] == one
    assert O.round_to_format(np.array([-mid]), O.F32, np.array([-1e-30]))[0] == -(one + 2.0 ** -23)
    # random (v, err) pairs against exact rational rounding
    rng = np.random.default_rng(3)
    for _ in range(2000):
        base = float(np.float32(rng.standard_normal()))
        ulp = np.spacing(np.float32(abs(base)))
        v = base + float(ulp) / 2 * rng.choice([-1, 1])  # a midpoint of f32 (exact in double)
        err = float(rng.choice([-1, 0, 1])) * 2.0 ** -70
        got = O.round_to_format(np.array([v]), O.F32, np.array([err]))[0]
        true = Fraction(v) + Fraction(err)
        lo = np.float32(v)
        cands = sorted({float(lo), float(np.nextafter(lo, np.float32(np.inf))),
                        float(np.nextafter(lo, np.float32(-np.inf)))})
        dists = [abs(Fraction(c) - true) for c in cands]
        best = min(dists)
        winners = [c for c, dd in zip(cands, dists) if dd == best]
        if len(winners) == 1:
            assert got == winners[0]
        else:  # exact tie: even significand
            evens = [c for c in winners if (np.float32(c).view(np.uint32) & 1) == 0]
            assert got == evens[0]


def test_residual_add_f32_bit_exact_vs_numpy_float32_add():
    rng = np.random.default_rng(4)
    n = 1 << 18
    x_bits = _torch_bf16_bits_from_f32(rng.standard_normal(n).astype(np.float32) *
                                       np.exp2(rng.integers(-40, 10, n)).astype(np.float32))
    x = O.bf16_decode(x_bits)
    r = (rng.standard_normal(n) * 4).astype(np.float32)
    ours = O.residual_add(x, r.astype(np.float64), "f32")
    ref = (x.astype(np.float32) + r).astype(np.float64)  # IEEE float32 add, one rounding
    assert np.array_equal(ours, ref)


def test_residual_add_bf16_bit_exact_vs_torch_bfloat16_add():
    rng = np.random.default_rng(5)
    n = 1 << 18
    a = _torch_bf16_bits_from_f32(rng.standard_normal(n).astype(np.float32))
    b = _torch_bf16_bits_from_f32((rng.standard_normal(n) *
                                   np.exp2(rng.integers(-30, 4, n))).astype(np.float32))
    ours = O.bf16_encode(O.residual_add(O.bf16_decode(a), O.bf16_decode(b), "bf16"))
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    ref = (ta + tb).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _load_landmarks(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "e4m3fn_landmarks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            code, val, label = line.split()
            rows.append((int(code, 16), float(val), label))
    return rows


def test_e4m3fn_landmarks_from_spec(golden_dir):
    rows = _load_landmarks(golden_dir)
    assert len(rows) >= 10
    for code, val, label in rows:
        got = O.e4m3fn_decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got), label
            continue
        assert got == val and np.signbit(got) == np.signbit(val), label
        assert O.e4m3fn_encode(np.array([val]))[0] == code, label


def test_e4m3fn_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_roundtrip_and_midpoints_to_even():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.e4m3fn_decode(codes)
    assert np.array_equal(O.e4m3fn_encode(vals), codes)
    pos = np.arange(0, 0x7E, dtype=np.uint8)  # pairs (c, c + 1) of positive finite codes
    lo, hi = O.e4m3fn_decode(pos), O.e4m3fn_decode(pos + 1)
    mids = (lo + hi) / 2
    got = O.e4m3fn_encode(mids)
    expect = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, expect)
    assert np.array_equal(O.e4m3fn_encode(-mids), expect | 0x80)


def test_e4m3fn_encode_random_vs_torch_in_range():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal(1 << 18) * np.exp2(rng.integers(-14, 9, 1 << 18))).astype(np.float32)
    v = np.clip(v, -448, 448)  # torch's out-of-range behaviour is not relied on
    ours = O.e4m3fn_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3fn_saturates_out_of_range():
    v = np.array([448.0, 449.0, 463.99, 464.0, 1e9, -500.0, -1e30])
    assert list(O.e4m3fn_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
