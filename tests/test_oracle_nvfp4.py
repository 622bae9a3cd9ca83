"""Pins for the oracle's NVFP4 output (E2M1 codes, an E4M3FN scale per 16
elements, a float32 scale per tensor).

Each check takes an implementation with the oracle's signature, so that the
same checks can be run against copies with planted mistakes (at the end of
this file): every such mutant must fail at least one check that the oracle
passes.  Expected codes are written out by hand from the format tables:
E4M3FN code = sign << 7 | (exponent + 7) << 3 | 3-bit fraction (subnormals
m * 2^-9), E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 are codes 0..7.
"""

import numpy as np
import pytest

from oracle import blockquant as B
from oracle import rownorm as O

def check_exact_block_max(impl):
    """Block maxima 6 * s_t * v for E4M3FN values v: the block scale is v's code
    and the maximum element encodes to exactly -6 (code 0xF)."""
    st = 0.15625  # 5 * 2^-5, a float32
    cases = [(1.0, 0x38), (0.875, 0x36), (448.0, 0x7E), (2.0 ** -9, 0x01), (3 * 2.0 ** -9, 0x03),
             (1.625, 0x3D), (240.0, 0x77), (2.0 ** -6, 0x08)]
    y = np.zeros((len(cases), 32))
    for r, (v, _) in enumerate(cases):
        y[r, 5] = -6.0 * st * v
        y[r, 2] = 6.0 * st * v * 0.3  # 1.8 in units of the block scale -> nearest 2.0, code 0x4
        y[r, 16:] = 6.0 * st * 0.5  # second block: amax/(6 s_t) = 0.5, code 0x30
    q = impl(y, st)
    for r, (v, code) in enumerate(cases):
        assert q["amax"][r, 0] == 6.0 * st * v
        assert q["scale_codes"][r, 0] == code, (v, q["scale_codes"][r, 0])
        assert q["scale_codes"][r, 1] == 0x30
        assert q["codes"][r, 5] == 0xF
        assert q["codes"][r, 2] == 0x4
        assert np.all(q["codes"][r, 16:] == 0x7)


def check_block_size(impl):
    """Blocks are 16 consecutive elements with independent scales."""
    st = 1.0
    y = np.zeros((1, 64))
    for k, v in enumerate((1.0, 4.0, 0.25, 2.0 ** -7)):
        y[0, 16 * k: 16 * k + 16] = np.linspace(-6.0 * v, 3.0 * v, 16)
    q = impl(y, st)
    assert list(q["scale_codes"][0]) == [0x38, 0x48, 0x28, 0x04]  # 2^-7 = 4 * 2^-9, subnormal
    assert q["amax"].shape == (1, 4)


def check_error_bounds(impl):
    """Random rows with outliers and the usual tensor scale amax / (6 * 448):
    the block scale is within half an E4M3FN step of amax_b / (6 s_t), every
    element within half an E2M1 step of y / (s_b s_t) or saturated, and each
    block's largest element lands on +-6."""
    rng = np.random.default_rng(50)
    y = rng.standard_normal((24, 512)) * np.exp2(rng.integers(-6, 6, (24, 1)))
    y[rng.random(y.shape) < 0.01] *= 20
    st = float(np.float32(np.max(np.abs(y)) / (6 * 448)))
    q = impl(y, st)
    b = y.reshape(24, -1, 16)
    amax = np.max(np.abs(b), axis=2)
    sv = amax / (6 * st)
    dec = O.e4m3fn_decode(q["scale_codes"])
    normal = (sv >= 2.0 ** -6) & (sv <= 448)
    assert np.all(np.abs(dec - sv)[normal] <= 2.0 ** -4 * sv[normal] * (1 + 1e-12))
    sub = sv < 2.0 ** -6
    assert np.all(np.abs(dec - sv)[sub] <= 2.0 ** -10 * (1 + 1e-12))
    d = (dec * st)[:, :, None]
    v = np.where(d > 0, b / np.where(d > 0, d, 1.0), 0.0)
    got = B.e2m1_decode(q["codes"]).reshape(b.shape)
    a = np.abs(v)
    half = np.select([a < 2.0, a < 4.0], [0.25, 0.5], 1.0)
    inside = a <= 6.0
    assert np.all(np.abs(got - v)[inside] <= half[inside] * (1 + 1e-12))
    assert np.all(np.abs(got[~inside]) == 6.0)
    assert np.all(np.signbit(got[~inside]) == np.signbit(v[~inside]))
    top = np.argmax(np.abs(b), axis=2)
    top_code = np.take_along_axis(q["codes"].reshape(b.shape), top[:, :, None], axis=2)[:, :, 0]
    assert np.all((top_code & 0x7)[normal] == 0x7)


def check_zero_and_tiny(impl):
    """A zero block, a block whose scale rounds to zero (codes all zero even for
    nonzero elements) and one that rounds up to the smallest subnormal scale."""
    y = np.zeros((1, 48))
    y[0, 16] = 6.0 * 2.0 ** -11  # amax/(6 s_t) = 2^-11 < 2^-10: scale code 0
    y[0, 17] = -3.0 * 2.0 ** -11
    y[0, 32] = 6.0 * 1.5 * 2.0 ** -10  # 1.5 * 2^-10 -> 2^-9 (code 0x01); element 4.5 -> 4, code 0x6
    y[0, 33] = -2.0 ** -9  # -1 in units of the block scale -> code 0xA
    q = impl(y, 1.0)
    assert list(q["scale_codes"][0]) == [0x00, 0x00, 0x01]
    assert np.all(q["codes"][0, :32] == 0)
    assert q["codes"][0, 32] == 0x6 and q["codes"][0, 33] == 0xA


def check_saturation(impl):
    """A block whose scale would exceed 448 saturates there; its elements
    saturate at 6."""
    y = np.zeros((1, 16))
    y[0, 0] = 6000.0  # amax/(6 s_t) = 1000 -> 448 (0x7E); 6000/448 = 13.4 -> 6 (0x7)
    y[0, 1] = -224.0  # -0.5 -> code 0x9
    q = impl(y, 1.0)
    assert q["scale_codes"][0, 0] == 0x7E
    assert q["codes"][0, 0] == 0x7 and q["codes"][0, 1] == 0x9


def check_given_scale(impl):
    """With the block scales given, codes are the E2M1 roundings of y / (s_b s_t):
    1.45 -> 1.5, a tie 3.5 -> 4 (even code), 0.245 -> 0, 50 -> 6."""
    y = np.zeros((1, 16))
    y[0, :4] = [2.9, -7.0, 0.49, 100.0]
    q = impl(y, 2.0, scale_codes=np.array([[0x38]], dtype=np.uint8))  # s_b = 1, s_b s_t = 2
    assert list(q["codes"][0, :4]) == [0x3, 0xE, 0x0, 0x7]


def check_pow2_invariance(impl):
    """Scaling the data and the tensor scale by the same power of two changes no code."""
    rng = np.random.default_rng(51)
    y = rng.standard_normal((4, 128))
    st = float(np.float32(np.max(np.abs(y)) / (6 * 448)))
    ref = impl(y, st)
    for k in (-9, 7):
        q = impl(y * 2.0 ** k, st * 2.0 ** k)
        assert np.array_equal(q["scale_codes"], ref["scale_codes"])
        assert np.array_equal(q["codes"], ref["codes"])


CHECKS = [check_exact_block_max, check_block_size, check_error_bounds, check_zero_and_tiny, check_saturation,
          check_given_scale, check_pow2_invariance]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(B.nvfp4_quantize)


def test_rejects_bad_tensor_scale():
    for st in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            B.nvfp4_quantize(np.ones((1, 16)), st)


# ---------------------------------------------------------------------------
# Planted mistakes (CPU copies only).
# ---------------------------------------------------------------------------

def _mutant(*, top=6.0, codes_without_tensor_scale=False, block=16, scale_round="nearest",
            signed_max=False, tensor_scale_times=False):
    def impl(y, tensor_scale, scale_codes=None):
        st = float(np.float32(tensor_scale))
        y = np.asarray(y, dtype=np.float64)
        b = y.reshape(y.shape[0], -1, block)
        amax = np.max(b, axis=2) if signed_max else np.max(np.abs(b), axis=2)
        sv = amax * (top * st) if tensor_scale_times else amax / (top * st)
        if scale_round == "nearest":
            own = O.e4m3fn_encode(sv)
        else:  # truncate or round up onto the E4M3FN grid
            grid = O.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
            idx = np.searchsorted(grid, np.minimum(sv, 448.0), side="right") - 1
            if scale_round == "up":
                idx = np.where(grid[np.clip(idx, 0, 126)] < sv, np.minimum(idx + 1, 126), idx)
            own = np.clip(idx, 0, 126).astype(np.uint8)
        sc = own if scale_codes is None else np.asarray(scale_codes, dtype=np.uint8)
        d = O.e4m3fn_decode(sc) * (1.0 if codes_without_tensor_scale else st)
        safe = np.where(d > 0, d, 1.0)
        codes = B.e2m1_encode(b / safe[:, :, None])
        codes[d == 0] = 0
        return {"amax": np.max(np.abs(b), axis=2), "scale_codes": own, "codes": codes.reshape(y.shape)}
    return impl


MUTANTS = {
    "scale_maps_max_to_448": _mutant(top=448.0),
    "scale_maps_max_to_4": _mutant(top=4.0),
    "codes_without_tensor_scale": _mutant(codes_without_tensor_scale=True),
    "block_of_32": _mutant(block=32),
    "block_of_8": _mutant(block=8),
    "scale_truncated": _mutant(scale_round="down"),
    "scale_rounded_up": _mutant(scale_round="up"),
    "signed_max": _mutant(signed_max=True),
    "tensor_scale_multiplied": _mutant(tensor_scale_times=True),
}


def test_unmutated_copy_passes():
    impl = _mutant()
    for check in CHECKS:
        check(impl)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    failed = []
    for check in CHECKS:
        try:
            check(MUTANTS[name])
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passes every check"
