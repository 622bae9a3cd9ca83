"""Acceptance rules for comparing an implementation's outputs with the oracle.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``).

Tolerances (the stated target of the work):
  * bf16 outputs: within one bf16 ulp of the exact value, ulp(v) =
    2**(floor(log2|v|) - 7) (so either neighbour of a value near a rounding
    midpoint is accepted);
  * f32 outputs: relative error at most 1e-5, or at most four float32
    subnormal quanta (4 * 2^-149) absolute: below about 2^-126 / 1e-5 the
    format's own spacing in the subnormal range is coarser than a relative
    1e-5 (gradual underflow, then zero).  The SwiGLU float32 output takes a
    wider absolute floor, 2^-126 (``SILU_F32_ABS_FLOOR``): its exp(-|g|) is a
    float32 subnormal with fewer bits past |g| = 87.3, a range limit its C
    header states;
  * fp8 e4m3fn codes: at most one step apart, counting steps on the signed
    magnitude index (code & 0x7F, negated for negative codes), so +0 and -0
    are the same point and crossing zero costs the steps on either side;
  * bit-exact where one correctly rounded operation fixes the result (the
    updated residual);
  * rounding discipline (check_rounding), on top of the bounds above: every
    rounded output (bf16 values, fp8 / fp4 codes) equals the round-to-nearest-
    even value of the exact result, except where the exact value lies within
    NEAR_MIDPOINT_REL (relative) of the midpoint between the two neighbours.
    There the implementation's own float32 evaluation (sum order, rsqrt,
    hardware exp / reciprocal: a few 1e-6 relative) may land on either side.
    The one-step bounds alone would also accept a truncating conversion.
"""

from __future__ import annotations

from typing import Dict

import numpy as np

from .rownorm import BF16, Format, bf16_decode, round_to_format

__all__ = ["F32_ABS_FLOOR", "NEAR_MIDPOINT_REL", "SILU_F32_ABS_FLOOR", "bf16_ulp", "check_bf16", "check_f32",
           "check_fp8_codes", "check_fp4_codes", "check_rounding", "signed_index"]

# Window around a rounding midpoint inside which either neighbour is accepted:
# 2^-15 relative, about 5x the float32 evaluation error of the kernels' values
# (float32 sums of up to 32768 squares in any order: ~sqrt(H) * 2^-24; the
# hardware exp2 / reciprocal forms: ~2^-18).
NEAR_MIDPOINT_REL = 2.0 ** -15


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """ulp of |v| in bfloat16 (the spacing of the binade |v| lies in)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(E - 1, BF16.emin)
    e = np.where(a > 0, e, BF16.emin)
    return np.ldexp(1.0, e - (BF16.precision - 1))


# Absolute midpoint window for bf16 values in float32's subnormal range, where
# the implementation's float32 intermediates carry absolute (not relative)
# errors of a few 2^-149.
BF16_SUBNORMAL_WINDOW = 2.0 ** -140


def check_bf16(gpu_bits: np.ndarray, exact: np.ndarray) -> Dict[str, float]:
    """bf16 bits vs exact doubles: pass iff every |gpu - exact| <= ulp(exact) and the
    rounding discipline holds (``check_rounding``)."""
    g = bf16_decode(gpu_bits)
    y = np.asarray(exact, dtype=np.float64)
    err = np.abs(g - y)
    ulp = bf16_ulp(y)
    finite = np.isfinite(y)
    ok = np.where(finite, err <= ulp, np.isnan(g) == np.isnan(y))
    ratio = np.where(finite, err / ulp, 0.0)
    rnd = check_rounding(g[finite], y[finite], BF16, abs_tol=BF16_SUBNORMAL_WINDOW)
    return {"ok": bool(ok.all()) and rnd["ok"], "max_ulp": float(ratio.max(initial=0.0)),
            "n_bad": int((~ok).sum()), "n_bad_rounding": rnd["n_bad"],
            "n_near_midpoint_other_side": rnd["n_near_midpoint_other_side"], "n": int(ok.size)}


F32_MIN_NORMAL = 2.0 ** -126
F32_ABS_FLOOR = 4 * 2.0 ** -149      # four subnormal quanta
SILU_F32_ABS_FLOOR = F32_MIN_NORMAL  # the SwiGLU float32 output (see above)


def check_f32(gpu: np.ndarray, exact: np.ndarray, rtol: float = 1e-5,
              abs_floor: float = F32_ABS_FLOOR) -> Dict[str, float]:
    g = np.asarray(gpu, dtype=np.float64)
    y = np.asarray(exact, dtype=np.float64)
    err = np.abs(g - y)
    tol = np.maximum(rtol * np.abs(y), abs_floor)
    ok = (err <= tol) | (g == y)
    rel = np.where(y != 0, err / np.where(y != 0, np.abs(y), 1.0), np.where(err == 0, 0.0, np.inf))
    return {"ok": bool(ok.all()), "max_rel": float(rel.max(initial=0.0)),
            "n_bad": int((~ok).sum()), "n": int(ok.size)}


def signed_index(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_fp8_codes(gpu: np.ndarray, ref: np.ndarray, max_steps: int = 1) -> Dict[str, float]:
    d = np.abs(signed_index(gpu) - signed_index(ref))
    return {"ok": bool((d <= max_steps).all()), "max_steps": int(d.max(initial=0)),
            "frac_exact": float((d == 0).mean()) if d.size else 1.0, "n_bad": int((d > max_steps).sum()),
            "n": int(d.size)}


def check_fp4_codes(gpu: np.ndarray, ref: np.ndarray, max_steps: int = 1) -> Dict[str, float]:
    """4-bit E2M1 codes (unpacked, 0..15): steps on the signed magnitude index."""
    def idx(c):
        c = np.asarray(c, dtype=np.int64)
        mag = c & 0x7
        return np.where(c & 0x8, -mag, mag)
    d = np.abs(idx(gpu) - idx(ref))
    return {"ok": bool((d <= max_steps).all()), "max_steps": int(d.max(initial=0)),
            "frac_exact": float((d == 0).mean()) if d.size else 1.0, "n_bad": int((d > max_steps).sum()),
            "n": int(d.size)}


def check_rounding(gpu_values: np.ndarray, exact: np.ndarray, fmt: Format, rel_tol: float = NEAR_MIDPOINT_REL,
                   abs_tol: float = 0.0) -> Dict[str, float]:
    """Round-to-nearest-even discipline of rounded outputs.

    ``gpu_values`` are the implementation's outputs decoded to doubles,
    ``exact`` the exact values they round.  Every output must equal the
    correctly rounded exact value (``round_to_format``), or be its other
    neighbour with the exact value within ``max(rel_tol |v|, abs_tol)`` of the
    midpoint between the two.
    """
    g = np.asarray(gpu_values, dtype=np.float64)
    v = np.asarray(exact, dtype=np.float64)
    ref = round_to_format(v, fmt)
    diff = g != ref  # -0.0 == 0.0
    lo, hi = np.minimum(g, ref), np.maximum(g, ref)
    near = (v >= lo) & (v <= hi) & (np.abs(v - (lo + hi) / 2) <= np.maximum(rel_tol * np.abs(v), abs_tol))
    bad = diff & ~near
    return {"ok": bool(not bad.any()), "n_bad": int(bad.sum()), "n_near_midpoint_other_side": int((diff & near).sum()),
            "n": int(g.size)}
