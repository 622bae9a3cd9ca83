"""CPU oracle for fused residual-add + RMSNorm over rows, per-head QK-norm, and
per-row fp8 e4m3fn output quantization.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module.  The HIP library never uses
it, and it shares no code, header, table or helper with the HIP library: the
only thing both sides share is the seeded input generator (``workloads``).

Everything is computed in IEEE double precision from the exact values of the
stored input bits, one plain step per line, with no blocking, fusion or
reordering beyond what the definition states.

Source of the definition
------------------------
"CuTeDSL at Perplexity" (Perplexity blog), section "QK Norm":
  * the kernel listing ``_qk_norm_kernel`` computes, for each row (one head
    of one token), the f32 sum of squares of the row, ``rms = rsqrt(sum /
    head_dim + EPS)``, and ``(w + WEIGHT_BIAS) * (x * rms)`` cast back to the
    element type;
  * the prose formula in the same section drops the rsqrt and the weight
    bias; it is read as garbled and the listing is taken as the definition;
  * ``WEIGHT_BIAS`` selects the plain weight ``w`` (bias 0) or the ``1 + w``
    form (bias 1) -- the page's "Inference at Perplexity" section names the
    weight bias of RMS norm as a compile-time knob;
  * each (token, head) row of Q uses the Q weight and of K the K weight; the
    weight is indexed by the position inside the head and shared by all heads.

Readings where the pages are silent (each listed with its reason in the
design notes):
  * residual add: the pages never show one.  ``h = round_res(x + residual)``
    is written as the updated residual, and the norm is taken over that
    rounded ``h`` (the stored residual stream is the canonical value);
  * eps is the float32 value the library receives (its argument is a C float);
  * the final cast rounds to nearest, ties to even;
  * fp8 output: OCP E4M3FN (max 448), per-row ``scale = amax / 448`` in
    float32 with ``amax = max |y|`` over the row, codes ``= RNE(y / scale)``
    saturated to +-448; an all-zero row has scale 0 and all-zero codes.

Pins (all run with ``pytest -m "not gpu"``):
  * ``round_to_format`` / ``bf16_*`` / ``f32`` rounding: exhaustive and
    random checks against torch's CPU casts and numpy's IEEE float32
    arithmetic (tests/test_oracle_codecs.py);
  * ``e4m3fn_*``: all 256 codes against the OCP FP8 specification's landmark
    values (tests/golden/e4m3fn_landmarks.txt) and torch's CPU float8 cast;
  * ``residual_add``: bit-exact against numpy float32 addition and torch's
    bfloat16 addition (tests/test_oracle_codecs.py);
  * ``rmsnorm_rows``: closed forms (constant rows, zero rows, unit weights,
    the 2-element row (3, 4)), exact-rational brute force on tiny rows,
    torch's float64 ``rms_norm`` as an independent library routine, scale
    invariance and weight-bias equivalences (tests/test_oracle_rmsnorm.py);
  * ``fp8_quantize_rows``: the format's error bounds and the saturation
    invariant (tests/test_oracle_fp8.py);
  * ``qknorm``: a head-by-head Python loop over the page's (token, head)
    row order (tests/test_oracle_rmsnorm.py);
  * ``exact_sum`` / ``rmsnorm_rows_partials``: exact rational brute force
    (``fractions.Fraction``) on mixed-magnitude and adversarial terms, ties
    decided by a remainder below double precision, order independence,
    torch's float32 sum where it is exact, and the one-partial case against
    ``residual_add`` / ``rmsnorm_rows`` (tests/test_oracle_partials.py).

Partial inputs (``rmsnorm_rows_partials``): x arrives as K partial tensors
whose sum it is -- the per-rank partials that a tensor-parallel all-reduce
sums in front of the norm.  The page fuses such a local sum with the
all-reduce in one decode launch ("CuTeDSL at Perplexity", MoE
dispatch/combine, single-node tensor-parallel part).  Reading: x is the
exact sum; with a residual, h = round_res(x + residual) is one rounding of
the exact sum of all the terms; without one, the norm is taken over the
exact x.
"""

from __future__ import annotations

from dataclasses import dataclass
import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Format",
    "BF16",
    "F32",
    "E4M3FN",
    "FORMATS",
    "round_to_format",
    "bf16_decode",
    "bf16_encode",
    "e4m3fn_decode",
    "e4m3fn_encode",
    "decode",
    "encode",
    "residual_add",
    "rmsnorm_rows",
    "exact_sum",
    "rmsnorm_rows_partials",
    "fp8_scale_from_amax",
    "fp8_quantize_rows",
    "qknorm",
]


# ---------------------------------------------------------------------------
# Number formats, written from their definitions.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Format:
    """A binary floating-point format with ``precision`` significant bits.

    ``emin`` is the exponent of the smallest normal number; numbers below it
    are subnormal with a fixed quantum ``2**(emin - precision + 1)``.
    ``max_finite`` is the largest finite magnitude.  ``saturate`` selects
    what happens to a rounded magnitude above ``max_finite``: clamp to it
    (the "satfinite" conversion) or become infinity (IEEE overflow).
    """

    name: str
    precision: int
    emin: int
    max_finite: float
    saturate: bool


# IEEE 754 binary32.
F32 = Format("f32", 24, -126, float(np.finfo(np.float32).max), saturate=False)
# bfloat16: binary32 with the low 16 fraction bits dropped (8 significant bits).
BF16 = Format("bf16", 8, -126, (2.0 - 2.0 ** -7) * 2.0 ** 127, saturate=False)
# OCP 8-bit float E4M3 ("FN": finite only): 4 exponent bits, bias 7, 3 mantissa
# bits; exponent field 15 with mantissa 7 is NaN, so the largest finite value
# is 1.75 * 2**8 = 448; subnormals are m * 2**-9.  Out-of-range values saturate.
E4M3FN = Format("fp8_e4m3fn", 4, -6, 448.0, saturate=True)

FORMATS = {"f32": F32, "bf16": BF16, "fp8_e4m3fn": E4M3FN}


def round_to_format(v: np.ndarray, fmt: Format, err: Optional[np.ndarray] = None) -> np.ndarray:
    """Round ``v`` to the nearest value of ``fmt``, ties to even.

    ``v`` is an exact double, or -- when ``err`` is given -- the double
    nearest to the true value ``v + err`` (``|err|`` at most half an ulp of
    ``v``).  ``err`` only breaks exact ties in ``v``: when ``v`` sits on a
    midpoint of ``fmt`` but the true value does not, the true value lies on
    the side of ``err``.  Returns doubles holding values of ``fmt`` (or
    +-inf on IEEE overflow).
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = (v != 0) & np.isfinite(v)
    a = np.abs(v[nz])
    # Exponent of the leading bit: a = m * 2**E with 0.5 <= m < 1, so floor(log2 a) = E - 1.
    _, E = np.frexp(a)
    e = np.maximum(E - 1, fmt.emin)  # subnormals share the quantum of the smallest normal binade
    quantum = np.ldexp(1.0, e - (fmt.precision - 1))
    t = a / quantum  # exact: division by a power of two
    n = np.floor(t)
    frac = t - n
    up = frac > 0.5
    tie = frac == 0.5
    if err is not None:
        err_nz = np.asarray(err, dtype=np.float64)[nz] * np.sign(v[nz])  # error measured away from zero
        up |= tie & (err_nz > 0)
        tie &= err_nz == 0
    up |= tie & (np.fmod(n, 2.0) == 1.0)
    mag = (n + up) * quantum
    over = mag > fmt.max_finite
    mag[over] = fmt.max_finite if fmt.saturate else np.inf
    out[nz] = np.copysign(mag, v[nz])
    out[~nz] = v[~nz]  # zeros (sign kept), and non-finite values pass through
    return out


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact values as doubles.

    A bfloat16 is the upper 16 bits of an IEEE binary32 (sign, 8-bit
    exponent, 7-bit fraction).
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_encode(v: np.ndarray, err: Optional[np.ndarray] = None) -> np.ndarray:
    """Doubles -> bfloat16 bit patterns, round to nearest even (see ``round_to_format``)."""
    r = round_to_format(v, BF16, err)
    bits32 = r.astype(np.float32).view(np.uint32)  # exact: r is a bfloat16 value
    return (bits32 >> np.uint32(16)).astype(np.uint16)


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes (uint8) -> values as doubles (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, ef - 7)
    subnormal = np.ldexp(m.astype(np.float64), -9)
    val = np.where(ef == 0, subnormal, normal)
    val = np.where((ef == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """Doubles -> OCP E4M3FN codes: round to nearest even, saturate to +-448."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3fn_encode: NaN input")
    r = round_to_format(v, E4M3FN)
    a = np.abs(r)
    sign = np.signbit(r).astype(np.int64) << 7
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = E - 1
    normal = a >= 2.0 ** -6
    mant_normal = (np.ldexp(a, -e) - 1.0) * 8.0  # 3 fraction bits
    code_normal = ((e + 7) << 3) | mant_normal.astype(np.int64)
    code_sub = (a * 2.0 ** 9).astype(np.int64)  # multiples of 2**-9 below 2**-6
    mag = np.where(normal, code_normal, code_sub)
    return (sign | mag).astype(np.uint8)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (bf16 bits or float32) -> exact doubles."""
    if dtype == "bf16":
        return bf16_decode(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "fp8_e4m3fn":
        return e4m3fn_decode(a)
    raise ValueError(dtype)


def encode(v: np.ndarray, dtype: str) -> np.ndarray:
    """Doubles -> stored representation of ``dtype`` (rounded to nearest even)."""
    if dtype == "bf16":
        return bf16_encode(v)
    if dtype == "f32":
        return round_to_format(v, F32).astype(np.float32)
    if dtype == "fp8_e4m3fn":
        return e4m3fn_encode(v)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# The method.
# ---------------------------------------------------------------------------

def _two_sum(a: np.ndarray, b: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """s = fl(a + b) and the exact error e with a + b = s + e (Knuth's TwoSum)."""
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    return s, e


def residual_add(x: np.ndarray, residual: np.ndarray, res_dtype: str) -> np.ndarray:
    """Updated residual ``h = round_res(x + residual)`` (exact sum, one rounding).

    Reading (the pages have no residual add): the sum is rounded once to the
    residual dtype; that rounded value is both the residual written back and
    the input of the norm.
    """
    s, e = _two_sum(x, residual)
    return round_to_format(s, FORMATS[res_dtype], e)


def rmsnorm_rows(x: np.ndarray, weight: np.ndarray, eps: float, weight_bias: float,
                 residual: Optional[np.ndarray] = None, res_dtype: Optional[str] = None
                 ) -> Dict[str, np.ndarray]:
    """RMSNorm of each row of ``x`` (doubles, shape [rows, H]), optionally after a residual add.

    Follows "CuTeDSL at Perplexity", section "QK Norm" (the ``_qk_norm_kernel``
    listing): ``y = (w + WEIGHT_BIAS) * h * rsqrt(sum(h^2) / H + EPS)``.

    ``weight_bias`` is 0 (plain ``w``) or 1 (``1 + w``); ``eps`` is used as
    the float32 value the kernel receives.  Returns
      ``h``     -- the normalized input (the updated residual when a residual is given),
      ``inv``   -- the inverse RMS per row,
      ``y``     -- the unrounded output, shape [rows, H].
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("rows must be a 2-D array")
    H = x.shape[1]
    if residual is not None:
        h = residual_add(x, np.asarray(residual, dtype=np.float64), res_dtype)
    else:
        h = x
    eps32 = float(np.float32(eps))
    mean_square = np.sum(h * h, axis=1) / H  # squares of f32 values are exact in double
    inv = 1.0 / np.sqrt(mean_square + eps32)
    wb = np.asarray(weight, dtype=np.float64) + weight_bias
    y = wb[None, :] * h * inv[:, None]
    return {"h": h, "inv": inv, "y": y}


def exact_sum(terms: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Elementwise exact sum of equally shaped arrays of doubles.

    Returns ``(s, e)``: ``s`` is the exact sum rounded once to double and
    ``e`` the remainder (exact sum - ``s``) rounded to double, so that
    ``round_to_format(s, fmt, e)`` rounds the exact sum once to a narrower
    format (``e`` decides a tie that ``s`` alone would show).  Python's
    ``math.fsum`` computes both, element by element.  Signed zeros follow
    IEEE addition: the sum is -0 only when every term is -0.
    """
    arrs = [np.asarray(t, dtype=np.float64) for t in terms]
    if not arrs:
        raise ValueError("at least one term")
    shape = arrs[0].shape
    for a in arrs:
        if a.shape != shape:
            raise ValueError("terms must have one shape")
    cols = np.stack([a.reshape(-1) for a in arrs], axis=1)
    s = np.empty(cols.shape[0])
    e = np.empty(cols.shape[0])
    for i, row in enumerate(cols.tolist()):
        si = math.fsum(row)
        s[i] = si
        e[i] = math.fsum(row + [-si])
    all_neg_zero = np.all((cols == 0) & np.signbit(cols), axis=1)
    s[all_neg_zero] = -0.0
    return s.reshape(shape), e.reshape(shape)


def rmsnorm_rows_partials(partials: Sequence[np.ndarray], weight: np.ndarray, eps: float, weight_bias: float,
                          residual: Optional[np.ndarray] = None, res_dtype: Optional[str] = None
                          ) -> Dict[str, np.ndarray]:
    """``rmsnorm_rows`` with x given as the sum of ``partials`` (doubles, shape [rows, H] each).

    With a residual, ``h = round_res(sum_k partials[k] + residual)``: one
    rounding of the exact sum of all the terms.  Without one, the norm is
    taken over the exact sum of the partials (as a double: within 2^-53
    relative of it).  Returns what ``rmsnorm_rows`` returns.
    """
    terms = list(partials)
    if residual is not None:
        terms.append(residual)
    s, e = exact_sum(terms)
    if residual is not None:
        h = round_to_format(s, FORMATS[res_dtype], e)
    else:
        h = s
    return rmsnorm_rows(h, weight, eps, weight_bias)


def fp8_scale_from_amax(amax: np.ndarray) -> np.ndarray:
    """Per-row scale ``amax / 448`` as the IEEE float32 division of float32(amax) by 448.

    The quotient of two float32 values rounded once to double and then to
    float32 equals the correctly rounded float32 quotient (double carries
    more than twice float32's precision plus two bits).
    """
    a32 = np.asarray(amax, dtype=np.float64).astype(np.float32).astype(np.float64)
    return (a32 / 448.0).astype(np.float32)


def fp8_quantize_rows(y: np.ndarray, scale: Optional[np.ndarray] = None
                      ) -> Dict[str, np.ndarray]:
    """Per-row dynamic fp8 e4m3fn quantization of unrounded outputs ``y`` [rows, H].

    ``amax = max |y|`` per row and ``scale = amax / 448`` (float32).  Codes are
    ``RNE_e4m3fn(y / scale)``, using ``scale`` when the caller passes one (to
    judge codes against the scale another implementation actually produced),
    else the scale computed here.  A row with ``scale == 0`` gets all-zero codes.
    """
    y = np.asarray(y, dtype=np.float64)
    amax = np.max(np.abs(y), axis=1)
    own_scale = fp8_scale_from_amax(amax)
    s = own_scale if scale is None else np.asarray(scale, dtype=np.float32)
    s64 = s.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    codes = e4m3fn_encode(y / safe[:, None])
    codes[s64 == 0, :] = 0
    return {"amax": amax, "scale": own_scale, "codes": codes}


def qknorm(q: np.ndarray, k: Optional[np.ndarray], q_weight: np.ndarray,
           k_weight: Optional[np.ndarray], eps: float, weight_bias: float
           ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Per-head RMSNorm of Q [T, nq, D] and K [T, nk, D] (doubles); unrounded outputs.

    "CuTeDSL at Perplexity", section "QK Norm": every (token, head) pair is
    one row of length ``head_dim``; Q rows use ``q_weight`` and K rows use
    ``k_weight``; no residual.
    """
    def one(t, w):
        T, nh, D = t.shape
        y = rmsnorm_rows(t.reshape(T * nh, D), w, eps, weight_bias)["y"]
        return y.reshape(T, nh, D)

    qy = one(np.asarray(q, dtype=np.float64), q_weight)
    ky = None if k is None else one(np.asarray(k, dtype=np.float64), k_weight)
    return qy, ky
