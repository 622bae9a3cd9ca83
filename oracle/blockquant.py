"""CPU oracle for block-scaled quantized outputs of a normalized row.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the HIP library
shares no code with it.

Source: "CuTeDSL at Perplexity" (Perplexity blog), section "Blackwell support":
the quantization schemes MXFP8 and MXFP4 (an absolute maximum over 32
elements) and FP8 block-wise scaling were added to the existing kernels.  The
pages name the schemes but do not define them; the definitions below are the
public format specifications, and the readings are stated per function:

  * FP8 block-wise (group) scaling: every group of ``group`` consecutive
    elements of a row gets its own float32 scale ``amax_g / 448`` (the per-row
    e4m3fn scheme of ``rownorm.fp8_quantize_rows`` applied per group);
  * OCP Microscaling (MX) v1.0: a block of 32 elements shares one E8M0 scale
    X = 2^(floor(log2(max |v|)) - emax_elem), with emax_elem = 8 for FP8 E4M3
    and 2 for FP4 E2M1; every element is stored as the element-format value
    nearest to v / X (ties to even), values past the element format's largest
    normal saturating to it.  Reading for blocks the specification leaves
    open: an all-zero block gets the smallest scale (E8M0 code 0, 2^-127) and
    zero codes, and the shared exponent is clamped to E8M0's range [-127, 127];
  * NVFP4 (the same section: an absolute maximum over 16 elements): E2M1
    elements, one FP8 E4M3FN scale per block of 16 and one float32 scale per
    tensor, supplied by the caller.  Reading: the two scales together map the
    block's maximum onto E2M1's largest value 6, so the block scale is the
    E4M3FN rounding of ``amax_b / (6 s_t)`` and the elements are the E2M1
    roundings of ``y / (s_b s_t)``.

Pins (tests/test_oracle_blockquant.py, tests/test_oracle_nvfp4.py): the E2M1
and E8M0 value tables of the MX specification (tests/golden/mx_landmarks.txt),
brute-force nearest-value rounding for E2M1, closed forms for power-of-two
block maxima, the top-binade invariant, format error bounds, and per-group
fp8 with one group per row equal to the (separately pinned) per-row scheme;
for NVFP4, block maxima that are exact multiples of E4M3FN values, the error
bounds of both roundings, zero, underflowing and saturating block scales,
power-of-two invariance, and planted mistakes that each fail a pin.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .rownorm import Format, e4m3fn_decode, e4m3fn_encode, fp8_scale_from_amax, round_to_format

__all__ = [
    "E2M1",
    "EMAX_ELEM",
    "e2m1_decode",
    "e2m1_encode",
    "e8m0_decode",
    "fp8_quantize_groups",
    "mx_quantize",
    "nvfp4_quantize",
    "pack_fp4",
    "unpack_fp4",
]

# OCP MX FP4 E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; no inf or
# NaN; values 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Smallest normal 1 = 2^0; subnormal
# quantum 0.5; out-of-range values saturate to 6.
E2M1 = Format("fp4_e2m1", 2, 0, 6.0, saturate=True)

# Exponent of the largest normal of each element format (MX specification).
EMAX_ELEM = {"fp8_e4m3fn": 8, "fp4_e2m1": 2}


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes (0..15) -> values as doubles."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    val = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e - 1))
    return sign * val


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Doubles -> 4-bit E2M1 codes (uint8 0..15): nearest, ties to even, saturate to 6."""
    r = round_to_format(np.asarray(v, dtype=np.float64), E2M1)
    a = np.abs(r)
    sign = np.signbit(r).astype(np.int64) << 3
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = E - 1  # floor(log2 a) for a >= 1
    normal = a >= 1.0
    mant = np.where(normal, (np.ldexp(a, -np.where(normal, e, 0)) - 1.0) * 2.0, 0.0)
    code_normal = ((e + 1) << 1) | mant.astype(np.int64)
    code_sub = (a * 2.0).astype(np.int64)  # 0 or 1 (0 or 0.5)
    return (sign | np.where(normal, code_normal, code_sub)).astype(np.uint8)


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale codes -> 2^(code - 127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes two per byte along the last axis: element 2k in the
    low nibble, element 2k + 1 in the high nibble (reading: the MX
    specification leaves the byte packing to the implementation)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _blocks(y: np.ndarray, size: int) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    if y.ndim != 2 or y.shape[1] % size:
        raise ValueError(f"rows of length {y.shape[-1]} do not split into blocks of {size}")
    return y.reshape(y.shape[0], y.shape[1] // size, size)


def fp8_quantize_groups(y: np.ndarray, group: int = 128, scale: Optional[np.ndarray] = None
                        ) -> Dict[str, np.ndarray]:
    """FP8 e4m3fn codes with one float32 scale per ``group`` consecutive elements.

    ``amax_g = max |y|`` over the group and ``scale_g = amax_g / 448``
    (float32 division of float32(amax_g)); codes are ``RNE_e4m3fn(y /
    scale_g)`` saturated, using the caller's scales when given; a zero group
    has scale 0 and zero codes.  Returns amax [rows, H/group], scale (same
    shape, float32) and codes [rows, H].
    """
    b = _blocks(y, group)
    amax = np.max(np.abs(b), axis=2)
    own = fp8_scale_from_amax(amax)
    s = own if scale is None else np.asarray(scale, dtype=np.float32)
    s64 = s.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    codes = e4m3fn_encode(b / safe[:, :, None])
    codes[s64 == 0] = 0
    return {"amax": amax, "scale": own, "codes": codes.reshape(np.asarray(y).shape)}


def mx_quantize(y: np.ndarray, elem: str, block: int = 32, shared_exp: Optional[np.ndarray] = None
                ) -> Dict[str, np.ndarray]:
    """OCP MX quantization of rows ``y`` [rows, H] into ``elem`` with E8M0 block scales.

    ``shared_exp = clamp(floor(log2(amax)) - emax_elem, -127, 127)`` per block
    (all-zero block: -127); element codes are the ``elem`` encoding of
    ``y * 2^-shared_exp`` (exact power-of-two scaling; nearest, ties to even,
    saturating).  When ``shared_exp`` is given it is used for the codes (to
    judge codes against the exponent another implementation chose).  Returns
    amax, shared_exp, scale_codes (E8M0, uint8) [rows, H/block] and codes
    [rows, H] (4-bit codes unpacked for fp4).
    """
    if elem not in EMAX_ELEM:
        raise ValueError(elem)
    b = _blocks(y, block)
    amax = np.max(np.abs(b), axis=2)
    _, E = np.frexp(np.where(amax > 0, amax, 1.0))
    own = np.where(amax > 0, np.clip((E - 1) - EMAX_ELEM[elem], -127, 127), -127).astype(np.int64)
    se = own if shared_exp is None else np.asarray(shared_exp, dtype=np.int64)
    scaled = np.ldexp(b, -se[:, :, None])
    codes = e4m3fn_encode(scaled) if elem == "fp8_e4m3fn" else e2m1_encode(scaled)
    return {"amax": amax, "shared_exp": own, "scale_codes": (own + 127).astype(np.uint8),
            "codes": codes.reshape(np.asarray(y).shape)}


def nvfp4_quantize(y: np.ndarray, tensor_scale: float, block: int = 16,
                   scale_codes: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """NVFP4 quantization of rows ``y`` [rows, H] with the per-tensor scale ``tensor_scale``.

    For each block of ``block`` consecutive elements: ``amax_b = max |y|``,
    block scale code ``s_b = RNE_e4m3fn(amax_b / (6 * s_t))`` (saturating at
    448), element codes ``RNE_e2m1(y / (decode(s_b) * s_t))`` (saturating at
    6); a block scale that rounds to zero gives zero codes.  ``s_t`` is used
    as the exact value of the float32 the caller passes.  When
    ``scale_codes`` is given it is used for the element codes (to judge codes
    against the block scales another implementation chose).  Both quotients
    are rounded once to double and then to the narrow format; a double
    rounding would need the double quotient to fall on a narrow-format
    midpoint that the exact quotient misses, which the 5- and 3-bit grids make
    vanishingly rare.  Returns amax [rows, H/block], scale_codes (uint8 E4M3FN,
    same shape) and codes [rows, H] (4-bit codes, unpacked).
    """
    st = float(np.float32(tensor_scale))
    if not (np.isfinite(st) and st > 0):
        raise ValueError("tensor_scale must be a positive finite float32")
    b = _blocks(y, block)
    amax = np.max(np.abs(b), axis=2)
    own = e4m3fn_encode(amax / (6.0 * st))
    sc = own if scale_codes is None else np.asarray(scale_codes, dtype=np.uint8)
    d = e4m3fn_decode(sc) * st
    safe = np.where(d > 0, d, 1.0)
    codes = e2m1_encode(b / safe[:, :, None])
    codes[d == 0] = 0
    return {"amax": amax, "scale_codes": own, "codes": codes.reshape(np.asarray(y).shape)}
