"""Seeded synthetic inputs for the row-normalization workloads.

This module is shared by the tests, the benchmark and the smoke check, and it
feeds both sides of every parity comparison: the HIP library and the CPU
oracle receive the very same bits.  It holds none of the normalization's
arithmetic: it only draws random numbers, applies the outlier recipe, and
rounds the draws to their storage dtype with a library cast.

Storage convention (used by both sides):
  * ``"bf16"`` tensors are ``numpy.uint16`` arrays holding bfloat16 bit patterns;
  * ``"f32"`` tensors are ``numpy.float32`` arrays.

Recipe for one workload (seed ``s``):
  1. ``SeedSequence(s).spawn(5)`` gives one child stream per tensor, in the
     fixed order x, residual, weight, outlier mask of x, outlier mask of the
     residual (children are spawned even when a tensor is absent, so a stream
     never shifts when another tensor is added or removed);
  2. each stream is a ``numpy.random.Generator(PCG64(child))``; a tensor of
     shape ``[rows, hidden]`` is drawn as float32 standard normals, row by row
     in row-major order, then scaled by the std and shifted by the mean
     (``N(m, s)`` is read as mean m and standard deviation s);
  3. outliers (when the workload has them): an independent uniform draw per
     element from the mask stream; elements whose draw is below the outlier
     fraction are multiplied by the outlier factor;
  4. the float32 values are rounded to bfloat16 with torch's CPU cast
     (round to nearest even) when the storage dtype is bf16.

Drawing rows ``[r0, r0 + n)`` alone (``row_range``) reproduces exactly those
rows of the full tensor, so a large workload can be checked on sampled rows
without materializing it twice.

Partial-input workloads (``PartialsWorkload``): partial k is drawn like x
from ``SeedSequence([s, k + 1]).spawn(5)`` (stream x, outlier mask stream of
x); the residual and the weight come from ``SeedSequence(s)`` as above.
By default the partials are plain draws (general inputs).  The optional
``exact_sum`` recipe narrows them: every bf16-valued input of the sum (the
partials, and a bf16 residual) has each |value| below 2^-7 replaced by +0
after the storage rounding, and f32 partials are first rounded to bfloat16
values (kept in float32 storage).  Every nonzero term then lies in
[2^-7, 2^5) for the distributions used here (the tests check this), so every
float32 prefix sum of up to 8 such terms is exact.  It is kept as one extra
test case: inputs on which even a plain float32 sum in any order is exact.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Dist",
    "RowNormWorkload",
    "QKNormWorkload",
    "ActWorkload",
    "PartialsWorkload",
    "generate_act",
    "generate_partials",
    "WORKLOADS",
    "generate_rownorm",
    "generate_qknorm",
    "draw_tensor",
    "f32_to_bf16_bits",
]

# Stream order inside SeedSequence(seed).spawn(N_STREAMS).
STREAM_X, STREAM_RES, STREAM_W, STREAM_MASK_X, STREAM_MASK_RES = range(5)
N_STREAMS = 5


@dataclass(frozen=True)
class Dist:
    """Normal distribution N(mean, std) with an optional outlier recipe."""

    mean: float = 0.0
    std: float = 1.0
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0


@dataclass(frozen=True)
class RowNormWorkload:
    """Fused residual-add + RMSNorm over ``rows`` rows of length ``hidden``."""

    name: str
    kind: str  # "decode" or "prefill": what the workload models, not a kernel choice
    rows: int
    hidden: int
    x_dtype: str
    res_dtype: Optional[str]  # None: no residual stream
    w_dtype: str
    out_dtype: str  # "bf16", "f32" or "fp8_e4m3fn"
    x_dist: Dist
    res_dist: Optional[Dist]
    w_dist: Dist
    weight_plus_one: bool
    eps: float
    description: str = ""

    def with_rows(self, rows: int) -> "RowNormWorkload":
        return replace(self, rows=rows)

    def with_hidden(self, hidden: int) -> "RowNormWorkload":
        return replace(self, hidden=hidden)


@dataclass(frozen=True)
class QKNormWorkload:
    """Per-head RMSNorm of Q (and optionally K) over ``head_dim``."""

    name: str
    tokens: int
    num_q_heads: int
    num_k_heads: int
    head_dim: int
    dtype: str
    w_dtype: str
    x_dist: Dist
    w_dist: Dist
    weight_plus_one: bool
    eps: float
    description: str = ""

    def with_tokens(self, tokens: int) -> "QKNormWorkload":
        return replace(self, tokens=tokens)


@dataclass(frozen=True)
class ActWorkload:
    """SiLU-and-mul over rows of a merged gate/up projection ``[rows, 2 d]``."""

    name: str
    rows: int
    d: int
    x_dtype: str
    out_dtype: str
    x_dist: Dist
    description: str = ""

    def with_rows(self, rows: int) -> "ActWorkload":
        return replace(self, rows=rows)


@dataclass(frozen=True)
class PartialsWorkload:
    """Fused add+RMSNorm whose x is the sum of ``num_partials`` tensors."""

    name: str
    rows: int
    hidden: int
    num_partials: int
    x_dtype: str               # dtype of every partial
    res_dtype: Optional[str]
    w_dtype: str
    out_dtype: str
    part_dist: Dist
    res_dist: Optional[Dist]
    w_dist: Dist
    weight_plus_one: bool
    eps: float
    exact_sum: bool = False    # the optional recipe above that makes float32 sums exact
    description: str = ""

    def with_rows(self, rows: int) -> "PartialsWorkload":
        return replace(self, rows=rows)


N01 = Dist(0.0, 1.0)
W_N1 = Dist(1.0, 0.1)

WORKLOADS: Dict[str, object] = {
    "decode_8x1024": RowNormWorkload(
        name="decode_8x1024", kind="decode", rows=8, hidden=1024,
        x_dtype="bf16", res_dtype="bf16", w_dtype="bf16", out_dtype="bf16",
        x_dist=N01, res_dist=N01, w_dist=W_N1, weight_plus_one=False, eps=1e-6,
        description="decode fused add+RMSNorm, 8 x 1024 bf16, w ~ N(1,0.1), eps 1e-6",
    ),
    "decode_256x4096": RowNormWorkload(
        name="decode_256x4096", kind="decode", rows=256, hidden=4096,
        x_dtype="bf16", res_dtype="bf16", w_dtype="bf16", out_dtype="bf16",
        x_dist=N01, res_dist=N01, w_dist=Dist(0.0, 0.02), weight_plus_one=True, eps=1e-5,
        description="decode batch, 256 x 4096 bf16, (1+w) weight form with w ~ N(0,0.02), eps 1e-5",
    ),
    "prefill_16384x8192": RowNormWorkload(
        name="prefill_16384x8192", kind="prefill", rows=16384, hidden=8192,
        x_dtype="bf16", res_dtype="f32", w_dtype="bf16", out_dtype="bf16",
        x_dist=N01, res_dist=Dist(0.0, 4.0), w_dist=W_N1, weight_plus_one=False, eps=1e-6,
        description="prefill, 16384 x 8192, bf16 x, f32 residual stream ~ N(0,4) in and out, bf16 out",
    ),
    "qknorm_4096x32x128": QKNormWorkload(
        name="qknorm_4096x32x128", tokens=4096, num_q_heads=32, num_k_heads=0, head_dim=128,
        dtype="bf16", w_dtype="bf16", x_dist=N01, w_dist=W_N1, weight_plus_one=False, eps=1e-6,
        description="per-head QK-norm, 4096 tokens x 32 heads x head_dim 128 bf16, no residual",
    ),
    "prefill_fp8_8192x7168": RowNormWorkload(
        name="prefill_fp8_8192x7168", kind="prefill", rows=8192, hidden=7168,
        x_dtype="bf16", res_dtype="bf16", w_dtype="bf16", out_dtype="fp8_e4m3fn",
        x_dist=Dist(0.0, 1.0, 0.01, 20.0), res_dist=Dist(0.0, 1.0, 0.01, 20.0), w_dist=W_N1,
        weight_plus_one=False, eps=1e-6,
        description="prefill with fp8 e4m3fn out + per-row scale amax/448, 8192 x 7168 bf16, "
                    "1% outliers x20 on x and residual",
    ),
    "silu_mul_8192x14336": ActWorkload(
        name="silu_mul_8192x14336", rows=8192, d=14336, x_dtype="bf16", out_dtype="bf16", x_dist=N01,
        description="SwiGLU silu(gate) * up, 8192 tokens, merged gate/up projection 2 x 14336 bf16 "
                    "~ N(0,1), bf16 out",
    ),
    "partials_8x2048x8192": PartialsWorkload(
        name="partials_8x2048x8192", rows=2048, hidden=8192, num_partials=8,
        x_dtype="bf16", res_dtype="f32", w_dtype="bf16", out_dtype="bf16",
        part_dist=Dist(0.0, 0.5), res_dist=Dist(0.0, 4.0), w_dist=W_N1, weight_plus_one=False, eps=1e-6,
        description="sum of 8 bf16 partials ~ N(0,0.5) (one GPU's 2048-token share of an 8-way "
                    "tensor-parallel reduce-scatter) + f32 residual ~ N(0,4) + RMSNorm, 8192 wide, bf16 out",
    ),
    "partials_decode_8x64x8192": PartialsWorkload(
        name="partials_decode_8x64x8192", rows=64, hidden=8192, num_partials=8,
        x_dtype="bf16", res_dtype="f32", w_dtype="bf16", out_dtype="bf16",
        part_dist=Dist(0.0, 0.5), res_dist=Dist(0.0, 4.0), w_dist=W_N1, weight_plus_one=False, eps=1e-6,
        description="decode: 8 bf16 partials of a 64-token batch summed (the local arithmetic of a one-shot "
                    "all-reduce over 8 GPUs) + f32 residual + RMSNorm, 8192 wide, bf16 out",
    ),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with torch's CPU cast; return the bits."""
    import torch  # local import: torch is only needed for this storage cast

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _children(seed: int, salt: Optional[int] = None):
    entropy = seed if salt is None else [seed, salt]
    return np.random.SeedSequence(entropy).spawn(N_STREAMS)


def draw_tensor(seed: int, stream: int, mask_stream: Optional[int], shape: Tuple[int, int],
                dist: Dist, dtype: str, row_range: Optional[Tuple[int, int]] = None,
                salt: Optional[int] = None) -> np.ndarray:
    """Draw one ``[rows, cols]`` tensor (or a row range of it) following the recipe above
    (``salt``: the second entropy word of a partial's seed sequence)."""
    rows, cols = shape
    r0, r1 = (0, rows) if row_range is None else row_range
    if not (0 <= r0 <= r1 <= rows):
        raise ValueError(f"row range {row_range} outside [0, {rows}]")
    kids = _children(seed, salt)
    gen = np.random.Generator(np.random.PCG64(kids[stream]))
    n = (r1 - r0) * cols
    if r0:
        _skip_normals(gen, r0 * cols)
    vals = gen.standard_normal(n, dtype=np.float32)
    vals *= np.float32(dist.std)
    vals += np.float32(dist.mean)
    if dist.outlier_frac > 0.0:
        if mask_stream is None:
            raise ValueError("outliers need a mask stream")
        mgen = np.random.Generator(np.random.PCG64(kids[mask_stream]))
        if r0:
            _skip_uniforms(mgen, r0 * cols)
        mask = mgen.random(n, dtype=np.float64) < dist.outlier_frac
        vals[mask] *= np.float32(dist.outlier_mult)
    vals = vals.reshape(r1 - r0, cols)
    if dtype == "bf16":
        return f32_to_bf16_bits(vals)
    if dtype == "f32":
        return vals
    raise ValueError(f"unsupported storage dtype {dtype!r}")


def _skip_normals(gen: np.random.Generator, count: int, chunk: int = 1 << 24) -> None:
    # float32 normals use a variable number of raw draws (ziggurat), so a row
    # offset cannot be jumped to: draw and discard instead.
    while count > 0:
        k = min(chunk, count)
        gen.standard_normal(k, dtype=np.float32)
        count -= k


def _skip_uniforms(gen: np.random.Generator, count: int, chunk: int = 1 << 24) -> None:
    while count > 0:
        k = min(chunk, count)
        gen.random(k, dtype=np.float64)
        count -= k


def generate_rownorm(wl: RowNormWorkload, seed: int = 0,
                     row_range: Optional[Tuple[int, int]] = None) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of a fused add+RMSNorm workload: ``x``, ``residual`` (or None), ``weight``.

    The weight is a ``[1, hidden]`` draw returned as a 1-D array.
    """
    shape = (wl.rows, wl.hidden)
    x = draw_tensor(seed, STREAM_X, STREAM_MASK_X, shape, wl.x_dist, wl.x_dtype, row_range)
    res = None
    if wl.res_dtype is not None:
        res = draw_tensor(seed, STREAM_RES, STREAM_MASK_RES, shape, wl.res_dist, wl.res_dtype, row_range)
    w = draw_tensor(seed, STREAM_W, None, (1, wl.hidden), wl.w_dist, wl.w_dtype)[0]
    return {"x": x, "residual": res, "weight": w}


def generate_qknorm(wl: QKNormWorkload, seed: int = 0) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of a QK-norm workload: ``q`` [tokens, nq, D], ``k`` [tokens, nk, D] or None, weights [D]."""
    D = wl.head_dim
    q = draw_tensor(seed, STREAM_X, None, (wl.tokens, wl.num_q_heads * D), wl.x_dist, wl.dtype)
    q = q.reshape(wl.tokens, wl.num_q_heads, D)
    k = None
    if wl.num_k_heads:
        k = draw_tensor(seed, STREAM_RES, None, (wl.tokens, wl.num_k_heads * D), wl.x_dist, wl.dtype)
        k = k.reshape(wl.tokens, wl.num_k_heads, D)
    qw = draw_tensor(seed, STREAM_W, None, (1, D), wl.w_dist, wl.w_dtype)[0]
    kw = draw_tensor(seed, STREAM_MASK_X, None, (1, D), wl.w_dist, wl.w_dtype)[0]
    return {"q": q, "k": k, "q_weight": qw, "k_weight": kw}


def generate_act(wl: ActWorkload, seed: int = 0, row_range: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """Input ``x`` [rows, 2 d] of a SiLU-and-mul workload (stream x, outliers on the x mask stream)."""
    return draw_tensor(seed, STREAM_X, STREAM_MASK_X, (wl.rows, 2 * wl.d), wl.x_dist, wl.x_dtype, row_range)


EXACT_SUM_FLUSH = 2.0 ** -7  # |value| below this becomes +0 under the exact-sum recipe


def _flush_small_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns with |value| < EXACT_SUM_FLUSH replaced by +0 (exponent field test, no arithmetic)."""
    biased_exp = (bits >> 7) & 0xFF
    small = biased_exp < 127 - 7  # |v| < 2^-7
    out = bits.copy()
    out[small] = 0
    return out


def generate_partials(wl: PartialsWorkload, seed: int = 0,
                      row_range: Optional[Tuple[int, int]] = None) -> Dict[str, object]:
    """Inputs of a partial-input workload: ``partials`` (a list of ``num_partials``
    [rows, hidden] tensors), ``residual`` (or None) and ``weight`` [hidden]."""
    shape = (wl.rows, wl.hidden)
    parts = []
    for k in range(wl.num_partials):
        if wl.exact_sum:
            p = draw_tensor(seed, STREAM_X, STREAM_MASK_X, shape, wl.part_dist, "bf16", row_range, salt=k + 1)
            p = _flush_small_bf16(p)
            if wl.x_dtype == "f32":
                p = (p.astype(np.uint32) << 16).view(np.float32)
        else:
            p = draw_tensor(seed, STREAM_X, STREAM_MASK_X, shape, wl.part_dist, wl.x_dtype, row_range, salt=k + 1)
        parts.append(p)
    res = None
    if wl.res_dtype is not None:
        res = draw_tensor(seed, STREAM_RES, STREAM_MASK_RES, shape, wl.res_dist, wl.res_dtype, row_range)
        if wl.exact_sum and wl.res_dtype == "bf16":
            res = _flush_small_bf16(res)
    w = draw_tensor(seed, STREAM_W, None, (1, wl.hidden), wl.w_dist, wl.w_dtype)[0]
    return {"partials": parts, "residual": res, "weight": w}
