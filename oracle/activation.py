"""CPU oracle for the SiLU-and-mul (SwiGLU) activation over rows.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the HIP library
shares no code with it.

Source: "Tile-Level Activation Overlap for Efficient LLM Inference" (summary
page): the MLP's SwiGLU step combines two computations (the gate projection
and the up projection) into one result, and materializing it costs 30-37% of
the time of small models; "CuTeDSL at Perplexity", section "Inference at
Perplexity", lists activation kernels in the kernel library and the
activation function as a compile-time knob.  Neither page prints a formula.
Reading: SwiGLU is the usual gated linear unit with the SiLU (Swish, beta =
1) gate,

    out[r, i] = silu(gate[r, i]) * up[r, i],   silu(g) = g / (1 + exp(-g)),

over a merged gate/up projection ``x[r, :]`` of length ``2 d`` whose first
half is the gate and second half the up projection.  Computed in float64 from
the exact input values; quantized outputs reuse the per-row, per-128 and MX
schemes of ``rownorm`` and ``blockquant``.

Pins (tests/test_oracle_activation.py): torch's float64 ``silu`` as an
independent library routine, the closed forms silu(0) = 0, silu(g) - silu(-g)
= g and the limits, and a 40-digit Decimal evaluation on sample points.
"""

from __future__ import annotations

import numpy as np

__all__ = ["silu", "silu_mul_rows"]


def silu(g: np.ndarray) -> np.ndarray:
    """g * sigmoid(g) in float64, written so that no intermediate overflows."""
    g = np.asarray(g, dtype=np.float64)
    e = np.exp(-np.abs(g))  # in (0, 1]
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g * sig


def silu_mul_rows(x: np.ndarray, d: int) -> np.ndarray:
    """SwiGLU of each row of ``x`` [rows, 2 d] (doubles): silu(x[:, :d]) * x[:, d:]."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != 2 * d:
        raise ValueError(f"rows must be [rows, {2 * d}]")
    return silu(x[:, :d]) * x[:, d:]
