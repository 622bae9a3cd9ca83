"""Moving the generator's numpy arrays to the device and results back, and
judging a fused add+RMSNorm result against the oracle.  Test code only."""

from __future__ import annotations

import numpy as np
import torch

from oracle import compare as C
from oracle import rownorm as O

TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8_e4m3fn": torch.float8_e4m3fn}


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    raise ValueError(dtype)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Stored bits/values: bf16 -> uint16 bits, f32 -> float32, fp8 -> uint8 codes."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    raise ValueError(t.dtype)


def judge_rows(inputs: dict, x_dtype: str, res_dtype, w_dtype: str, out_dtype: str, eps: float,
               weight_plus_one: bool, out: np.ndarray, res_out, scale=None, amax=None) -> dict:
    """Compare the outputs of some rows (already on the host) with the oracle.

    ``inputs`` holds the same rows of x / residual and the full weight, as the
    generator produced them.  Returns a report; ``report["ok"]`` is the verdict.
    """
    X = O.decode(inputs["x"], x_dtype)
    RES = None if inputs.get("residual") is None else O.decode(inputs["residual"], res_dtype)
    W = O.decode(inputs["weight"], w_dtype)
    ref = O.rmsnorm_rows(X, W, eps, 1.0 if weight_plus_one else 0.0, residual=RES, res_dtype=res_dtype)
    rep = {"ok": True}
    if RES is not None:
        expect = O.encode(ref["h"], res_dtype)
        same = np.array_equal(np.asarray(res_out).view(np.uint8), np.asarray(expect).view(np.uint8))
        rep["res_out_bit_exact"] = same
        rep["ok"] &= same
    if out_dtype == "bf16":
        r = C.check_bf16(out, ref["y"])
        rep["out"] = r
        rep["out_frac_rne"] = float((out == O.bf16_encode(ref["y"])).mean())
        rep["ok"] &= r["ok"]
    elif out_dtype == "f32":
        r = C.check_f32(out, ref["y"])
        rep["out"] = r
        rep["ok"] &= r["ok"]
    else:
        q = O.fp8_quantize_rows(ref["y"])
        scale = np.asarray(scale, dtype=np.float32)
        sc = C.check_f32(scale, q["scale"])
        rep["scale"] = sc
        rep["scale_frac_bit_exact"] = float((scale == q["scale"]).mean())
        rep["ok"] &= sc["ok"]
        if amax is not None:
            amax = np.asarray(amax, dtype=np.float32)
            formula = np.array_equal(scale, amax / np.float32(448.0))
            rep["scale_formula_bit_exact"] = formula
            rep["amax"] = C.check_f32(amax, q["amax"])
            rep["ok"] &= formula and rep["amax"]["ok"]
        codes_ref = O.fp8_quantize_rows(ref["y"], scale=scale)["codes"]
        cr = C.check_fp8_codes(out, codes_ref)
        rep["codes"] = cr
        rep["ok"] &= cr["ok"]
    return rep
