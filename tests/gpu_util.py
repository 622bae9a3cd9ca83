"""Judging a fused add+RMSNorm result against the oracle (and, re-exported
from ``workloads.device``, moving arrays to the device and back).  Test code
only."""

from __future__ import annotations

import numpy as np

from oracle import blockquant as BQ
from oracle import compare as C
from oracle import rownorm as O
from workloads.device import TORCH_DTYPES, to_dev, to_host  # noqa: F401  (re-exported for the tests)


def nvfp4_tensor_scale(y: np.ndarray) -> float:
    """The usual per-tensor NVFP4 scale, amax / (6 * 448), as a float32 value."""
    return float(np.float32(np.max(np.abs(y)) / (6.0 * 448.0)))


def judge_rows(inputs: dict, x_dtype: str, res_dtype, w_dtype: str, out_dtype: str, eps: float,
               weight_plus_one: bool, out: np.ndarray, res_out, scale=None, amax=None,
               scale_scheme: str = "row", tensor_scale=None) -> dict:
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
    y = ref["y"]
    rep.update(judge_y(y, out_dtype, out, scale, amax, scale_scheme, tensor_scale))
    rep["ok"] = rep["ok"] and rep.pop("y_ok")
    return rep


def judge_y(y: np.ndarray, out_dtype: str, out: np.ndarray, scale=None, amax=None,
            scale_scheme: str = "row", tensor_scale=None, f32_abs_floor: float = C.F32_ABS_FLOOR) -> dict:
    """Judge an output tensor (host bits) against the exact pre-rounding values y [rows, n]
    (``f32_abs_floor``: the absolute floor of float32 outputs, wider for SwiGLU's)."""
    rep = {"ok": True}
    if out_dtype == "bf16":
        r = C.check_bf16(out, y)
        rep["out"] = r
        rep["out_frac_rne"] = float((out == O.bf16_encode(y)).mean())
        rep["ok"] &= r["ok"]
    elif out_dtype == "f32":
        r = C.check_f32(out, y, abs_floor=f32_abs_floor)
        rep["out"] = r
        rep["ok"] &= r["ok"]
    elif scale_scheme in ("row", "group128"):
        if scale_scheme == "row":
            q = O.fp8_quantize_rows(y)
            own = lambda sc: O.fp8_quantize_rows(y, scale=sc)["codes"]  # noqa: E731
        else:
            q = BQ.fp8_quantize_groups(y, 128)
            own = lambda sc: BQ.fp8_quantize_groups(y, 128, scale=sc)["codes"]  # noqa: E731
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
        cr = C.check_fp8_codes(out, own(scale))
        rep["codes"] = cr
        rep["ok"] &= cr["ok"]
        # rounding discipline of the codes against the exact y / scale (GPU scales)
        if scale_scheme == "row":
            s64 = np.broadcast_to(scale.astype(np.float64).reshape(-1, 1), y.shape)
        else:
            s64 = np.repeat(scale.astype(np.float64).reshape(y.shape[0], -1), 128, axis=1)
        v = np.where(s64 > 0, y / np.where(s64 > 0, s64, 1.0), 0.0)
        rep["codes_rounding"] = C.check_rounding(O.e4m3fn_decode(out), v, O.E4M3FN)
        rep["ok"] &= rep["codes_rounding"]["ok"]
    elif scale_scheme == "nv16":  # NVFP4: E4M3FN block scale per 16, float32 tensor scale
        q = BQ.nvfp4_quantize(y, tensor_scale)
        sc = np.asarray(scale, dtype=np.uint8)
        # the GPU's block scale follows from its own amax exactly:
        # e4m3fn(fl32(amax / fl32(6 s_t))), nearest even, saturating
        if amax is not None:
            amax = np.asarray(amax, dtype=np.float32)
            t6 = np.float32(6.0) * np.float32(tensor_scale)
            own = O.e4m3fn_encode((amax / t6).astype(np.float32).astype(np.float64))
            rep["scale_formula_exact"] = bool(np.array_equal(own, sc))
            rep["amax"] = C.check_f32(amax, q["amax"])
            rep["ok"] &= rep["scale_formula_exact"] and rep["amax"]["ok"]
        # ... and is within one step of the oracle's
        rep["scale_codes"] = C.check_fp8_codes(sc, q["scale_codes"])
        rep["scale_frac_exact"] = float((sc == q["scale_codes"]).mean())
        rep["ok"] &= rep["scale_codes"]["ok"]
        codes_ref = BQ.nvfp4_quantize(y, tensor_scale, scale_codes=sc)["codes"]
        cr = C.check_fp4_codes(BQ.unpack_fp4(out), codes_ref)
        rep["codes"] = cr
        rep["ok"] &= cr["ok"]
        d = np.repeat(O.e4m3fn_decode(sc) * float(np.float32(tensor_scale)), 16, axis=1)
        v = np.where(d > 0, y / np.where(d > 0, d, 1.0), 0.0)
        rep["codes_rounding"] = C.check_rounding(BQ.e2m1_decode(BQ.unpack_fp4(out)), v, BQ.E2M1)
        rep["ok"] &= rep["codes_rounding"]["ok"]
    else:  # MX, E8M0 scale per 32 elements
        q = BQ.mx_quantize(y, out_dtype)
        se = np.asarray(scale, dtype=np.uint8).astype(np.int64) - 127
        emax = BQ.EMAX_ELEM[out_dtype]
        # the GPU's exponent follows from its own amax exactly ...
        if amax is not None:
            amax = np.asarray(amax, dtype=np.float32).astype(np.float64)
            _, E = np.frexp(np.where(amax > 0, amax, 1.0))
            own_se = np.where(amax > 0, np.clip(E - 1 - emax, -127, 127), -127)
            rep["exp_formula_exact"] = bool(np.array_equal(own_se, se))
            rep["amax"] = C.check_f32(amax, q["amax"])
            rep["ok"] &= rep["exp_formula_exact"] and rep["amax"]["ok"]
        # ... and matches the oracle's, except by one where the exact amax sits
        # within float32 rounding of a power of two
        d = np.abs(se - q["shared_exp"])
        near_pow2 = np.abs(np.log2(np.where(q["amax"] > 0, q["amax"], 1.0)) -
                           np.round(np.log2(np.where(q["amax"] > 0, q["amax"], 1.0)))) < 1e-5
        exp_ok = (d == 0) | ((d == 1) & near_pow2)
        rep["exp_match"] = float((d == 0).mean())
        rep["ok"] &= bool(exp_ok.all())
        codes_ref = BQ.mx_quantize(y, out_dtype, shared_exp=se)["codes"]
        if out_dtype == "fp4_e2m1":
            cr = C.check_fp4_codes(BQ.unpack_fp4(out), codes_ref)
        else:
            cr = C.check_fp8_codes(out, codes_ref)
        rep["codes"] = cr
        rep["ok"] &= cr["ok"]
        v = np.ldexp(y, -np.repeat(se, 32, axis=1))
        got = BQ.e2m1_decode(BQ.unpack_fp4(out)) if out_dtype == "fp4_e2m1" else O.e4m3fn_decode(out)
        rep["codes_rounding"] = C.check_rounding(got, v, BQ.E2M1 if out_dtype == "fp4_e2m1" else O.E4M3FN)
        rep["ok"] &= rep["codes_rounding"]["ok"]
    rep["y_ok"] = rep.pop("ok")
    return rep


def judge_partials_rows(inputs: dict, x_dtype: str, res_dtype, w_dtype: str, out_dtype: str, eps: float,
                        weight_plus_one: bool, out: np.ndarray, res_out, scale=None, amax=None,
                        ref=None, scale_scheme: str = "row", tensor_scale=None) -> dict:
    """Compare the outputs of some rows of a partial-input call with the oracle.

    ``inputs`` holds the same rows of every partial (``partials``) and of the
    residual, and the full weight.  The rules are those of ``judge_rows``: the
    updated residual is the exact sum of the partials and the residual rounded
    once (bit-exact), and the outputs are within the usual tolerances of the
    norm of that sum.  ``ref`` may pass the oracle's result for these rows,
    computed once.
    """
    parts = [O.decode(p, x_dtype) for p in inputs["partials"]]
    RES = None if inputs.get("residual") is None else O.decode(inputs["residual"], res_dtype)
    W = O.decode(inputs["weight"], w_dtype)
    bias = 1.0 if weight_plus_one else 0.0
    if ref is None:
        ref = O.rmsnorm_rows_partials(parts, W, eps, bias, residual=RES, res_dtype=res_dtype)
    rep = {"ok": True}
    if RES is not None:
        # the oracle's h is already the once-rounded exact sum: encoding it is exact
        expect = O.encode(ref["h"], res_dtype)
        same = np.asarray(res_out).view(np.uint8).reshape(-1) == np.asarray(expect).view(np.uint8).reshape(-1)
        rep["res_out_bit_exact"] = bool(same.all())
        rep["res_out_mismatches"] = int((~same).sum())
        rep["ok"] &= rep["res_out_bit_exact"]
    rep.update(judge_y(ref["y"], out_dtype, out, scale, amax, scale_scheme, tensor_scale))
    rep["ok"] = rep["ok"] and rep.pop("y_ok")
    return rep
