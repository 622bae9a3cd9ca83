"""GPU parity of the partial-input entry point (rmsnorm_fwd_partials) against the oracle.

Inputs come from ``workloads.generate_partials`` as plain draws (general
inputs), plus one case of its exact-sum recipe and hand-made rows that put
the exact sum where a float32 sum in slot order rounds differently: on or
next to a rounding midpoint, under cancellation, and across wide magnitude
spans.  The kernel must return the exact sum rounded once: the updated
residual bit-exact, the outputs to ``oracle.compare``'s tolerances, every
output scheme included.
"""

import numpy as np
import pytest
import torch

import residual_add_rmsnorm_rows_amd as R
import workloads as WL
from oracle import rownorm as O
from residual_add_rmsnorm_rows_amd import _lib as L
from tests.gpu_util import TORCH_DTYPES, judge_partials_rows, to_dev, to_host

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _wl(rows, hidden, k, x="bf16", res="f32", w="bf16", out="bf16", bias=False, exact=False, eps=1e-6,
        part_std=0.5):
    return WL.PartialsWorkload(
        name="t", rows=rows, hidden=hidden, num_partials=k, x_dtype=x, res_dtype=res, w_dtype=w, out_dtype=out,
        part_dist=WL.Dist(0.0, part_std), res_dist=None if res is None else WL.Dist(0.0, 4.0 if res == "f32" else 1.0),
        w_dist=WL.Dist(0.0, 0.02) if bias else WL.Dist(1.0, 0.1), weight_plus_one=bias, eps=eps, exact_sum=exact)


def run_partials(wl, inputs, config=None, out_into_part=None):
    parts = [to_dev(p, wl.x_dtype) for p in inputs["partials"]]
    res = None if inputs["residual"] is None else to_dev(inputs["residual"], wl.res_dtype)
    w = to_dev(inputs["weight"], wl.w_dtype)
    kw = {}
    if out_into_part is not None:
        kw["out"] = parts[out_into_part]
    r = R.fused_partials_add_rmsnorm(parts, res, w, wl.eps, weight_plus_one=wl.weight_plus_one,
                                     out_dtype=TORCH_DTYPES[wl.out_dtype], return_amax=wl.out_dtype == "fp8_e4m3fn",
                                     config=config, **kw)
    torch.cuda.synchronize()
    return r


def oracle_ref(wl, inputs):
    parts = [O.decode(p, wl.x_dtype) for p in inputs["partials"]]
    res = None if inputs["residual"] is None else O.decode(inputs["residual"], wl.res_dtype)
    return O.rmsnorm_rows_partials(parts, O.decode(inputs["weight"], wl.w_dtype), wl.eps,
                                   1.0 if wl.weight_plus_one else 0.0, residual=res, res_dtype=wl.res_dtype)


def judge(wl, inputs, r, rows=None, ref=None):
    sel = slice(None) if rows is None else rows
    sub = {"partials": [p[sel] for p in inputs["partials"]],
           "residual": None if inputs["residual"] is None else inputs["residual"][sel], "weight": inputs["weight"]}
    out = to_host(r.out)[sel]
    res_out = None if r.residual_out is None else to_host(r.residual_out)[sel]
    scale = None if r.scale is None else to_host(r.scale)[sel]
    amax = None if r.amax is None else to_host(r.amax)[sel]
    return judge_partials_rows(sub, wl.x_dtype, wl.res_dtype, wl.w_dtype, wl.out_dtype, wl.eps, wl.weight_plus_one,
                               out, res_out, scale, amax, ref=ref)


def test_workload_small():
    wl = WL.WORKLOADS["partials_8x2048x8192"].with_rows(300)
    _announce(f"partials workload 300 rows cfg={R.query_partials_config(300, 8192, 8, res_dtype='f32')}")
    inp = WL.generate_partials(wl, seed=1)
    rep = judge(wl, inp, run_partials(wl, inp))
    assert rep["ok"], rep


def test_workload_full_size_sampled():
    """2048 x 8192 with 8 partials in the selector's launch configuration; the
    oracle checks sampled rows, including the first and the last."""
    wl = WL.WORKLOADS["partials_8x2048x8192"]
    _announce(f"partials full size cfg={R.query_partials_config(wl.rows, wl.hidden, 8, res_dtype='f32')}")
    inp = WL.generate_partials(wl, seed=0)
    r = run_partials(wl, inp)
    rows = np.array([0, 1, 517, 1024, 2046, 2047])
    rep = judge(wl, inp, r, rows=rows)
    assert rep["ok"], rep



def test_block_scaled_full_size_sampled():
    """2048 x 8192 with 8 partials and MXFP4 output in the selector's launch
    configuration (16 waves x 1 vector per lane); the oracle checks sampled
    rows, including the first and the last."""
    from dataclasses import replace

    wl = replace(WL.WORKLOADS["partials_8x2048x8192"], out_dtype="fp4_e2m1")
    cfg = R.query_partials_config(wl.rows, wl.hidden, 8, res_dtype="f32", out_dtype="fp4_e2m1", scale_scheme="mx32")
    assert (cfg["waves_per_row"], cfg["vecs_per_lane"]) == (16, 1)
    _announce(f"partials full size MXFP4 cfg={cfg}")
    inp = WL.generate_partials(wl, seed=0)
    parts = [to_dev(p, wl.x_dtype) for p in inp["partials"]]
    r = R.fused_partials_add_rmsnorm(parts, to_dev(inp["residual"], wl.res_dtype), to_dev(inp["weight"], wl.w_dtype),
                                     wl.eps, out_dtype=TORCH_DTYPES["fp4_e2m1"], scale_scheme="mx32", return_amax=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 517, 1024, 2046, 2047])
    sub = {"partials": [p[rows] for p in inp["partials"]], "residual": inp["residual"][rows], "weight": inp["weight"]}
    rep = judge_partials_rows(sub, wl.x_dtype, wl.res_dtype, wl.w_dtype, "fp4_e2m1", wl.eps, wl.weight_plus_one,
                              to_host(r.out)[rows], to_host(r.residual_out)[rows], to_host(r.scale)[rows],
                              to_host(r.amax)[rows], scale_scheme="mx32")
    assert rep["ok"], rep

CASES = [  # (x, res, w, out, bias)
    ("bf16", "f32", "bf16", "bf16", False), ("bf16", "bf16", "bf16", "bf16", True),
    ("bf16", None, "bf16", "bf16", False), ("bf16", "f32", "f32", "f32", False),
    ("bf16", "bf16", "bf16", "fp8_e4m3fn", False), ("bf16", None, "f32", "fp8_e4m3fn", True),
    ("f32", "f32", "f32", "f32", False), ("f32", None, "bf16", "bf16", True), ("f32", "f32", "bf16", "fp8_e4m3fn", False),
]


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("x,res,w,out,bias", CASES)
@pytest.mark.parametrize("rows,hidden", [(37, 1000), (5, 4096)])
def test_dtype_combinations(x, res, w, out, bias, k, rows, hidden):
    wl = _wl(rows, hidden, k, x, res, w, out, bias)
    _announce(f"partials k={k} {x}/{res}/{w}->{out} bias={bias} {rows}x{hidden}")
    inp = WL.generate_partials(wl, seed=7 + k)
    rep = judge(wl, inp, run_partials(wl, inp))
    assert rep["ok"], rep


def _variants(hidden, vec):
    nvec = -(-hidden // vec)
    for W in range(1, 17):
        for NV in (1, 2):
            if 64 * W * NV >= nvec and (NV == 1 or 64 * W < nvec or W == 1):
                yield W, NV


@pytest.mark.parametrize("k", [2, 4, 8])
@pytest.mark.parametrize("x,out", [("bf16", "bf16"), ("bf16", "fp8_e4m3fn"), ("f32", "f32")])
def test_every_launch_variant(k, x, out):
    hidden = 3000 if x == "bf16" else 1500
    wl = _wl(41, hidden, k, x, "f32", "bf16", out)
    inp = WL.generate_partials(wl, seed=3)
    ref = oracle_ref(wl, inp)
    for i, (W, NV) in enumerate(_variants(hidden, 8 if x == "bf16" else 4)):
        for grid in (41, 13) if i % 4 == 0 else (41,):
            cfg = L.LaunchConfig()
            cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = 0, W, NV, grid
            _announce(f"partials variant k={k} {x}->{out} W={W} NV={NV} grid={grid}")
            rep = judge(wl, inp, run_partials(wl, inp, config=cfg), ref=ref)
            assert rep["ok"], (W, NV, grid, rep)


@pytest.mark.parametrize("x,k,res,out", [("f32", 8, "f32", "f32"), ("f32", 8, "f32", "bf16"), ("f32", 3, None, "f32"),
                                         ("bf16", 5, "bf16", "bf16"), ("bf16", 8, "f32", "bf16"),
                                         ("f32", 4, "f32", "fp8_e4m3fn"), ("bf16", 6, "bf16", "fp8_e4m3fn")])
def test_wide_float32_partials(x, k, res, out):
    """Partials N(0, 1) in float32: their float32 sum in slot order rounds at
    most additions, so only an exact sum gives the oracle's bits."""
    wl = _wl(64, 2048, k, x, res, "bf16", out, part_std=1.0)
    _announce(f"partials general {x} k={k} res={res} out={out}")
    inp = WL.generate_partials(wl, seed=11)
    rep = judge(wl, inp, run_partials(wl, inp))
    assert rep["ok"], rep


def test_exact_sum_recipe():
    """The narrowed inputs of the exact-sum recipe (every float32 prefix sum exact)."""
    wl = _wl(64, 8192, 8, exact=True)
    _announce("partials exact-sum recipe")
    inp = WL.generate_partials(wl, seed=12)
    rep = judge(wl, inp, run_partials(wl, inp))
    assert rep["ok"], rep


def _bf16_bits(vals):
    bits = np.asarray(vals, dtype=np.float32).view(np.uint32)
    assert (bits & 0xFFFF == 0).all(), "hazard terms must be bfloat16 values"
    return (bits >> 16).astype(np.uint16)


# Rows of (partials..., residual) terms, each chosen so that the exact sum and
# a float32 sum in slot order round differently (or to exercise signed zeros):
HAZARDS_F32_RES = [
    # exact sum just above the float32 midpoint 1 + 2^-24: rounds up to 1 + 2^-23
    ([1.0, 2.0 ** -24, 2.0 ** -60], 0.0),
    ([1.0, 2.0 ** -24, -(2.0 ** -60)], 0.0),          # just below it: 1
    ([1.0, 2.0 ** -24, 0.0], 0.0),                    # on it: nearest even, 1
    ([1.0 + 2.0 ** -7, 2.0 ** -24, 0.0], 2.0 ** -22),  # the residual carries a float32 bit
    ([-1.0, -(2.0 ** -24), -(2.0 ** -70)], 0.0),       # negative side, away from zero
    ([2.0 ** 60, 1.0, -(2.0 ** 60)], 0.5),             # cancellation: 1.5
    ([2.0 ** 40, 3.0, -(2.0 ** 40), 2.0 ** -30], 0.0), # 3 + 2^-30
    ([-0.0, -0.0, -0.0], -0.0),                        # every term -0: -0
    ([-0.0, 0.0, -0.0], -0.0),                         # a +0 term: +0
    ([2.0 ** 30, 2.0 ** -30, -(2.0 ** 30), 2.0 ** -36], 2.0 ** -37),  # small terms survive cancellation
]


@pytest.mark.parametrize("res_dtype", ["f32", "bf16", None])
@pytest.mark.parametrize("out,scheme", [("bf16", "row"), ("f32", "row"), ("fp8_e4m3fn", "row"), ("fp4_e2m1", "mx32")])
def test_rounding_hazards(res_dtype, out, scheme):
    """Hand-made terms where a float32 sum in slot order would round the
    updated residual (or the normalized sum) differently from the exact sum."""
    H, K = 128, 4
    rows = len(HAZARDS_F32_RES) + 2
    wl = _wl(rows, H, K, "bf16", res_dtype, "bf16", out, part_std=1.0)
    inp = WL.generate_partials(wl, seed=21)
    # one hazard per row, placed at a different column of each row; the other
    # columns keep their random draws
    for r, (terms, rv) in enumerate(HAZARDS_F32_RES):
        col = (r * 37) % H
        terms = list(terms) + [-0.0] * (K - len(terms))  # -0 leaves every sum unchanged
        for k, t in enumerate(_bf16_bits(terms)):
            inp["partials"][k][r, col] = t
        if res_dtype == "f32":
            inp["residual"][r, col] = np.float32(rv)
        elif res_dtype == "bf16":
            inp["residual"][r, col] = _bf16_bits([rv])[0]
    # the bf16 residual's own midpoint hazard: 1 + 2^-8 (+ a tiny term) in the last rows
    if res_dtype == "bf16":
        for r, tiny in ((rows - 2, 2.0 ** -40), (rows - 1, 0.0)):
            for k, t in enumerate(_bf16_bits([1.0, 2.0 ** -8, tiny, -0.0])):
                inp["partials"][k][r, 5] = t
            inp["residual"][r, 5] = 0
    _announce(f"partials rounding hazards res={res_dtype} out={out}/{scheme}")
    ref = oracle_ref(wl, inp)
    ts = None
    if scheme == "nv16":
        from tests.gpu_util import nvfp4_tensor_scale
        ts = nvfp4_tensor_scale(ref["y"])
    parts = [to_dev(p, "bf16") for p in inp["partials"]]
    res = None if res_dtype is None else to_dev(inp["residual"], res_dtype)
    r = R.fused_partials_add_rmsnorm(parts, res, to_dev(inp["weight"], "bf16"), wl.eps,
                                     out_dtype=TORCH_DTYPES[out], scale_scheme=scheme, tensor_scale=ts,
                                     return_amax=out in ("fp8_e4m3fn", "fp4_e2m1"))
    torch.cuda.synchronize()
    rep = judge_partials_rows(inp, "bf16", res_dtype, "bf16", out, wl.eps, False, to_host(r.out),
                              None if r.residual_out is None else to_host(r.residual_out),
                              None if r.scale is None else to_host(r.scale),
                              None if r.amax is None else to_host(r.amax), ref=ref, scale_scheme=scheme,
                              tensor_scale=ts)
    assert rep["ok"], rep


@pytest.mark.parametrize("rows", [1, 32, 256])
def test_decode_shapes(rows):
    wl = WL.WORKLOADS["partials_8x2048x8192"].with_rows(rows)
    _announce(f"partials decode rows={rows} cfg={R.query_partials_config(rows, 8192, 8, res_dtype='f32')}")
    inp = WL.generate_partials(wl, seed=rows)
    rep = judge(wl, inp, run_partials(wl, inp))
    assert rep["ok"], rep


def test_out_in_place_over_a_partial():
    wl = _wl(33, 2048, 4, "bf16", "bf16", "bf16", "bf16")
    _announce("partials in place")
    inp = WL.generate_partials(wl, seed=5)
    r = run_partials(wl, inp, out_into_part=2)
    rep = judge(wl, inp, r)
    assert rep["ok"], rep


def test_single_partial_and_zero_partials_match_the_single_input_kernel():
    """[x] and [x, 0, 0] give the bits of fused_add_rmsnorm(x)."""
    wl = _wl(20, 4096, 1, "bf16", "f32", "bf16", "fp8_e4m3fn")
    _announce("partials vs single input")
    inp = WL.generate_partials(wl, seed=2)
    x = to_dev(inp["partials"][0], "bf16")
    res = to_dev(inp["residual"], "f32")
    w = to_dev(inp["weight"], "bf16")
    ref = R.fused_add_rmsnorm(x, res, w, wl.eps, out_dtype=torch.float8_e4m3fn)
    z = torch.zeros_like(x)
    for parts in ([x], [x, z, z]):
        got = R.fused_partials_add_rmsnorm(parts, res, w, wl.eps, out_dtype=torch.float8_e4m3fn)
        torch.cuda.synchronize()
        assert torch.equal(got.out.view(torch.uint8), ref.out.view(torch.uint8))
        assert torch.equal(got.residual_out, ref.residual_out)
        assert torch.equal(got.scale, ref.scale)


def test_zero_rows_and_all_zero_partials():
    wl = _wl(6, 1024, 3, "bf16", None, "bf16", "fp8_e4m3fn")
    inp = WL.generate_partials(wl, seed=9)
    for p in inp["partials"]:
        p[2] = 0
    _announce("partials zero row")
    r = run_partials(wl, inp)
    rep = judge(wl, inp, r)
    assert rep["ok"], rep
    assert float(r.scale[2]) == 0.0 and not to_host(r.out)[2].any()
    empty = [torch.empty(0, 1024, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    e = R.fused_partials_add_rmsnorm(empty, None, to_dev(inp["weight"], "bf16"), 1e-6)
    assert e.out.shape == (0, 1024)


BLOCK_SCHEMES = [("fp8_e4m3fn", "group128"), ("fp8_e4m3fn", "mx32"), ("fp4_e2m1", "mx32"), ("fp4_e2m1", "nv16")]


@pytest.mark.parametrize("k", [2, 3, 8])
@pytest.mark.parametrize("out,scheme", BLOCK_SCHEMES)
@pytest.mark.parametrize("x,res,rows,hidden", [("bf16", "f32", 37, 1024), ("bf16", "bf16", 5, 4096),
                                               ("f32", "f32", 9, 2048)])
def test_block_scaled_outputs(k, out, scheme, x, res, rows, hidden):
    """Partial inputs with every block-scaled output (per-128 fp8, MXFP8, MXFP4, NVFP4)."""
    from tests.gpu_util import nvfp4_tensor_scale

    wl = _wl(rows, hidden, k, x, res, "bf16", out)
    _announce(f"partials k={k} {x}/{res} -> {out}/{scheme} {rows}x{hidden}")
    inp = WL.generate_partials(wl, seed=31 + k)
    ref = oracle_ref(wl, inp)
    ts = nvfp4_tensor_scale(ref["y"]) if scheme == "nv16" else None
    parts = [to_dev(p, x) for p in inp["partials"]]
    r = R.fused_partials_add_rmsnorm(parts, to_dev(inp["residual"], res), to_dev(inp["weight"], "bf16"), wl.eps,
                                     out_dtype=TORCH_DTYPES[out], scale_scheme=scheme, tensor_scale=ts,
                                     return_amax=True)
    torch.cuda.synchronize()
    rep = judge_partials_rows(inp, x, res, "bf16", out, wl.eps, False, to_host(r.out), to_host(r.residual_out),
                              to_host(r.scale), to_host(r.amax), ref=ref, scale_scheme=scheme, tensor_scale=ts)
    assert rep["ok"], rep


@pytest.mark.parametrize("out,scheme", BLOCK_SCHEMES)
def test_block_scaled_every_launch_variant(out, scheme):
    from tests.gpu_util import nvfp4_tensor_scale

    wl = _wl(21, 2048, 8, "bf16", "f32", "bf16", out)
    inp = WL.generate_partials(wl, seed=41)
    ref = oracle_ref(wl, inp)
    ts = nvfp4_tensor_scale(ref["y"]) if scheme == "nv16" else None
    parts = [to_dev(p, "bf16") for p in inp["partials"]]
    res, w = to_dev(inp["residual"], "f32"), to_dev(inp["weight"], "bf16")
    for W, NV in _variants(2048, 8):
        cfg = L.LaunchConfig()
        cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = 0, W, NV, 21
        _announce(f"partials block variant {out}/{scheme} W={W} NV={NV}")
        r = R.fused_partials_add_rmsnorm(parts, res, w, wl.eps, out_dtype=TORCH_DTYPES[out], scale_scheme=scheme,
                                         tensor_scale=ts, return_amax=True, config=cfg)
        torch.cuda.synchronize()
        rep = judge_partials_rows(inp, "bf16", "f32", "bf16", out, wl.eps, False, to_host(r.out),
                                  to_host(r.residual_out), to_host(r.scale), to_host(r.amax), ref=ref,
                                  scale_scheme=scheme, tensor_scale=ts)
        assert rep["ok"], (W, NV, rep)
