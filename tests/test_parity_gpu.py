"""GPU parity: the HIP library (called through the C ABI) against the CPU oracle.

Inputs come from the seeded generator in ``workloads``; both sides see the
same bits.  Tolerances are those of ``oracle.compare``: bf16 outputs within
one bf16 ulp, f32 within 1e-5 relative, fp8 codes within one step, the
updated residual bit-exact, fp8 scales within 1e-5 relative with the
``amax / 448`` formula bit-exact on the GPU's own amax.
"""

import itertools

import numpy as np
import pytest
import torch

import residual_add_rmsnorm_rows_amd as R
import workloads as WL
from oracle import compare as C
from oracle import rownorm as O
from residual_add_rmsnorm_rows_amd import _lib as L
from oracle import activation as ACT
from tests.gpu_util import TORCH_DTYPES, judge_rows, judge_y, nvfp4_tensor_scale, to_dev, to_host

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def oracle_y(wl, inputs):
    """The oracle's unrounded outputs y for the given rows (to pick an NVFP4 tensor scale)."""
    X = O.decode(inputs["x"], wl.x_dtype)
    RES = None if inputs.get("residual") is None else O.decode(inputs["residual"], wl.res_dtype)
    return O.rmsnorm_rows(X, O.decode(inputs["weight"], wl.w_dtype), wl.eps, 1.0 if wl.weight_plus_one else 0.0,
                          residual=RES, res_dtype=wl.res_dtype)["y"]


def run_rownorm(wl, inputs, config=None, inplace=False, scale_scheme="row", tensor_scale=None):
    x = to_dev(inputs["x"], wl.x_dtype)
    res = None if inputs["residual"] is None else to_dev(inputs["residual"], wl.res_dtype)
    w = to_dev(inputs["weight"], wl.w_dtype)
    kw = {}
    if inplace:
        if TORCH_DTYPES[wl.out_dtype] == x.dtype:
            kw["out"] = x
        if res is not None:
            kw["residual_out"] = res
    r = R.fused_add_rmsnorm(x, res, w, wl.eps, weight_plus_one=wl.weight_plus_one,
                            out_dtype=TORCH_DTYPES[wl.out_dtype],
                            return_amax=wl.out_dtype in ("fp8_e4m3fn", "fp4_e2m1"),
                            scale_scheme=scale_scheme, tensor_scale=tensor_scale, config=config, **kw)
    torch.cuda.synchronize()
    return r


def judge(wl, inputs, r, rows=None, scale_scheme="row", tensor_scale=None):
    sel = slice(None) if rows is None else rows
    sub = {"x": inputs["x"][sel], "residual": None if inputs["residual"] is None else inputs["residual"][sel],
           "weight": inputs["weight"]}
    out = to_host(r.out)[sel]
    res_out = None if r.residual_out is None else to_host(r.residual_out)[sel]
    scale = None if r.scale is None else to_host(r.scale)[sel]
    amax = None if r.amax is None else to_host(r.amax)[sel]
    return judge_rows(sub, wl.x_dtype, wl.res_dtype, wl.w_dtype, wl.out_dtype, wl.eps, wl.weight_plus_one,
                      out, res_out, scale, amax, scale_scheme=scale_scheme, tensor_scale=tensor_scale)


ROW_WORKLOADS = ["decode_8x1024", "decode_256x4096", "prefill_16384x8192", "prefill_fp8_8192x7168"]


@pytest.mark.parametrize("name", ROW_WORKLOADS)
def test_workload_parity_small(name):
    """Each fused add+RMSNorm workload at its hidden size, with few enough rows
    for the oracle to check every element (ragged row count, several tiles)."""
    wl = WL.WORKLOADS[name]
    wl = wl.with_rows(min(wl.rows, 300))
    _announce(f"{name} rows={wl.rows} hidden={wl.hidden}")
    inputs = WL.generate_rownorm(wl, seed=0)
    rep = judge(wl, inputs, run_rownorm(wl, inputs))
    print(rep)
    assert rep["ok"], rep


@pytest.mark.parametrize("name,out_dtype,scheme", [("decode_8x1024", None, "row"), ("decode_256x4096", None, "row"),
                                                    ("prefill_fp8_8192x7168", None, "row"),
                                                    ("prefill_fp8_8192x7168", "fp8_e4m3fn", "mx32"),
                                                    ("prefill_fp8_8192x7168", "fp4_e2m1", "nv16")])
def test_prepared_call(name, out_dtype, scheme):
    """prepare_fused_add_rmsnorm (the library's call record, rmsnorm_fwd_call):
    every call re-reads its buffers, so new inputs copied into them between
    calls give the oracle's outputs for those inputs, bit-identical to
    fused_add_rmsnorm's on the same inputs."""
    from dataclasses import replace

    wl = WL.WORKLOADS[name]
    if out_dtype is not None:
        wl = replace(wl, out_dtype=out_dtype)
    wl = wl.with_rows(min(wl.rows, 64))
    quant = wl.out_dtype in ("fp8_e4m3fn", "fp4_e2m1")
    _announce(f"prepared call {name} out={wl.out_dtype}/{scheme} rows={wl.rows}")
    seeds = [WL.generate_rownorm(wl, seed=s) for s in (0, 1, 2)]
    for inputs in seeds[1:]:
        inputs["weight"] = seeds[0]["weight"]  # the weight buffer is part of the prepared call
    ts = nvfp4_tensor_scale(oracle_y(wl, seeds[0])) if scheme == "nv16" else None
    x = to_dev(seeds[0]["x"], wl.x_dtype)
    res = to_dev(seeds[0]["residual"], wl.res_dtype)
    w = to_dev(seeds[0]["weight"], wl.w_dtype)
    call = R.prepare_fused_add_rmsnorm(x, res, w, wl.eps, weight_plus_one=wl.weight_plus_one,
                                       out_dtype=TORCH_DTYPES[wl.out_dtype], return_amax=quant, scale_scheme=scheme,
                                       tensor_scale=ts)
    for inputs in seeds[1:] + seeds[:1]:
        x.copy_(to_dev(inputs["x"], wl.x_dtype))
        res.copy_(to_dev(inputs["residual"], wl.res_dtype))
        r = call()
        torch.cuda.synchronize()
        rep = judge(wl, inputs, r, scale_scheme=scheme, tensor_scale=ts)
        assert rep["ok"], rep
        ref = run_rownorm(wl, inputs, scale_scheme=scheme, tensor_scale=ts)
        for a, b in ((r.out, ref.out), (r.residual_out, ref.residual_out), (r.scale, ref.scale),
                     (r.amax, ref.amax)):
            assert (a is None) == (b is None)
            if a is not None:
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("name", ["prefill_16384x8192", "prefill_fp8_8192x7168", "decode_256x4096"])
def test_workload_parity_full_size_sampled(name):
    """Full-size workload in the benchmark's launch configuration (the
    selector's); the oracle checks sampled rows, including the first and last."""
    wl = WL.WORKLOADS[name]
    _announce(f"{name} full size rows={wl.rows} hidden={wl.hidden} cfg={R.query_config(wl.rows, wl.hidden, x_dtype=wl.x_dtype, res_dtype=wl.res_dtype, out_dtype=wl.out_dtype)}")
    inputs = WL.generate_rownorm(wl, seed=0)
    r = run_rownorm(wl, inputs)
    rng = np.random.default_rng(123)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(wl.rows - 4, wl.rows),
                                     rng.integers(0, wl.rows, 56)]))
    rep = judge(wl, inputs, r, rows)
    print(rep)
    assert rep["ok"], rep


def test_share_of_eight_full_size():
    """The headline's 2048-row share over 8 GPUs (a bench line), all rows, in the
    selector's launch configuration."""
    wl = WL.WORKLOADS["prefill_16384x8192"].with_rows(2048)
    _announce(f"prefill 2048 x 8192 cfg={R.query_config(wl.rows, wl.hidden, res_dtype='f32')}")
    inputs = WL.generate_rownorm(wl, seed=0)
    r = run_rownorm(wl, inputs)
    rows = np.arange(0, wl.rows, 7)
    rep = judge(wl, inputs, r, rows)
    assert rep["ok"], rep


def test_qknorm_workload_full():
    wl = WL.WORKLOADS["qknorm_4096x32x128"]
    _announce(f"{wl.name} tokens={wl.tokens} heads={wl.num_q_heads} D={wl.head_dim} "
              f"cfg={R.query_qknorm_config(wl.tokens, wl.num_q_heads, 0, wl.head_dim)}")
    inp = WL.generate_qknorm(wl, seed=0)
    q = to_dev(inp["q"].reshape(wl.tokens, -1), wl.dtype).view(wl.tokens, wl.num_q_heads, wl.head_dim)
    qw = to_dev(inp["q_weight"], wl.w_dtype)
    q_out, _ = R.qk_norm(q, None, qw, None, wl.eps, weight_plus_one=wl.weight_plus_one, inplace=False)
    torch.cuda.synchronize()
    qy, _ = O.qknorm(O.decode(inp["q"], wl.dtype), None, O.decode(inp["q_weight"], wl.w_dtype), None, wl.eps,
                     1.0 if wl.weight_plus_one else 0.0)
    rep = C.check_bf16(to_host(q_out), qy)
    print(rep)
    assert rep["ok"], rep
    # in place (the page's form) gives the same bits
    R.qk_norm(q, None, qw, None, wl.eps, inplace=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(q), to_host(q_out))


DTYPE_COMBOS = [
    (x, res, w, out, b)
    for x in ("bf16", "f32")
    for res in ((None, "bf16", "f32") if x == "bf16" else (None, "f32"))
    for w in ("bf16", "f32")
    for out in ("bf16", "f32", "fp8_e4m3fn")
    for b in (False, True)
]


@pytest.mark.parametrize("x,res,w,out,b", DTYPE_COMBOS)
@pytest.mark.parametrize("rows", [37, 300])
def test_every_dtype_combination(x, res, w, out, b, rows):
    H = 1000
    wl = WL.RowNormWorkload(name="combo", kind="test", rows=rows, hidden=H, x_dtype=x, res_dtype=res, w_dtype=w,
                            out_dtype=out, x_dist=WL.Dist(0, 1, 0.01, 20.0), res_dist=WL.Dist(0, 2),
                            w_dist=WL.Dist(0.0 if b else 1.0, 0.1), weight_plus_one=b, eps=1e-5)
    _announce(f"combo x={x} res={res} w={w} out={out} plus_one={b} rows={rows} H={H}")
    inputs = WL.generate_rownorm(wl, seed=7)
    rep = judge(wl, inputs, run_rownorm(wl, inputs))
    assert rep["ok"], rep


def _variants(hidden, vec):
    nvec = hidden // vec
    for W in range(1, 17):
        for NV in (1, 2, 4, 8):
            if 64 * W > (512 if NV == 8 else 1024):
                continue
            if 64 * W * NV >= nvec and 64 * W * (NV // 2 if NV > 1 else 0) < nvec + 64 * W:
                yield W, NV


@pytest.mark.parametrize("name", ["decode_8x1024", "decode_256x4096"])
def test_decode_one_wave_per_row(name):
    """The one-wave64-per-row decode shape (whole row in one wave's registers,
    no LDS, no barrier) on the decode workloads, next to the selector's shape."""
    wl = WL.WORKLOADS[name]
    inputs = WL.generate_rownorm(wl, seed=0)
    vec = 8
    nv = next(n for n in (1, 2, 4, 8) if 64 * n * vec >= wl.hidden)
    cfg = L.LaunchConfig()
    cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = L.RN_KERNEL_ROWS, 1, nv, wl.rows
    _announce(f"{name} one wave per row, {nv} vectors per lane")
    r1 = run_rownorm(wl, inputs, config=cfg)
    rep = judge(wl, inputs, r1)
    assert rep["ok"], rep
    r2 = run_rownorm(wl, inputs)
    # both shapes sum in float32 in different orders: equal within the same bar, and
    # the updated residual (no reduction involved) bit-identical
    assert np.array_equal(to_host(r1.residual_out), to_host(r2.residual_out))
    assert judge(wl, inputs, r2)["ok"]


@pytest.mark.parametrize("hidden,x,out", [(8192, "bf16", "bf16"), (7168, "bf16", "fp8_e4m3fn"),
                                          (1000, "bf16", "bf16"), (1000, "f32", "f32"), (64, "bf16", "bf16"),
                                          (8, "bf16", "fp8_e4m3fn"), (3072, "f32", "bf16")])
def test_every_launch_variant(hidden, x, out):
    """Every (waves per row, vectors per lane) variant that covers the row, with
    a workgroup per row and with fewer workgroups than rows (row striding)."""
    res = "f32"
    wl = WL.RowNormWorkload(name="variant", kind="test", rows=67, hidden=hidden, x_dtype=x, res_dtype=res,
                            w_dtype="bf16", out_dtype=out, x_dist=WL.Dist(0, 1), res_dist=WL.Dist(0, 4),
                            w_dist=WL.Dist(1, 0.1), weight_plus_one=False, eps=1e-6)
    inputs = WL.generate_rownorm(wl, seed=3)
    vec = 8 if x == "bf16" else 4
    n = 0
    for W, NV in _variants(hidden, vec):
        for grid in (wl.rows, 5):
            cfg = L.LaunchConfig()
            cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = L.RN_KERNEL_ROWS, W, NV, grid
            _announce(f"variant H={hidden} x={x} out={out} W={W} NV={NV} grid={grid}")
            rep = judge(wl, inputs, run_rownorm(wl, inputs, config=cfg))
            assert rep["ok"], (W, NV, grid, rep)
            n += 1
    assert n > 0


BLOCK_CASES = [
    # scheme, out dtype, x, residual
    ("group128", "fp8_e4m3fn", "bf16", "bf16"), ("group128", "fp8_e4m3fn", "bf16", "f32"),
    ("group128", "fp8_e4m3fn", "f32", "f32"), ("group128", "fp8_e4m3fn", "bf16", None),
    ("mx32", "fp8_e4m3fn", "bf16", "bf16"), ("mx32", "fp8_e4m3fn", "bf16", "f32"),
    ("mx32", "fp8_e4m3fn", "f32", None), ("mx32", "fp4_e2m1", "bf16", "bf16"),
    ("mx32", "fp4_e2m1", "bf16", "f32"), ("mx32", "fp4_e2m1", "f32", "f32"), ("mx32", "fp4_e2m1", "bf16", None),
    ("nv16", "fp4_e2m1", "bf16", "bf16"), ("nv16", "fp4_e2m1", "bf16", "f32"), ("nv16", "fp4_e2m1", "f32", "f32"),
    ("nv16", "fp4_e2m1", "bf16", None),
]


@pytest.mark.parametrize("scheme,out,x,res", BLOCK_CASES)
@pytest.mark.parametrize("rows,hidden", [(37, 1024), (300, 7168), (5, 8192)])
def test_block_scaled_outputs(scheme, out, x, res, rows, hidden):
    """fp8 with per-128 scales, OCP MX (fp8 / fp4 with E8M0 per 32) and NVFP4
    (fp4 with E4M3FN per 16 and the usual tensor scale amax / 2688): scales,
    exponents and codes against the oracle, zero groups included."""
    wl = WL.RowNormWorkload(name="block", kind="test", rows=rows, hidden=hidden, x_dtype=x, res_dtype=res,
                            w_dtype="bf16", out_dtype=out, x_dist=WL.Dist(0, 1, 0.01, 20.0),
                            res_dist=None if res is None else WL.Dist(0, 1, 0.01, 20.0),
                            w_dist=WL.Dist(1, 0.1), weight_plus_one=False, eps=1e-6)
    _announce(f"block scheme={scheme} out={out} x={x} res={res} rows={rows} H={hidden}")
    inputs = WL.generate_rownorm(wl, seed=12)
    # one all-zero group of 128 in row 0
    if x == "bf16":
        inputs["x"][0, 128:256] = 0
    else:
        inputs["x"][0, 128:256] = 0.0
    if res is not None:
        inputs["residual"][0, 128:256] = 0
    ts = nvfp4_tensor_scale(oracle_y(wl, inputs)) if scheme == "nv16" else None
    r = run_rownorm(wl, inputs, scale_scheme=scheme, tensor_scale=ts)
    rep = judge(wl, inputs, r, scale_scheme=scheme, tensor_scale=ts)
    assert rep["ok"], rep
    sc = to_host(r.scale)
    if scheme == "mx32":
        assert np.all(sc[0, 4:8] == 0)  # 2^-127 for the zero blocks
    elif scheme == "nv16":
        assert np.all(sc[0, 8:16] == 0)  # scale 0 for the zero blocks
    else:
        assert np.all(sc[0, 1] == 0)


@pytest.mark.parametrize("x,res,w,out,scheme,hidden,shape", [
    ("bf16", None, "bf16", "bf16", "row", 2816, (3, 2)), ("bf16", None, "bf16", "bf16", "row", 6656, (7, 2)),
    ("bf16", None, "bf16", "fp8_e4m3fn", "row", 4352, (3, 4)), ("bf16", None, "bf16", "fp4_e2m1", "mx32", 6656, (4, 4)),
    ("bf16", None, "bf16", "fp4_e2m1", "nv16", 2816, (2, 4)), ("f32", None, "bf16", "bf16", "row", 4352, (5, 4)),
    ("f32", None, "bf16", "f32", "row", 2816, (6, 2)), ("f32", "f32", "bf16", "fp8_e4m3fn", "group128", 3328, (7, 2)),
    ("bf16", "bf16", "bf16", "fp8_e4m3fn", "row", 6656, (7, 2)),
    ("bf16", "bf16", "bf16", "fp8_e4m3fn", "group128", 4352, (5, 2)),
    ("bf16", "bf16", "bf16", "fp4_e2m1", "mx32", 6656, (7, 2)), ("bf16", "bf16", "bf16", "fp4_e2m1", "nv16", 6144, (8, 2)),
    ("bf16", None, "f32", "bf16", "row", 7168, (7, 2)), ("bf16", None, "f32", "fp8_e4m3fn", "row", 5120, (3, 4)),
    ("bf16", "bf16", "f32", "bf16", "row", 6656, (4, 4)),
])
def test_selector_more_vectors_rule(x, res, w, out, scheme, hidden, shape):
    """The selector's 2- and 4-vectors-per-lane shapes for rows without a
    residual and for quantized outputs with a residual of the x dtype (rows
    whose last wave is partly idle), in the selector's own launch
    configuration."""
    rows = 300
    cfg = R.query_config(rows, hidden, x_dtype=x, res_dtype=res, w_dtype=w, out_dtype=out, scale_scheme=scheme,
                         num_cus=0)
    _announce(f"more-vectors rule x={x} res={res} w={w} out={out}/{scheme} {rows}x{hidden} cfg={cfg}")
    assert (cfg["waves_per_row"], cfg["vecs_per_lane"]) == shape
    wl = WL.RowNormWorkload(name="rule", kind="test", rows=rows, hidden=hidden, x_dtype=x, res_dtype=res,
                            w_dtype=w, out_dtype=out, x_dist=WL.Dist(0, 1, 0.01, 20.0),
                            res_dist=None if res is None else WL.Dist(0, 1, 0.01, 20.0),
                            w_dist=WL.Dist(1, 0.1), weight_plus_one=False, eps=1e-6)
    inputs = WL.generate_rownorm(wl, seed=14)
    ts = nvfp4_tensor_scale(oracle_y(wl, inputs)) if scheme == "nv16" else None
    r = run_rownorm(wl, inputs, scale_scheme=scheme, tensor_scale=ts)
    rep = judge(wl, inputs, r, scale_scheme=scheme, tensor_scale=ts)
    assert rep["ok"], rep


@pytest.mark.parametrize("scheme,out", [("group128", "fp8_e4m3fn"), ("mx32", "fp4_e2m1"), ("mx32", "fp8_e4m3fn"),
                                        ("nv16", "fp4_e2m1")])
def test_block_scaled_every_launch_variant(scheme, out):
    H = 7168
    wl = WL.RowNormWorkload(name="bv", kind="test", rows=19, hidden=H, x_dtype="bf16", res_dtype="f32",
                            w_dtype="bf16", out_dtype=out, x_dist=WL.Dist(0, 1), res_dist=WL.Dist(0, 4),
                            w_dist=WL.Dist(1, 0.1), weight_plus_one=True, eps=1e-6)
    inputs = WL.generate_rownorm(wl, seed=13)
    ts = nvfp4_tensor_scale(oracle_y(wl, inputs)) if scheme == "nv16" else None
    n = 0
    for W, NV in _variants(H, 8):
        for grid in (wl.rows, 4):
            cfg = L.LaunchConfig()
            cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = L.RN_KERNEL_ROWS, W, NV, grid
            _announce(f"block variant {scheme} {out} W={W} NV={NV} grid={grid}")
            r = run_rownorm(wl, inputs, config=cfg, scale_scheme=scheme, tensor_scale=ts)
            rep = judge(wl, inputs, r, scale_scheme=scheme, tensor_scale=ts)
            assert rep["ok"], (W, NV, grid, rep)
            n += 1
    assert n > 0


@pytest.mark.parametrize("scheme,out", [("group128", "fp8_e4m3fn"), ("mx32", "fp4_e2m1"), ("nv16", "fp4_e2m1")])
def test_block_scaled_full_size_sampled(scheme, out):
    wl = WL.WORKLOADS["prefill_fp8_8192x7168"]
    wl = WL.RowNormWorkload(**{**wl.__dict__, "out_dtype": out})
    _announce(f"block full size {scheme} {out} cfg={R.query_config(wl.rows, wl.hidden, res_dtype=wl.res_dtype, out_dtype=out, scale_scheme=scheme)}")
    inputs = WL.generate_rownorm(wl, seed=0)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(3), np.arange(wl.rows - 3, wl.rows), rng.integers(0, wl.rows, 40)]))
    sub = {"x": inputs["x"][rows], "residual": inputs["residual"][rows], "weight": inputs["weight"]}
    # NVFP4: the tensor scale from the sampled rows' amax (any positive value is a valid input)
    ts = nvfp4_tensor_scale(oracle_y(wl, sub)) if scheme == "nv16" else None
    r = run_rownorm(wl, inputs, scale_scheme=scheme, tensor_scale=ts)
    rep = judge(wl, inputs, r, rows, scale_scheme=scheme, tensor_scale=ts)
    assert rep["ok"], rep


@pytest.mark.parametrize("factor", [2.0 ** -6, 2.0 ** 14])
def test_nvfp4_tensor_scale_extremes(factor):
    """A tensor scale far below the usual one (block scales saturate at 448,
    elements at 6) and far above it (block scales in E4M3FN's subnormal range
    and rounding to zero)."""
    wl = WL.RowNormWorkload(name="nvx", kind="test", rows=64, hidden=2048, x_dtype="bf16", res_dtype="bf16",
                            w_dtype="bf16", out_dtype="fp4_e2m1", x_dist=WL.Dist(0, 1, 0.01, 20.0),
                            res_dist=WL.Dist(0, 1), w_dist=WL.Dist(1, 0.1), weight_plus_one=False, eps=1e-6)
    inputs = WL.generate_rownorm(wl, seed=14)
    ts = float(np.float32(nvfp4_tensor_scale(oracle_y(wl, inputs)) * factor))
    _announce(f"nvfp4 tensor scale x{factor}: {ts}")
    r = run_rownorm(wl, inputs, scale_scheme="nv16", tensor_scale=ts)
    rep = judge(wl, inputs, r, scale_scheme="nv16", tensor_scale=ts)
    assert rep["ok"], rep
    sc = to_host(r.scale)
    if factor < 1:
        assert np.mean(sc == 0x7E) > 0.5  # mostly saturated block scales
    else:
        assert np.mean(sc < 0x08) > 0.5 and np.any(sc == 0)  # subnormal and zero block scales


@pytest.mark.parametrize("nbytes", [16, 8192, 3 * 8192 + 48, 1 << 22])
def test_reference_copy(nbytes):
    _announce(f"reference copy {nbytes} bytes")
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    L.check(L.lib().rn_launch_copy(src.data_ptr(), dst.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert int(dst[nbytes:].count_nonzero()) == 0  # nothing written past the end


def test_edge_cases():
    base = WL.WORKLOADS["decode_8x1024"]
    # rows == 0: no launch, empty outputs
    _announce("rows=0")
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    r = R.fused_add_rmsnorm(x, x.clone(), torch.ones(1024, dtype=torch.bfloat16, device="cuda"), 1e-6)
    assert r.out.shape == (0, 1024)
    # one row; largest hidden; smallest hidden
    for rows, H in ((1, 1024), (3, 32768), (5, 8), (2, 16384)):
        _announce(f"rows={rows} H={H}")
        wl = base.with_rows(rows).with_hidden(H)
        inputs = WL.generate_rownorm(wl, seed=11)
        rep = judge(wl, inputs, run_rownorm(wl, inputs))
        assert rep["ok"], (rows, H, rep)
    # all-zero rows: y = 0 exactly; fp8 scale 0, codes 0
    _announce("zero rows")
    for out in ("bf16", "fp8_e4m3fn"):
        wl = WL.WORKLOADS["prefill_fp8_8192x7168"].with_rows(4)
        wl = WL.RowNormWorkload(**{**wl.__dict__, "out_dtype": out})
        inputs = WL.generate_rownorm(wl, seed=0)
        inputs["x"][1:3] = 0
        inputs["residual"][1:3] = 0
        r = run_rownorm(wl, inputs)
        o = to_host(r.out)
        assert np.all(o[1:3] == 0)
        if out == "fp8_e4m3fn":
            assert np.all(r.scale.cpu().numpy()[1:3] == 0)
        rep = judge(wl, inputs, r)
        assert rep["ok"], rep
    # eps = 0 on non-zero rows
    _announce("eps=0")
    wl = WL.RowNormWorkload(**{**base.__dict__, "eps": 0.0})
    inputs = WL.generate_rownorm(wl, seed=2)
    rep = judge(wl, inputs, run_rownorm(wl, inputs))
    assert rep["ok"], rep


@pytest.mark.parametrize("name", ["decode_256x4096", "prefill_16384x8192"])
def test_in_place(name):
    wl = WL.WORKLOADS[name].with_rows(64)
    _announce(f"in place {name}")
    inputs = WL.generate_rownorm(wl, seed=5)
    r = run_rownorm(wl, inputs, inplace=True)
    rep = judge(wl, inputs, r)
    assert rep["ok"], rep


QK_CASES = [
    # dtype, w dtype, head_dim, tokens, nq, nk, plus_one, strided
    ("bf16", "bf16", 128, 4096, 32, 0, False, False),
    ("bf16", "bf16", 128, 333, 32, 8, False, True),
    ("bf16", "bf16", 64, 77, 16, 4, True, False),
    ("bf16", "bf16", 256, 51, 8, 2, False, True),
    ("bf16", "f32", 128, 19, 5, 3, True, False),
    ("f32", "f32", 64, 41, 7, 1, False, False),
    ("f32", "bf16", 128, 29, 4, 4, True, True),
    ("f32", "f32", 256, 13, 3, 2, False, False),
    ("bf16", "bf16", 128, 1, 1, 0, False, False),
]


@pytest.mark.parametrize("dt,wdt,D,T,nq,nk,b,strided", QK_CASES)
def test_qknorm_parity(dt, wdt, D, T, nq, nk, b, strided):
    _announce(f"qknorm dt={dt} w={wdt} D={D} T={T} nq={nq} nk={nk} plus_one={b} strided={strided}")
    qwl = WL.QKNormWorkload(name="qk", tokens=T, num_q_heads=nq, num_k_heads=nk, head_dim=D, dtype=dt, w_dtype=wdt,
                            x_dist=WL.Dist(0, 2), w_dist=WL.Dist(0.0 if b else 1.0, 0.1), weight_plus_one=b,
                            eps=1e-6)
    inp = WL.generate_qknorm(qwl, seed=9)
    qh = to_dev(inp["q"].reshape(T, -1), dt)
    kh = None if nk == 0 else to_dev(inp["k"].reshape(T, -1), dt)
    if strided:
        # Q and K as views of one fused [T, (nq + 2 nk) * D] QKV buffer
        qkv = torch.zeros((T, (nq + 2 * nk) * D), dtype=qh.dtype, device="cuda")
        qkv[:, : nq * D] = qh
        if nk:
            qkv[:, nq * D: (nq + nk) * D] = kh
        q = qkv[:, : nq * D].view(T, nq, D)
        k = None if nk == 0 else qkv[:, nq * D: (nq + nk) * D].view(T, nk, D)
    else:
        q = qh.view(T, nq, D)
        k = None if nk == 0 else kh.view(T, nk, D)
    qw = to_dev(inp["q_weight"], wdt)
    kw = None if nk == 0 else to_dev(inp["k_weight"], wdt)
    before = None if not strided else to_host(qkv[:, (nq + nk) * D:]).copy()
    R.qk_norm(q, k, qw, kw, qwl.eps, weight_plus_one=b, inplace=True)
    torch.cuda.synchronize()
    qy, ky = O.qknorm(O.decode(inp["q"], dt), None if nk == 0 else O.decode(inp["k"], dt),
                      O.decode(inp["q_weight"], wdt), None if nk == 0 else O.decode(inp["k_weight"], wdt),
                      qwl.eps, 1.0 if b else 0.0)
    chk = C.check_bf16 if dt == "bf16" else C.check_f32
    rq = chk(to_host(q.reshape(T, -1) if not strided else q.contiguous()).reshape(qy.shape), qy)
    assert rq["ok"], rq
    if nk:
        rk = chk(to_host(k.contiguous()).reshape(ky.shape), ky)
        assert rk["ok"], rk
    if strided:  # the V part of the fused buffer is untouched
        assert np.array_equal(to_host(qkv[:, (nq + nk) * D:]), before)


@pytest.mark.parametrize("dt,D,T,nq,nk", [("bf16", 128, 77, 32, 8), ("bf16", 64, 50, 9, 3), ("bf16", 256, 21, 5, 2),
                                          ("f32", 128, 33, 6, 2), ("f32", 256, 9, 3, 1)])
def test_every_qknorm_launch_variant(dt, D, T, nq, nk):
    """Every (heads per lane group, workgroup size) variant of the per-head kernel."""
    qwl = WL.QKNormWorkload(name="qkv", tokens=T, num_q_heads=nq, num_k_heads=nk, head_dim=D, dtype=dt,
                            w_dtype=dt, x_dist=WL.Dist(0, 1), w_dist=WL.Dist(1, 0.1), weight_plus_one=False,
                            eps=1e-6)
    inp = WL.generate_qknorm(qwl, seed=21)
    q = to_dev(inp["q"].reshape(T, -1), dt).view(T, nq, D)
    k = to_dev(inp["k"].reshape(T, -1), dt).view(T, nk, D)
    qw, kw = to_dev(inp["q_weight"], dt), to_dev(inp["k_weight"], dt)
    qy, ky = O.qknorm(O.decode(inp["q"], dt), O.decode(inp["k"], dt), O.decode(inp["q_weight"], dt),
                      O.decode(inp["k_weight"], dt), qwl.eps, 0.0)
    chk = C.check_bf16 if dt == "bf16" else C.check_f32
    for rpl in (1, 2, 4):
        for block in (64, 128, 256):
            _announce(f"qknorm variant dt={dt} D={D} T={T} nq={nq} nk={nk} rpl={rpl} block={block}")
            cfg = L.LaunchConfig()
            cfg.kernel, cfg.rows_per_lane, cfg.block_threads = L.RN_KERNEL_HEADS, rpl, block
            qo, ko = R.qk_norm(q, k, qw, kw, qwl.eps, inplace=False, config=cfg)
            torch.cuda.synchronize()
            rq = chk(to_host(qo).reshape(qy.shape), qy)
            rk = chk(to_host(ko).reshape(ky.shape), ky)
            assert rq["ok"] and rk["ok"], (rpl, block, rq, rk)


def test_qknorm_equals_rmsnorm_on_reshaped_rows():
    """GPU vs GPU: per-head norm of [T, H, D] == row norm of [T*H, D] (same bits)."""
    _announce("qknorm vs rmsnorm reshape")
    wl = WL.WORKLOADS["qknorm_4096x32x128"].with_tokens(512)
    inp = WL.generate_qknorm(wl, seed=1)
    q = to_dev(inp["q"].reshape(wl.tokens, -1), "bf16").view(wl.tokens, wl.num_q_heads, wl.head_dim)
    w = to_dev(inp["q_weight"], "bf16")
    a, _ = R.qk_norm(q, None, w, None, wl.eps, inplace=False)
    b = R.rmsnorm(q.reshape(-1, wl.head_dim), w, wl.eps).out
    torch.cuda.synchronize()
    assert np.array_equal(to_host(a).reshape(-1), to_host(b).reshape(-1))


def test_deterministic():
    wl = WL.WORKLOADS["prefill_fp8_8192x7168"].with_rows(512)
    _announce("determinism")
    inputs = WL.generate_rownorm(wl, seed=4)
    r1 = run_rownorm(wl, inputs)
    r2 = run_rownorm(wl, inputs)
    assert np.array_equal(to_host(r1.out), to_host(r2.out))
    assert np.array_equal(r1.scale.cpu().numpy(), r2.scale.cpu().numpy())


def test_empty_kernel_launch():
    L.check(L.lib().rn_launch_empty(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()


ACT_OUTS = [("bf16", "row"), ("f32", "row"), ("fp8_e4m3fn", "row"), ("fp8_e4m3fn", "group128"),
            ("fp8_e4m3fn", "mx32"), ("fp4_e2m1", "mx32"), ("fp4_e2m1", "nv16")]


def act_tensor_scale(wl, x_np, scale_scheme, rows=None):
    """NVFP4: the usual tensor scale from the oracle's outputs (of the given rows); else None."""
    if scale_scheme != "nv16":
        return None
    sel = slice(None) if rows is None else rows
    return nvfp4_tensor_scale(ACT.silu_mul_rows(O.decode(x_np[sel], wl.x_dtype), wl.d))


def run_act(wl, x_np, scale_scheme, config=None, tensor_scale=None):
    x = to_dev(x_np, wl.x_dtype)
    r = R.silu_mul(x, out_dtype=TORCH_DTYPES[wl.out_dtype], scale_scheme=scale_scheme,
                   return_amax=wl.out_dtype in ("fp8_e4m3fn", "fp4_e2m1"), tensor_scale=tensor_scale,
                   config=config)
    torch.cuda.synchronize()
    return r


def judge_act(wl, x_np, r, scale_scheme, rows=None, tensor_scale=None):
    sel = slice(None) if rows is None else rows
    y = ACT.silu_mul_rows(O.decode(x_np[sel], wl.x_dtype), wl.d)
    scale = None if r.scale is None else to_host(r.scale)[sel]
    amax = None if r.amax is None else to_host(r.amax)[sel]
    rep = judge_y(y, wl.out_dtype, to_host(r.out)[sel], scale, amax, scale_scheme, tensor_scale,
                  f32_abs_floor=C.SILU_F32_ABS_FLOOR)
    rep["ok"] = rep.pop("y_ok")
    return rep


@pytest.mark.parametrize("out,scheme", ACT_OUTS)
@pytest.mark.parametrize("x", ["bf16", "f32"])
@pytest.mark.parametrize("rows,d", [(37, 1024), (300, 3584), (3, 14336)])
def test_silu_mul_parity(out, scheme, x, rows, d):
    wl = WL.ActWorkload(name="act", rows=rows, d=d, x_dtype=x, out_dtype=out, x_dist=WL.Dist(0, 2, 0.01, 20.0))
    _announce(f"silu_mul x={x} out={out} scheme={scheme} rows={rows} d={d}")
    xn = WL.generate_act(wl, seed=17)
    if x == "bf16":
        xn[0, 256:512] = 0  # a zero group of the output (gate zero)
    else:
        xn[0, 256:512] = 0.0
    ts = act_tensor_scale(wl, xn, scheme)
    rep = judge_act(wl, xn, run_act(wl, xn, scheme, tensor_scale=ts), scheme, tensor_scale=ts)
    assert rep["ok"], rep


# (gate, up) pairs far from the usual activations: products beyond 2^64
# with a positive gate (silu(g) u close to g u), and negative gates whose
# result is small but still a normal float32.
SILU_LARGE = [(2.0 ** 33, 2.0 ** 33), (2.0 ** 40, 2.0 ** 20), (100.0, 2.0 ** 70), (10240.0, 2.0 ** 60),
              (-20.0, 2.0 ** 60), (-80.0, 2.0 ** 60), (3.5, -(2.0 ** 80)), (0.75, 2.0 ** 100), (-1.5, -(2.0 ** 90))]


@pytest.mark.parametrize("out,scheme", ACT_OUTS)
@pytest.mark.parametrize("x", ["bf16", "f32"])
def test_silu_mul_large_products(out, scheme, x):
    """|gate * up| up to 2^100: every intermediate stays finite where the result is."""
    rows, d = 3, 1024
    wl = WL.ActWorkload(name="actl", rows=rows, d=d, x_dtype=x, out_dtype=out, x_dist=WL.Dist(0, 1))
    xn = WL.generate_act(wl, seed=23)
    vals = np.array(SILU_LARGE, dtype=np.float32)  # every value is a bf16 value too
    for r in range(rows):
        cols = (np.arange(len(SILU_LARGE)) * 97 + 13 * r) % d
        if x == "bf16":
            xn[r, cols] = (vals[:, 0].view(np.uint32) >> 16).astype(np.uint16)
            xn[r, d + cols] = (vals[:, 1].view(np.uint32) >> 16).astype(np.uint16)
        else:
            xn[r, cols] = vals[:, 0]
            xn[r, d + cols] = vals[:, 1]
    _announce(f"silu_mul large products x={x} out={out} scheme={scheme}")
    ts = act_tensor_scale(wl, xn, scheme)
    rep = judge_act(wl, xn, run_act(wl, xn, scheme, tensor_scale=ts), scheme, tensor_scale=ts)
    assert rep["ok"], rep


@pytest.mark.parametrize("out,scheme", [("bf16", "row"), ("fp8_e4m3fn", "row"), ("fp4_e2m1", "mx32"),
                                        ("fp4_e2m1", "nv16")])
def test_silu_mul_every_launch_variant(out, scheme):
    d = 3584
    wl = WL.ActWorkload(name="actv", rows=23, d=d, x_dtype="bf16", out_dtype=out, x_dist=WL.Dist(0, 1))
    xn = WL.generate_act(wl, seed=18)
    ts = act_tensor_scale(wl, xn, scheme)
    n = 0
    for W, NV in _variants(d, 8):
        for grid in (wl.rows, 4):
            cfg = L.LaunchConfig()
            cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = L.RN_KERNEL_ROWS, W, NV, grid
            _announce(f"silu_mul variant out={out} W={W} NV={NV} grid={grid}")
            rep = judge_act(wl, xn, run_act(wl, xn, scheme, config=cfg, tensor_scale=ts), scheme, tensor_scale=ts)
            assert rep["ok"], (W, NV, grid, rep)
            n += 1
    assert n > 0


@pytest.mark.parametrize("out,scheme", [("bf16", "row"), ("fp8_e4m3fn", "mx32"), ("fp4_e2m1", "nv16")])
def test_silu_mul_full_size_sampled(out, scheme):
    wl = WL.WORKLOADS["silu_mul_8192x14336"]
    wl = WL.ActWorkload(**{**wl.__dict__, "out_dtype": out})
    _announce(f"silu_mul full size out={out} scheme={scheme} cfg={R.query_silu_mul_config(wl.rows, wl.d, out_dtype=out, scale_scheme=scheme)}")
    xn = WL.generate_act(wl, seed=0)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([np.arange(3), np.arange(wl.rows - 3, wl.rows), rng.integers(0, wl.rows, 30)]))
    ts = act_tensor_scale(wl, xn, scheme, rows)
    r = run_act(wl, xn, scheme, tensor_scale=ts)
    rep = judge_act(wl, xn, r, scheme, rows, tensor_scale=ts)
    assert rep["ok"], rep


def test_silu_mul_edge_cases():
    """rows == 0, the smallest and largest d, ragged d (not a multiple of 64 lanes)."""
    _announce("silu_mul rows=0")
    x = torch.empty((0, 2048), dtype=torch.bfloat16, device="cuda")
    r = R.silu_mul(x)
    assert r.out.shape == (0, 1024)
    for xd, rows, d in (("bf16", 3, 8), ("bf16", 2, 32768), ("f32", 2, 16384), ("bf16", 5, 1000), ("f32", 4, 12)):
        wl = WL.ActWorkload(name="acte", rows=rows, d=d, x_dtype=xd, out_dtype="bf16", x_dist=WL.Dist(0, 2, 0.01, 20.0))
        _announce(f"silu_mul edge x={xd} rows={rows} d={d}")
        xn = WL.generate_act(wl, seed=19)
        rep = judge_act(wl, xn, run_act(wl, xn, "row"), "row")
        assert rep["ok"], (xd, rows, d, rep)
    # unsupported sizes are refused before any launch
    with pytest.raises(R.RNError):
        R.silu_mul(torch.zeros((2, 2 * 1000), dtype=torch.bfloat16, device="cuda"),
                   out_dtype=torch.float8_e4m3fn, scale_scheme="mx32")


def test_concurrent_host_threads():
    """Entry points called from several host threads at once, each on its own
    stream (default priority): results equal the single-threaded ones bit for
    bit, and each thread's last-error message is its own."""
    import threading

    shapes = [("decode_8x1024", 8), ("decode_256x4096", 256), ("prefill_fp8_8192x7168", 96), ("prefill_16384x8192", 64)]
    jobs = []
    for name, rows in shapes:
        wl = WL.WORKLOADS[name].with_rows(rows)
        inputs = WL.generate_rownorm(wl, seed=21)
        ref = run_rownorm(wl, inputs)
        jobs.append((wl, inputs, to_host(ref.out), to_host(ref.residual_out)))
    _announce("concurrent host threads x5")
    errors, msgs = [], {}
    lib = L.lib()

    def worker(k):
        wl, inputs, ref_out, ref_res = jobs[k]
        stream = torch.cuda.Stream()  # default priority
        try:
            with torch.cuda.stream(stream):
                for i in range(20):
                    r = run_rownorm(wl, inputs)
                    if not (np.array_equal(to_host(r.out), ref_out) and np.array_equal(to_host(r.residual_out), ref_res)):
                        errors.append((k, i))
                        return
            if k == 0:  # a failing call on this thread only
                st = lib.rmsnorm_fwd(0x10000, None, 0x10000, 0x20000, None, None, 4, 1001, 1e-6, 0, None)
                msgs[k] = (st, lib.rn_last_error().decode())
            else:
                msgs[k] = (0, lib.rn_last_error().decode())
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append((k, repr(e)))

    # a fifth thread drives the partial-input entry point
    pwl = WL.WORKLOADS["partials_8x2048x8192"].with_rows(48)
    pin = WL.generate_partials(pwl, seed=23)
    pparts = [to_dev(p, "bf16") for p in pin["partials"]]
    pres, pw = to_dev(pin["residual"], "f32"), to_dev(pin["weight"], "bf16")
    pref = R.fused_partials_add_rmsnorm(pparts, pres, pw, pwl.eps)
    torch.cuda.synchronize()
    pref_out, pref_res = to_host(pref.out), to_host(pref.residual_out)

    def partials_worker():
        stream = torch.cuda.Stream()
        try:
            with torch.cuda.stream(stream):
                for i in range(20):
                    r = R.fused_partials_add_rmsnorm(pparts, pres, pw, pwl.eps)
                    stream.synchronize()
                    if not (np.array_equal(to_host(r.out), pref_out) and np.array_equal(to_host(r.residual_out),
                                                                                         pref_res)):
                        errors.append(("partials", i))
                        return
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(("partials", repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(jobs))]
    threads.append(threading.Thread(target=partials_worker))
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    torch.cuda.synchronize()
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    assert msgs[0][0] == L.RN_ERR_UNSUPPORTED and msgs[0][1]
    assert all(msgs[k][1] == "" for k in range(1, len(jobs))), msgs


def test_graph_capture_replays():
    """The entry points captured in one HIP graph (the library records kernel
    launches only: no memset, no allocation) and replayed several times, with
    eager work that changes the inputs between replays: every replay equals the
    eager result for the inputs it saw."""
    wl = WL.WORKLOADS["prefill_fp8_8192x7168"].with_rows(64)
    inputs = WL.generate_rownorm(wl, seed=22)
    x = to_dev(inputs["x"], "bf16")
    res = to_dev(inputs["residual"], "bf16")
    w = to_dev(inputs["weight"], "bf16")
    out = torch.empty_like(x)
    ro = torch.empty_like(res)
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device="cuda")
    act_in = torch.cat([x, res], dim=1).contiguous()
    act_out = torch.empty_like(x)
    p_out = torch.empty_like(x)
    p_ro = torch.empty_like(res)
    _announce("graph capture of rmsnorm / fp8 / silu_mul / 3 partials, 4 replays")

    def step():
        R.fused_add_rmsnorm(x, res, w, wl.eps, out=out, residual_out=ro)
        r8 = R.fused_add_rmsnorm(x, res, w, wl.eps, out_dtype=torch.float8_e4m3fn, out=q,
                                 residual_out=torch.empty_like(res))
        R.silu_mul(act_in, out=act_out)
        R.fused_partials_add_rmsnorm([x, res, x], res, w, wl.eps, out=p_out, residual_out=p_ro)
        return r8

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        r8g = step()
    for k in range(4):
        # eager work between replays: new inputs in the captured buffers
        x.mul_(-1.0 if k % 2 else 0.5)
        act_in.copy_(torch.cat([x, res], dim=1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (to_host(out), to_host(ro), to_host(q), to_host(r8g.scale), to_host(act_out), to_host(p_out),
               to_host(p_ro))
        e = R.fused_add_rmsnorm(x, res, w, wl.eps)
        e8 = R.fused_add_rmsnorm(x, res, w, wl.eps, out_dtype=torch.float8_e4m3fn)
        ea = R.silu_mul(act_in)
        ep = R.fused_partials_add_rmsnorm([x, res, x], res, w, wl.eps)
        torch.cuda.synchronize()
        want = (to_host(e.out), to_host(e.residual_out), to_host(e8.out), to_host(e8.scale), to_host(ea.out),
                to_host(ep.out), to_host(ep.residual_out))
        for a, b in zip(got, want):
            assert np.array_equal(a, b), k
