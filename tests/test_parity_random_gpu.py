"""Seeded randomized parity: random shapes, dtypes, output schemes and
explicit launch configurations of the rows, per-head and SwiGLU kernels
against the oracle.  Every case is drawn from a fixed seed, so a failure names
a reproducible case."""

import numpy as np
import pytest
import torch

import residual_add_rmsnorm_rows_amd as R
import workloads as WL
from oracle import activation as ACT
from oracle import compare as C
from oracle import rownorm as O
from residual_add_rmsnorm_rows_amd import _lib as L
from tests.gpu_util import TORCH_DTYPES, judge_rows, judge_y, nvfp4_tensor_scale, to_dev, to_host

pytestmark = pytest.mark.gpu

GRANULE = {"row": 1, "group128": 128, "mx32": 32, "nv16": 16}
OUTS = [("bf16", "row"), ("f32", "row"), ("fp8_e4m3fn", "row"), ("fp8_e4m3fn", "group128"),
        ("fp8_e4m3fn", "mx32"), ("fp4_e2m1", "mx32"), ("fp4_e2m1", "nv16")]


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _random_config(rng, hidden, vec, rows):
    """A valid explicit rows-kernel configuration covering the row, or None (the selector's)."""
    if rng.random() < 0.3:
        return None
    nvec = -(-hidden // vec)
    opts = [(W, NV) for W in range(1, 17) for NV in (1, 2, 4, 8)
            if 64 * W <= (512 if NV == 8 else 1024) and 64 * W * NV >= nvec and 64 * W * NV <= 4 * nvec + 64]
    W, NV = opts[rng.integers(len(opts))]
    cfg = L.LaunchConfig()
    cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane = L.RN_KERNEL_ROWS, W, NV
    cfg.grid = int(rng.integers(1, rows + 1))
    return cfg


def _row_cases(n=48, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        x = ["bf16", "f32"][rng.integers(2)]
        res = [None, x, "f32"][rng.integers(3)]
        w = ["bf16", "f32"][rng.integers(2)]
        out, scheme = OUTS[rng.integers(len(OUTS))]
        vec = 8 if x == "bf16" else 4
        g = int(np.lcm(vec, GRANULE[scheme]))
        hmax = 8192 if x == "bf16" else 4096
        hidden = g * int(rng.integers(1, hmax // g + 1))
        rows = int(rng.integers(1, 25))
        cases.append((i, x, res, w, out, scheme, bool(rng.integers(2)), hidden, rows, int(rng.integers(1 << 30))))
    return cases


def _row_cases_prefill(n=24, seed=2026):
    """Row counts past the compute-unit count, where the selector's prefill
    tables and its more-vectors rule apply; always the selector's launch."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        x = ["bf16", "f32"][rng.integers(2)]
        res = [None, x, "f32"][rng.integers(3)]
        w = ["bf16", "f32"][rng.integers(2)]
        out, scheme = OUTS[rng.integers(len(OUTS))]
        vec = 8 if x == "bf16" else 4
        g = int(np.lcm(vec, GRANULE[scheme]))
        hmax = 8192 if x == "bf16" else 4096
        hidden = g * int(rng.integers(1024 // g + 1, hmax // g + 1))
        rows = int(rng.integers(257, 601))
        cases.append((i, x, res, w, out, scheme, bool(rng.integers(2)), hidden, rows, int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _row_cases(), ids=lambda c: f"r{c[0]}")
def test_random_rows(case):
    _row_case(case, selector_only=False)


@pytest.mark.parametrize("case", _row_cases_prefill(), ids=lambda c: f"rp{c[0]}")
def test_random_rows_prefill_selector(case):
    _row_case(case, selector_only=True)


def _row_case(case, selector_only):
    i, x, res, w, out, scheme, b, hidden, rows, seed = case
    rng = np.random.default_rng(seed)
    wl = WL.RowNormWorkload(name="rand", kind="test", rows=rows, hidden=hidden, x_dtype=x, res_dtype=res,
                            w_dtype=w, out_dtype=out, x_dist=WL.Dist(0, 1, 0.01, 20.0),
                            res_dist=None if res is None else WL.Dist(0, 3), w_dist=WL.Dist(0.0 if b else 1.0, 0.2),
                            weight_plus_one=b, eps=float(np.float32(10.0 ** rng.uniform(-7, -3))))
    cfg = None if selector_only else _random_config(rng, hidden, 8 if x == "bf16" else 4, rows)
    if cfg is None:
        q = R.query_config(rows, hidden, x_dtype=x, res_dtype=res, w_dtype=w, out_dtype=out, weight_plus_one=b,
                           scale_scheme=scheme, num_cus=0)
        cfg_txt = ("selector", q["waves_per_row"], q["vecs_per_lane"], q["grid"])
    else:
        cfg_txt = (cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid)
    _announce(f"random rows #{i}: x={x} res={res} w={w} out={out}/{scheme} plus_one={b} rows={rows} H={hidden} "
              f"cfg={cfg_txt}")
    inputs = WL.generate_rownorm(wl, seed=seed)
    X = to_dev(inputs["x"], x)
    RES = None if res is None else to_dev(inputs["residual"], res)
    W = to_dev(inputs["weight"], w)
    ts = None
    if scheme == "nv16":
        Y = O.rmsnorm_rows(O.decode(inputs["x"], x), O.decode(inputs["weight"], w), wl.eps, 1.0 if b else 0.0,
                           residual=None if res is None else O.decode(inputs["residual"], res), res_dtype=res)["y"]
        ts = nvfp4_tensor_scale(Y) * float(2.0 ** rng.integers(-3, 4))
    quant = out in ("fp8_e4m3fn", "fp4_e2m1")
    r = R.fused_add_rmsnorm(X, RES, W, wl.eps, weight_plus_one=b, out_dtype=TORCH_DTYPES[out], return_amax=quant,
                            scale_scheme=scheme, tensor_scale=ts, config=cfg)
    torch.cuda.synchronize()
    rep = judge_rows(inputs, x, res, w, out, wl.eps, b, to_host(r.out),
                     None if r.residual_out is None else to_host(r.residual_out),
                     None if r.scale is None else to_host(r.scale), None if r.amax is None else to_host(r.amax),
                     scale_scheme=scheme, tensor_scale=ts)
    assert rep["ok"], rep


def _head_cases(n=24, seed=2025):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = ["bf16", "f32"][rng.integers(2)]
        D = [64, 128, 256][rng.integers(3)]
        nq = int(rng.integers(1, 17))
        nk = int(rng.integers(0, 9))
        T = int(rng.integers(1, 70))
        cases.append((i, dt, ["bf16", "f32"][rng.integers(2)], D, nq, nk, T, bool(rng.integers(2)),
                      bool(rng.integers(2)), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _head_cases(), ids=lambda c: f"h{c[0]}")
def test_random_qknorm(case):
    i, dt, wdt, D, nq, nk, T, b, strided, seed = case
    rng = np.random.default_rng(seed)
    _announce(f"random qknorm #{i}: dt={dt} w={wdt} D={D} nq={nq} nk={nk} T={T} plus_one={b} strided={strided}")
    wl = WL.QKNormWorkload(name="rq", tokens=T, num_q_heads=nq, num_k_heads=nk, head_dim=D, dtype=dt, w_dtype=wdt,
                           x_dist=WL.Dist(0, 2), w_dist=WL.Dist(0.0 if b else 1.0, 0.2),
                           weight_plus_one=b, eps=1e-6)
    inp = WL.generate_qknorm(wl, seed=seed)
    extra = 8 * (1 + int(rng.integers(4))) if strided else 0  # token stride padding (elements)
    qn = inp["q"].reshape(T, nq * D)
    # q (and k) as views of one fused buffer [T, nq*D + nk*D + extra]
    width = (nq + nk) * D + extra
    host = np.zeros((T, width), dtype=qn.dtype)
    host[:, :nq * D] = qn
    if nk:
        host[:, nq * D:(nq + nk) * D] = inp["k"].reshape(T, nk * D)
    buf = to_dev(host, dt)
    q = buf[:, :nq * D].view(T, nq, D) if not strided else torch.as_strided(buf, (T, nq, D), (width, D, 1))
    k = None
    if nk:
        k = torch.as_strided(buf, (T, nk, D), (width, D, 1), storage_offset=nq * D)
    qw = to_dev(inp["q_weight"], wdt)
    kw = None if nk == 0 else to_dev(inp["k_weight"], wdt)
    qo, ko = R.qk_norm(q, k, qw, kw, wl.eps, weight_plus_one=b, inplace=False)
    torch.cuda.synchronize()
    qy, ky = O.qknorm(O.decode(inp["q"], dt), None if nk == 0 else O.decode(inp["k"], dt),
                      O.decode(inp["q_weight"], wdt), None if nk == 0 else O.decode(inp["k_weight"], wdt),
                      wl.eps, 1.0 if b else 0.0)
    check = C.check_bf16 if dt == "bf16" else C.check_f32
    rq = check(to_host(qo.contiguous()).reshape(qy.shape), qy)
    assert rq["ok"], rq
    if nk:
        rk = check(to_host(ko.contiguous()).reshape(ky.shape), ky)
        assert rk["ok"], rk


def _act_cases(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        x = ["bf16", "f32"][rng.integers(2)]
        out, scheme = OUTS[rng.integers(len(OUTS))]
        vec = 8 if x == "bf16" else 4
        g = int(np.lcm(vec, GRANULE[scheme]))
        dmax = 8192 if x == "bf16" else 4096
        d = g * int(rng.integers(1, dmax // g + 1))
        cases.append((i, x, out, scheme, d, int(rng.integers(1, 25)), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _act_cases(), ids=lambda c: f"a{c[0]}")
def test_random_silu_mul(case):
    i, x, out, scheme, d, rows, seed = case
    rng = np.random.default_rng(seed)
    cfg = _random_config(rng, d, 8 if x == "bf16" else 4, rows)
    cfg_txt = None if cfg is None else (cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid)
    _announce(f"random silu_mul #{i}: x={x} out={out}/{scheme} rows={rows} d={d} cfg={cfg_txt}")
    wl = WL.ActWorkload(name="ra", rows=rows, d=d, x_dtype=x, out_dtype=out, x_dist=WL.Dist(0, 2, 0.01, 20.0))
    xn = WL.generate_act(wl, seed=seed)
    y = ACT.silu_mul_rows(O.decode(xn, x), d)
    ts = nvfp4_tensor_scale(y) * float(2.0 ** rng.integers(-3, 4)) if scheme == "nv16" else None
    quant = out in ("fp8_e4m3fn", "fp4_e2m1")
    r = R.silu_mul(to_dev(xn, x), out_dtype=TORCH_DTYPES[out], scale_scheme=scheme, return_amax=quant,
                   tensor_scale=ts, config=cfg)
    torch.cuda.synchronize()
    rep = judge_y(y, out, to_host(r.out), None if r.scale is None else to_host(r.scale),
                  None if r.amax is None else to_host(r.amax), scheme, ts, f32_abs_floor=C.SILU_F32_ABS_FLOOR)
    assert rep["y_ok"], rep


def _partials_cases(n=32, seed=77):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        x = ["bf16", "f32"][rng.integers(2)]
        res = [None, x, "f32"][rng.integers(3)]
        w = ["bf16", "f32"][rng.integers(2)]
        out, scheme = OUTS[rng.integers(len(OUTS))]
        vec = 8 if x == "bf16" else 4
        g = int(np.lcm(vec, GRANULE[scheme]))
        k = int(rng.integers(1, 9))
        hmax = (16384 if x == "bf16" else 8192) if k > 1 else 4096
        hidden = g * int(rng.integers(1, min(hmax, 6144) // g + 1))
        rows = int(rng.integers(1, 40))
        exact = bool(rng.random() < 0.25)  # a quarter on the exact-sum recipe's narrowed inputs
        cases.append((i, x, res, w, out, scheme, bool(rng.integers(2)), k, hidden, rows, exact,
                      int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _partials_cases(), ids=lambda c: f"p{c[0]}")
def test_random_partials(case):
    """Random partial-input calls, judged like single-input rows: the updated
    residual is the exact sum rounded once (bit-exact), every output scheme
    within its usual tolerance."""
    from tests.gpu_util import judge_partials_rows

    i, x, res, w, out, scheme, b, k, hidden, rows, exact, seed = case
    rng = np.random.default_rng(seed)
    wl = WL.PartialsWorkload(name="rand", rows=rows, hidden=hidden, num_partials=k, x_dtype=x, res_dtype=res,
                             w_dtype=w, out_dtype=out, part_dist=WL.Dist(0, float(rng.uniform(0.2, 2.0))),
                             res_dist=None if res is None else WL.Dist(0, 3), w_dist=WL.Dist(0.0 if b else 1.0, 0.2),
                             weight_plus_one=b, eps=float(np.float32(10.0 ** rng.uniform(-7, -3))), exact_sum=exact)
    cfg = None
    if rng.random() < 0.6:
        vec = 8 if x == "bf16" else 4
        nvec = -(-hidden // vec)
        max_nv = 2 if k > 1 else 8
        opts = [(W, NV) for W in range(1, 17) for NV in (1, 2, 4, 8)
                if NV <= max_nv and 64 * W <= (512 if NV == 8 else 1024) and 64 * W * NV >= nvec
                and 64 * W * NV <= 4 * nvec + 64]
        W_, NV_ = opts[rng.integers(len(opts))]
        cfg = L.LaunchConfig()
        cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane = L.RN_KERNEL_ROWS, W_, NV_
        cfg.grid = int(rng.integers(1, rows + 1))
    cfg_txt = None if cfg is None else (cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid)
    _announce(f"random partials #{i}: k={k} x={x} res={res} w={w} out={out}/{scheme} plus_one={b} rows={rows} "
              f"H={hidden} exact={exact} cfg={cfg_txt}")
    inputs = WL.generate_partials(wl, seed=seed)
    ts = None
    if scheme == "nv16":
        Y = O.rmsnorm_rows_partials([O.decode(p, x) for p in inputs["partials"]], O.decode(inputs["weight"], w), wl.eps,
                                    1.0 if b else 0.0,
                                    residual=None if res is None else O.decode(inputs["residual"], res),
                                    res_dtype=res)["y"]
        ts = nvfp4_tensor_scale(Y) * float(2.0 ** rng.integers(-3, 4))
    parts = [to_dev(p, x) for p in inputs["partials"]]
    RES = None if res is None else to_dev(inputs["residual"], res)
    quant = out in ("fp8_e4m3fn", "fp4_e2m1")
    r = R.fused_partials_add_rmsnorm(parts, RES, to_dev(inputs["weight"], w), wl.eps, weight_plus_one=b,
                                     out_dtype=TORCH_DTYPES[out], return_amax=quant, scale_scheme=scheme,
                                     tensor_scale=ts, config=cfg)
    torch.cuda.synchronize()
    rep = judge_partials_rows(inputs, x, res, w, out, wl.eps, b, to_host(r.out),
                              None if r.residual_out is None else to_host(r.residual_out),
                              None if r.scale is None else to_host(r.scale), None if r.amax is None else to_host(r.amax),
                              scale_scheme=scheme, tensor_scale=ts)
    assert rep["ok"], rep
