"""GPU parity on tensors larger than 4 GiB (64-bit address arithmetic).

Each case holds at least one tensor of more than 2^32 bytes. A 32-bit byte
offset anywhere in a kernel's address arithmetic would then wrap, and the
rows past the boundary would read or write the wrong place.

The inputs are a seeded block of rows from ``workloads`` (the shared
generator), repeated on the device along the row (or token) axis by torch.
Sampled rows before, at and past the 4 GiB boundary, and the last rows, are
checked against the oracle on the matching block rows, under the usual rules.
"""

import numpy as np
import pytest
import torch

import residual_add_rmsnorm_rows_amd as R
import workloads as WL
from oracle import activation as ACT
from oracle import compare as C
from oracle import rownorm as O
from tests.gpu_util import judge_partials_rows, judge_rows, judge_y, to_dev, to_host

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32
BLOCK = 64  # generated rows, repeated to the full size


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _need(nbytes):
    free, _ = torch.cuda.mem_get_info()
    if free < 1.1 * nbytes:
        pytest.skip(f"needs {nbytes / 2**30:.1f} GiB of free device memory, {free / 2**30:.1f} GiB free")


def _sampled(rows, row_bytes):
    """The first rows, the rows around byte offset 4 GiB of a tensor with
    `row_bytes` per row, the middle row and the last rows."""
    b = GIB4 // row_bytes
    assert rows > b + 1, "the tensor must extend past 4 GiB"
    return np.unique(np.array([0, 1, b - 1, b, b + 1, rows // 2, rows - 2, rows - 1]))


def _rep(t, rows):
    return t.repeat((rows // t.shape[0],) + (1,) * (t.dim() - 1))


def _release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_rows_kernel_beyond_4gib():
    """69632 x 16384, bf16 x, f32 residual in and out (4.56 GB each), bf16 out."""
    rows, H = 69632, 16384
    _need(rows * H * (2 + 4 + 4 + 2))
    wl = WL.RowNormWorkload(name="big", kind="prefill", rows=BLOCK, hidden=H, x_dtype="bf16", res_dtype="f32",
                            w_dtype="bf16", out_dtype="bf16", x_dist=WL.Dist(0, 1), res_dist=WL.Dist(0, 4),
                            w_dist=WL.Dist(1, 0.1), weight_plus_one=False, eps=1e-6)
    _announce(f"rows kernel {rows} x {H} cfg={R.query_config(rows, H, res_dtype='f32')}")
    inp = WL.generate_rownorm(wl, seed=5)
    x = _rep(to_dev(inp["x"], "bf16"), rows)
    res = _rep(to_dev(inp["residual"], "f32"), rows)
    r = R.fused_add_rmsnorm(x, res, to_dev(inp["weight"], "bf16"), wl.eps)
    torch.cuda.synchronize()
    idx = _sampled(rows, H * 4)
    ti = torch.from_numpy(idx).cuda()
    sub = {"x": inp["x"][idx % BLOCK], "residual": inp["residual"][idx % BLOCK], "weight": inp["weight"]}
    rep = judge_rows(sub, "bf16", "f32", "bf16", "bf16", wl.eps, False, to_host(r.out[ti]),
                     to_host(r.residual_out[ti]))
    del x, res, r
    _release()
    assert rep["ok"], (idx.tolist(), rep)


def test_partials_beyond_4gib():
    """Two bf16 partials of 131328 x 16384 (4.3 GB each), no residual, bf16 out."""
    rows, H = 131328, 16384
    _need(rows * H * 2 * 3)
    wl = WL.PartialsWorkload(name="bigp", rows=BLOCK, hidden=H, num_partials=2, x_dtype="bf16", res_dtype=None,
                             w_dtype="bf16", out_dtype="bf16", part_dist=WL.Dist(0, 0.5), res_dist=None,
                             w_dist=WL.Dist(1, 0.1), weight_plus_one=False, eps=1e-6)
    _announce(f"partials 2 x {rows} x {H} cfg={R.query_partials_config(rows, H, 2)}")
    inp = WL.generate_partials(wl, seed=6)
    parts = [_rep(to_dev(p, "bf16"), rows) for p in inp["partials"]]
    r = R.fused_partials_add_rmsnorm(parts, None, to_dev(inp["weight"], "bf16"), wl.eps)
    torch.cuda.synchronize()
    idx = _sampled(rows, H * 2)
    ti = torch.from_numpy(idx).cuda()
    sub = {"partials": [p[idx % BLOCK] for p in inp["partials"]], "residual": None, "weight": inp["weight"]}
    rep = judge_partials_rows(sub, "bf16", None, "bf16", "bf16", wl.eps, False, to_host(r.out[ti]), None)
    del parts, r
    _release()
    assert rep["ok"], (idx.tolist(), rep)


def test_qknorm_beyond_4gib():
    """528384 tokens x 32 heads x 128 bf16 (4.33 GB), out of place."""
    tokens, nq, D = 528384, 32, 128
    _need(tokens * nq * D * 2 * 2)
    wl = WL.QKNormWorkload(name="bigq", tokens=BLOCK, num_q_heads=nq, num_k_heads=0, head_dim=D, dtype="bf16",
                           w_dtype="bf16", x_dist=WL.Dist(0, 1), w_dist=WL.Dist(1, 0.1), weight_plus_one=False,
                           eps=1e-6)
    _announce(f"qknorm {tokens} x {nq} x {D} cfg={R.query_qknorm_config(tokens, nq, 0, D)}")
    inp = WL.generate_qknorm(wl, seed=7)
    q = _rep(to_dev(inp["q"].reshape(BLOCK, -1), "bf16"), tokens).view(tokens, nq, D)
    q_out, _ = R.qk_norm(q, None, to_dev(inp["q_weight"], "bf16"), None, wl.eps, inplace=False)
    torch.cuda.synchronize()
    idx = _sampled(tokens, nq * D * 2)
    got = to_host(q_out[torch.from_numpy(idx).cuda()])
    qy, _ = O.qknorm(O.decode(inp["q"][idx % BLOCK], "bf16"), None, O.decode(inp["q_weight"], "bf16"), None,
                     wl.eps, 0.0)
    rep = C.check_bf16(got, qy)
    del q, q_out
    _release()
    assert rep["ok"], (idx.tolist(), rep)


def test_silu_mul_beyond_4gib():
    """75776 x (2 x 14336) bf16 (4.35 GB), bf16 out."""
    rows, d = 75776, 14336
    _need(rows * d * 2 * 3)
    wl = WL.ActWorkload(name="biga", rows=BLOCK, d=d, x_dtype="bf16", out_dtype="bf16", x_dist=WL.Dist(0, 1))
    _announce(f"silu_mul {rows} x {d} cfg={R.query_silu_mul_config(rows, d)}")
    xn = WL.generate_act(wl, seed=8)
    x = _rep(to_dev(xn, "bf16"), rows)
    r = R.silu_mul(x)
    torch.cuda.synchronize()
    idx = _sampled(rows, 2 * d * 2)
    got = to_host(r.out[torch.from_numpy(idx).cuda()])
    rep = judge_y(ACT.silu_mul_rows(O.decode(xn[idx % BLOCK], "bf16"), d), "bf16", got)
    del x, r
    _release()
    assert rep["y_ok"], (idx.tolist(), rep)
