"""Host-side tests of the C-ABI library: it loads, exports what the header
declares, rejects bad arguments before touching HIP, and the selector's
launch configurations cover every row.  No GPU is needed: no call here
reaches a kernel launch (every argument check fails first, or the call is a
host-only query with an explicit compute-unit count).
"""

import ctypes
import os
import re

import pytest

from residual_add_rmsnorm_rows_amd import _lib as L
import residual_add_rmsnorm_rows_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm_rows.h")


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_what_binding_knows():
    assert _declared_functions() == sorted(L.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_and_status_strings(lib):
    assert lib.rn_abi_version() == L.ABI_VERSION
    for st in range(5):
        assert lib.rn_status_string(st).decode().startswith("RN_")
    assert b"unknown" in lib.rn_status_string(99)


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced (every call below fails first)
BF = L.make_flags("bf16", "bf16", "bf16", "bf16", False)
FP4_MX_FLAGS = L.make_flags("bf16", "bf16", "bf16", "fp4_e2m1", False, "mx32")


def _fwd(lib, x=FAKE, res=FAKE, w=FAKE, out=FAKE + 0x1000, res_out=FAKE + 0x2000, scale=None, amax=None,
         ts=None, rows=4, hidden=1024, eps=1e-6, flags=BF):
    return lib.rmsnorm_fwd_ex(x, res, w, out, res_out, scale, amax, ts, rows, hidden, eps, flags, None)


REJECT_CASES = [
    (dict(rows=-1), L.RN_ERR_INVALID_ARG),
    (dict(hidden=0), L.RN_ERR_INVALID_ARG),
    (dict(flags=BF | (1 << 9)), L.RN_ERR_INVALID_ARG),
    (dict(flags=3), L.RN_ERR_INVALID_ARG),
    (dict(eps=-1.0), L.RN_ERR_INVALID_ARG),
    (dict(eps=float("nan")), L.RN_ERR_INVALID_ARG),
    (dict(eps=float("inf")), L.RN_ERR_INVALID_ARG),
    (dict(x=None), L.RN_ERR_INVALID_ARG),
    (dict(w=None), L.RN_ERR_INVALID_ARG),
    (dict(out=None), L.RN_ERR_INVALID_ARG),
    (dict(res_out=None), L.RN_ERR_INVALID_ARG),
    (dict(res=None), L.RN_ERR_INVALID_ARG),
    (dict(res_out=FAKE + 0x1000), L.RN_ERR_INVALID_ARG),  # out == residual_out
    (dict(scale=FAKE), L.RN_ERR_INVALID_ARG),  # scale without fp8
    (dict(flags=L.make_flags("bf16", "bf16", "bf16", "fp8_e4m3fn", False)), L.RN_ERR_INVALID_ARG),  # fp8, no scale
    (dict(hidden=1001), L.RN_ERR_UNSUPPORTED),
    (dict(hidden=32768 + 8), L.RN_ERR_UNSUPPORTED),
    (dict(flags=L.make_flags("f32", "bf16", "f32", "f32", False), hidden=1024), L.RN_ERR_UNSUPPORTED),
    (dict(flags=L.make_flags("fp8_e4m3fn", "bf16", "bf16", "bf16", False)), L.RN_ERR_UNSUPPORTED),
    (dict(x=FAKE + 8), L.RN_ERR_MISALIGNED),
    (dict(res_out=FAKE + 0x2004), L.RN_ERR_MISALIGNED),
    (dict(flags=L.make_flags("bf16", "bf16", "bf16", "fp8_e4m3fn", False), scale=FAKE + 2), L.RN_ERR_MISALIGNED),
    # in place only with equal element widths (a wider or narrower out row overlaps other rows of x)
    (dict(out=FAKE, flags=L.make_flags("bf16", "bf16", "bf16", "f32", False)), L.RN_ERR_INVALID_ARG),
    (dict(out=FAKE, flags=L.make_flags("f32", "f32", "bf16", "bf16", False)), L.RN_ERR_INVALID_ARG),
    (dict(out=FAKE, flags=L.make_flags("bf16", "bf16", "bf16", "fp8_e4m3fn", False), scale=FAKE + 0x3000),
     L.RN_ERR_INVALID_ARG),
    (dict(out=FAKE, flags=FP4_MX_FLAGS, scale=FAKE + 0x3000), L.RN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,status", REJECT_CASES)
def test_rmsnorm_rejects_before_any_hip_call(lib, kw, status):
    assert _fwd(lib, **kw) == status
    assert lib.rn_last_error().decode() != ""


def _call(lib, x=FAKE, res=FAKE, w=FAKE, out=FAKE + 0x1000, res_out=FAKE + 0x2000, scale=None, amax=None,
          ts=None, rows=4, hidden=1024, eps=1e-6, flags=BF):
    rec = L.RmsnormCall(x, res, w, out, res_out, scale, amax, ts, rows, hidden, eps, flags, None)
    return lib.rmsnorm_fwd_call(ctypes.byref(rec))


@pytest.mark.parametrize("kw,status", REJECT_CASES)
def test_call_record_checks_like_rmsnorm_fwd_ex(lib, kw, status):
    assert _call(lib, **kw) == status
    assert lib.rn_last_error().decode() != ""


def test_call_record_null_and_zero_rows(lib):
    assert lib.rmsnorm_fwd_call(None) == L.RN_ERR_INVALID_ARG
    assert _call(lib, x=None, res=None, w=None, out=None, res_out=None, rows=0) == L.RN_OK


def _qflags(out, scheme, x="bf16", res="bf16"):
    return L.make_flags(x, res, "bf16", out, False, scheme)


FP8_G = _qflags("fp8_e4m3fn", "group128")
FP8_MX = _qflags("fp8_e4m3fn", "mx32")
FP4_MX = _qflags("fp4_e2m1", "mx32")
FP4_NV = _qflags("fp4_e2m1", "nv16")
SC = FAKE + 0x3000  # scale buffer
TS = FAKE + 0x4000  # NVFP4 tensor scale


@pytest.mark.parametrize("kw,status", [
    (dict(flags=FP8_G, scale=SC, hidden=1024 + 64), L.RN_ERR_UNSUPPORTED),   # per-128 needs H % 128
    (dict(flags=FP8_MX, scale=SC, hidden=1024 + 16), L.RN_ERR_UNSUPPORTED),  # MX needs H % 32
    (dict(flags=FP4_NV, scale=SC, ts=TS, hidden=1024 + 8), L.RN_ERR_UNSUPPORTED),  # NVFP4 needs H % 16
    (dict(flags=_qflags("fp4_e2m1", "row"), scale=SC), L.RN_ERR_UNSUPPORTED),  # fp4 takes MX or NVFP4 scales
    (dict(flags=_qflags("fp4_e2m1", "group128"), scale=SC), L.RN_ERR_UNSUPPORTED),
    (dict(flags=_qflags("fp8_e4m3fn", "nv16"), scale=SC, ts=TS), L.RN_ERR_UNSUPPORTED),  # NVFP4 is fp4 only
    (dict(flags=FP4_NV, scale=SC), L.RN_ERR_INVALID_ARG),                    # NVFP4 without tensor scale
    (dict(flags=FP4_MX, scale=SC, ts=TS), L.RN_ERR_INVALID_ARG),             # tensor scale without NVFP4
    (dict(flags=BF, ts=TS), L.RN_ERR_INVALID_ARG),
    (dict(flags=FP4_NV, ts=TS), L.RN_ERR_INVALID_ARG),                       # no scale buffer
    (dict(flags=FP4_NV, scale=SC, ts=TS + 2), L.RN_ERR_MISALIGNED),
    (dict(flags=FP8_G, scale=SC + 2), L.RN_ERR_MISALIGNED),                  # float32 scales
    (dict(flags=FP8_G, scale=SC, amax=SC + 0x1002), L.RN_ERR_MISALIGNED),
    (dict(flags=BF, amax=SC), L.RN_ERR_INVALID_ARG),                         # amax without quantized out
])
def test_block_scaled_outputs_are_checked(lib, kw, status):
    assert _fwd(lib, **kw) == status
    assert lib.rn_last_error().decode() != ""


def test_byte_scales_need_no_alignment_and_base_entry_rejects_nvfp4(lib):
    # E8M0 / E4M3FN scales are bytes: an odd address passes every pointer check,
    # and the call stops at the (deliberately uncovering) explicit launch
    # configuration, checked after the pointers and before any HIP call
    cfg = L.LaunchConfig()
    cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = 0, 1, 1, 4
    for flags, ts in ((FP4_MX, None), (FP4_NV, TS)):
        st = lib.rmsnorm_fwd_config(FAKE, FAKE, FAKE, FAKE + 0x1000, FAKE + 0x2000, SC + 1, None, ts, 4, 1024,
                                    1e-6, flags, ctypes.byref(cfg), None)
        assert st == L.RN_ERR_INVALID_ARG and "config" in lib.rn_last_error().decode()
    # rmsnorm_fwd has no tensor_scale argument: NVFP4 is rejected there
    st = lib.rmsnorm_fwd(FAKE, FAKE, FAKE, FAKE + 0x1000, FAKE + 0x2000, SC, 4, 1024, 1e-6, FP4_NV, None)
    assert st == L.RN_ERR_INVALID_ARG and "tensor_scale" in lib.rn_last_error().decode()


def test_silu_mul_rejects_before_any_hip_call(lib):
    def call(x=FAKE, out=FAKE + 0x1000, scale=None, amax=None, ts=None, rows=4, d=1024,
             flags=(L.RN_DTYPE_BF16 << L.RN_FLAGS_X_SHIFT) | (L.RN_DTYPE_BF16 << L.RN_FLAGS_OUT_SHIFT)):
        return lib.silu_mul_fwd(x, out, scale, amax, ts, rows, d, flags, None)

    nv = (L.RN_DTYPE_FP4_E2M1 << L.RN_FLAGS_OUT_SHIFT) | (3 << L.RN_FLAGS_SCALE_SHIFT)
    assert call(rows=-1) == L.RN_ERR_INVALID_ARG
    assert call(d=0) == L.RN_ERR_INVALID_ARG
    assert call(flags=1 << L.RN_FLAGS_RES_SHIFT) == L.RN_ERR_INVALID_ARG  # residual bits are not silu_mul's
    assert call(flags=L.RN_FLAG_WEIGHT_PLUS_ONE) == L.RN_ERR_INVALID_ARG
    assert call(x=None) == L.RN_ERR_INVALID_ARG
    assert call(out=None) == L.RN_ERR_INVALID_ARG
    assert call(scale=SC) == L.RN_ERR_INVALID_ARG
    assert call(d=1004) == L.RN_ERR_UNSUPPORTED  # not a multiple of the 8-element bf16 vector
    assert call(x=FAKE + 8) == L.RN_ERR_MISALIGNED
    assert call(flags=nv, scale=SC) == L.RN_ERR_INVALID_ARG  # NVFP4 without tensor scale
    assert call(flags=nv, scale=SC, ts=TS + 1) == L.RN_ERR_MISALIGNED
    assert call(flags=nv, scale=SC, ts=TS, d=1024 + 8) == L.RN_ERR_UNSUPPORTED
    assert call(rows=0, x=None, out=None) == L.RN_OK
    cfg = L.LaunchConfig()
    assert lib.silu_mul_fwd_config(FAKE, FAKE, None, None, None, 4, 1024, 0, None, None) == L.RN_ERR_INVALID_ARG
    cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = 0, 1, 1, 4  # covers 512 of 1024
    assert lib.silu_mul_fwd_config(FAKE, FAKE + 0x1000, None, None, None, 4, 1024, 0, ctypes.byref(cfg),
                                   None) == L.RN_ERR_INVALID_ARG


def test_reference_copy_is_checked(lib):
    assert lib.rn_launch_copy(FAKE, FAKE + 0x10000, 1000, None) == L.RN_ERR_INVALID_ARG  # not a multiple of 16
    assert lib.rn_launch_copy(FAKE, FAKE + 0x10000, -16, None) == L.RN_ERR_INVALID_ARG
    assert lib.rn_launch_copy(None, FAKE, 1024, None) == L.RN_ERR_INVALID_ARG
    assert lib.rn_launch_copy(FAKE, FAKE + 512, 1024, None) == L.RN_ERR_INVALID_ARG  # overlap
    assert lib.rn_launch_copy(FAKE + 8, FAKE + 0x10000, 1024, None) == L.RN_ERR_MISALIGNED
    assert lib.rn_launch_copy(None, None, 0, None) == L.RN_OK


def test_rows_zero_is_a_noop(lib):
    assert _fwd(lib, rows=0, x=None, res=None, w=None, out=None, res_out=None) == L.RN_OK
    assert lib.rn_last_error() == b""


def test_qknorm_rejects_before_any_hip_call(lib):
    f = 0
    q = FAKE

    def call(**kw):
        a = dict(q=q, k=None, qw=q, kw=None, qo=q, ko=None, T=4, nq=2, nk=0, D=128, qs=0, ks=0, eps=1e-6, f=f)
        a.update(kw)
        return lib.qknorm_fwd(a["q"], a["k"], a["qw"], a["kw"], a["qo"], a["ko"], a["T"], a["nq"], a["nk"],
                              a["D"], a["qs"], a["ks"], a["eps"], a["f"], None)

    assert call(D=96) == L.RN_ERR_UNSUPPORTED
    assert call(nq=0) == L.RN_ERR_INVALID_ARG
    assert call(T=-1) == L.RN_ERR_INVALID_ARG
    assert call(f=1 << 6) == L.RN_ERR_INVALID_ARG       # out-dtype bits are not used by qknorm
    assert call(f=2) == L.RN_ERR_UNSUPPORTED            # fp8 tensors
    assert call(qs=100) == L.RN_ERR_INVALID_ARG         # stride below heads * head_dim
    assert call(nk=2) == L.RN_ERR_INVALID_ARG           # k missing
    assert call(q=FAKE + 4) == L.RN_ERR_MISALIGNED
    assert call(qs=256 + 4) == L.RN_ERR_MISALIGNED      # stride of 8 bytes past 16-byte alignment
    assert call(T=1 << 30, nq=4) == L.RN_ERR_UNSUPPORTED
    assert call(T=0, q=None, qw=None, qo=None) == L.RN_OK


def _cfg(rows, hidden, x="bf16", out="bf16", cus=256):
    return R.query_config(rows, hidden, x_dtype=x, out_dtype=out, num_cus=cus)


def _cfg_res(rows, hidden, res, x="bf16", out="bf16", cus=256):
    return R.query_config(rows, hidden, x_dtype=x, res_dtype=res, out_dtype=out, num_cus=cus)


@pytest.mark.parametrize("x", ["bf16", "f32"])
def test_selector_covers_every_row(x):
    vec = 8 if x == "bf16" else 4
    hmax = 32768 if x == "bf16" else 16384
    for hidden in list(range(vec, 4096 + 1, vec * 7)) + [7168, 8192, 12288, 16384, hmax]:
        if hidden > hmax:
            continue
        for rows in (1, 8, 255, 256, 257, 4096, 16384):
            c = _cfg(rows, hidden, x=x)
            W, NV = c["waves_per_row"], c["vecs_per_lane"]
            assert c["vec"] == vec
            assert 1 <= W <= 16 and NV in (1, 2, 4, 8)
            assert 64 * W * NV * vec >= hidden, (rows, hidden, c)
            assert c["block_threads"] == 64 * W
            assert c["block_threads"] <= (512 if NV == 8 else 1024)
            assert c["grid"] == rows


def test_selector_shapes_of_the_workloads():
    # decode: latency bound; one wave for rows of at most 128 vectors, else at
    # most 8 waves with the fewest vectors per lane
    c1, c2 = _cfg(8, 1024), _cfg(256, 4096)
    assert (c1["waves_per_row"], c1["vecs_per_lane"]) == (1, 2)
    assert (c2["waves_per_row"], c2["vecs_per_lane"]) == (8, 1)
    c = _cfg(8, 8192)
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (8, 2)
    c = _cfg(8, 32768)
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (8, 8)
    # prefill: the measured table (bf16 x with an f32 or bf16 residual stream)
    c3 = _cfg_res(16384, 8192, "f32")  # 4 x 4: +2.9% over 16 x 1 at this size
    assert (c3["waves_per_row"], c3["vecs_per_lane"]) == (4, 4)
    c5 = _cfg_res(8192, 7168, "bf16", out="fp8_e4m3fn")
    assert (c5["waves_per_row"], c5["vecs_per_lane"]) == (8, 2)
    # outside the table: the exact fit with the fewest vectors per lane
    c = _cfg_res(4096, 3072, "bf16")
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (6, 1)
    c = _cfg_res(4096, 10240, "bf16")
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (10, 2)
    # ... except bf16 rows without a residual (bf16 out) past 2 waves and
    # quantized outputs with a bf16 residual past 8 waves: 2 vectors per lane
    for hidden, shape in ((2304, (3, 2)), (2816, (3, 2)), (6656, (7, 2)), (1024, (2, 1))):
        c = _cfg(100000, hidden)
        assert (c["waves_per_row"], c["vecs_per_lane"]) == shape, (hidden, c)
    c = _cfg(100000, 3328, out="f32")  # f32 out keeps the exact fit
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (7, 1)
    for out, scheme in (("fp8_e4m3fn", "row"), ("fp8_e4m3fn", "group128"), ("fp4_e2m1", "mx32"), ("fp4_e2m1", "nv16")):
        for hidden, shape in ((6656, (7, 2)), (4352, (5, 2)), (3584, (7, 1)), (6144, (8, 2))):
            c = R.query_config(100000, hidden, res_dtype="bf16", out_dtype=out, scale_scheme=scheme)
            assert (c["waves_per_row"], c["vecs_per_lane"]) == shape, (out, scheme, hidden, c)
    c = _cfg_res(100000, 6656, "f32", out="fp8_e4m3fn")  # f32 residual keeps the exact fit
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (13, 1)
    # no residual and an output narrower than x: 4 vectors per lane; f32 rows
    # to f32: 2; quantized f32 rows with an f32 residual: 2 past 8 waves
    for x, out, scheme, hidden, shape in (("bf16", "fp8_e4m3fn", "row", 5376, (3, 4)),
                                          ("bf16", "fp4_e2m1", "mx32", 1536, (1, 4)),
                                          ("f32", "bf16", "row", 6144, (6, 4)), ("f32", "f32", "row", 3072, (6, 2))):
        c = R.query_config(100000, hidden, x_dtype=x, out_dtype=out, scale_scheme=scheme)
        assert (c["waves_per_row"], c["vecs_per_lane"]) == shape, (x, out, hidden, c)
    c = R.query_config(100000, 3584, x_dtype="f32", res_dtype="f32", out_dtype="fp8_e4m3fn")
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (7, 2)
    c = R.query_config(100000, 1536, x_dtype="f32", res_dtype="f32", out_dtype="fp8_e4m3fn")
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (6, 1)  # at most 8 waves: the exact fit
    # an f32 weight takes the same rules, plus 4 vectors per lane past 8 waves
    # with a bf16 residual and bf16 output
    for res, out, hidden, shape in ((None, "bf16", 7168, (7, 2)), (None, "fp8_e4m3fn", 5120, (3, 4)),
                                    ("bf16", "fp8_e4m3fn", 7168, (7, 2)), ("bf16", "bf16", 7168, (4, 4)),
                                    ("bf16", "bf16", 4096, (8, 1)), ("f32", "bf16", 7168, (14, 1))):
        c = R.query_config(100000, hidden, res_dtype=res, w_dtype="f32", out_dtype=out)
        assert (c["waves_per_row"], c["vecs_per_lane"]) == shape, (res, out, hidden, c)
    # mid-size calls: their own table per rows-per-CU bucket
    c = _cfg_res(1024, 8192, "bf16")
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (2, 8)
    c = _cfg_res(4097, 8192, "bf16")  # above 16 rows per CU: the prefill table
    assert (c["waves_per_row"], c["vecs_per_lane"]) == (16, 1)
    # SwiGLU: its own measured table at prefill sizes, the exact fit for decode
    a = R.query_silu_mul_config(8192, 14336)
    assert (a["waves_per_row"], a["vecs_per_lane"]) == (13, 4)
    a = R.query_silu_mul_config(8192, 14336, out_dtype="fp4_e2m1", scale_scheme="nv16")
    assert (a["waves_per_row"], a["vecs_per_lane"]) == (4, 8) and a["block_threads"] == 256
    a = R.query_silu_mul_config(16, 14336)
    assert (a["waves_per_row"], a["vecs_per_lane"]) == (14, 2)
    a = R.query_silu_mul_config(8192, 9728, out_dtype="fp4_e2m1", scale_scheme="nv16")
    assert (a["waves_per_row"], a["vecs_per_lane"]) == (6, 4)
    a = R.query_silu_mul_config(8192, 6144)
    assert (a["waves_per_row"], a["vecs_per_lane"]) == (13, 1)


def test_head_mapping_covers_each_row_once():
    """Replays the per-head kernel's row mapping on the CPU for the selector's grids."""
    for dtype, D in (("bf16", 64), ("bf16", 128), ("bf16", 256), ("f32", 64), ("f32", 128), ("f32", 256)):
        for tokens, nq, nk in ((4096, 32, 0), (7, 3, 1), (1, 1, 0), (33, 32, 8), (1000, 5, 3)):
            c = R.query_qknorm_config(tokens, nq, nk, D, dtype=dtype)
            vec = 8 if dtype == "bf16" else 4
            G = D // vec
            gpw = 64 // G
            rpl = c["rows_per_lane"]
            total = tokens * (nq + nk)
            seen = {}
            waves = c["grid"] * c["block_threads"] // 64
            for wave in range(waves):
                first = wave * gpw * rpl
                for j in range(rpl):
                    for grp in range(gpw):
                        row = first + j * gpw + grp
                        if row < total:
                            seen[row] = seen.get(row, 0) + 1
            assert len(seen) == total and set(seen.values()) == {1}, (dtype, D, tokens, nq, nk)
            # no workgroup lies wholly past the end
            assert (c["grid"] - 1) * (c["block_threads"] // 64) * gpw * rpl < total


def test_explicit_qknorm_config_is_checked(lib):
    cfg = L.LaunchConfig()

    def call(rpl, block, kernel=L.RN_KERNEL_HEADS):
        cfg.kernel, cfg.rows_per_lane, cfg.block_threads = kernel, rpl, block
        return lib.qknorm_fwd_config(FAKE, None, FAKE, None, FAKE, None, 4, 2, 0, 128, 0, 0, 1e-6, 0,
                                     ctypes.byref(cfg), None)

    assert call(3, 256) == L.RN_ERR_INVALID_ARG
    assert call(2, 512) == L.RN_ERR_INVALID_ARG
    assert call(2, 256, kernel=L.RN_KERNEL_ROWS) == L.RN_ERR_INVALID_ARG
    assert lib.qknorm_fwd_config(FAKE, None, FAKE, None, FAKE, None, 4, 2, 0, 128, 0, 0, 1e-6, 0, None,
                                 None) == L.RN_ERR_INVALID_ARG


def test_query_config_validates(lib):
    cfg = L.LaunchConfig()
    assert lib.rmsnorm_query_config(10, 1001, 0, 1, 256, ctypes.byref(cfg)) == L.RN_ERR_UNSUPPORTED
    assert lib.rmsnorm_query_config(10, 1024, 0, 1, 256, None) == L.RN_ERR_INVALID_ARG
    # a bf16 residual with f32 x is not built: rejected only when a residual is present
    f = L.make_flags("f32", "bf16", "f32", "f32", False)
    assert lib.rmsnorm_query_config(10, 1024, f, 1, 256, ctypes.byref(cfg)) == L.RN_ERR_UNSUPPORTED
    assert lib.rmsnorm_query_config(10, 1024, f, 0, 256, ctypes.byref(cfg)) == L.RN_OK
    assert lib.qknorm_query_config(10, 2, 0, 100, 0, 256, ctypes.byref(cfg)) == L.RN_ERR_UNSUPPORTED


def test_explicit_config_is_checked(lib):
    cfg = L.LaunchConfig()
    cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = 0, 1, 1, 4
    # 64 lanes x 1 vector x 8 < 1024 elements: rejected before any HIP call
    st = lib.rmsnorm_fwd_config(FAKE, FAKE, FAKE, FAKE + 0x1000, FAKE + 0x2000, None, None, None, 4, 1024, 1e-6, BF,
                                ctypes.byref(cfg), None)
    assert st == L.RN_ERR_INVALID_ARG
    cfg.waves_per_row, cfg.vecs_per_lane = 16, 8  # 1024 threads with 8 vectors per lane: not built
    st = lib.rmsnorm_fwd_config(FAKE, FAKE, FAKE, FAKE + 0x1000, FAKE + 0x2000, None, None, None, 4, 1024, 1e-6, BF,
                                ctypes.byref(cfg), None)
    assert st == L.RN_ERR_INVALID_ARG
    cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = 2, 1, 5  # grid above rows
    st = lib.rmsnorm_fwd_config(FAKE, FAKE, FAKE, FAKE + 0x1000, FAKE + 0x2000, None, None, None, 4, 1024, 1e-6, BF,
                                ctypes.byref(cfg), None)
    assert st == L.RN_ERR_INVALID_ARG


# --- partial inputs ---------------------------------------------------------

def _parts_ptrs(*ptrs):
    return (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)


P0, P1, P2 = FAKE + 0x10000, FAKE + 0x20000, FAKE + 0x30000


def _pfwd(lib, parts=(P0, P1), n=None, res=FAKE, w=FAKE, out=FAKE + 0x1000, res_out=FAKE + 0x2000, scale=None,
          amax=None, ts=None, rows=4, hidden=1024, eps=1e-6, flags=BF):
    arr = None if parts is None else _parts_ptrs(*parts)
    return lib.rmsnorm_fwd_partials(arr, len(parts or ()) if n is None else n, res, w, out, res_out, scale, amax, ts,
                                    rows, hidden, eps, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), L.RN_ERR_INVALID_ARG),
    (dict(n=9, parts=(P0,) * 9), L.RN_ERR_INVALID_ARG),
    (dict(n=-1), L.RN_ERR_INVALID_ARG),
    (dict(parts=None, n=2), L.RN_ERR_INVALID_ARG),
    (dict(parts=(P0, None)), L.RN_ERR_INVALID_ARG),
    (dict(parts=(P0, P1 + 8)), L.RN_ERR_MISALIGNED),
    (dict(parts=(P0, FAKE + 0x2000)), L.RN_ERR_INVALID_ARG),  # residual_out is a partial
    (dict(res_out=FAKE + 0x1000), L.RN_ERR_INVALID_ARG),  # out == residual_out
    (dict(res=None), L.RN_ERR_INVALID_ARG),
    (dict(w=None), L.RN_ERR_INVALID_ARG),
    (dict(hidden=16384 + 8), L.RN_ERR_UNSUPPORTED),  # above 2048 lane vectors with more than one partial
    (dict(flags=_qflags("fp8_e4m3fn", "group128"), hidden=1000, scale=FAKE + 0x3000), L.RN_ERR_UNSUPPORTED),
    (dict(flags=_qflags("fp4_e2m1", "nv16"), scale=FAKE + 0x3000), L.RN_ERR_INVALID_ARG),  # NVFP4 without tensor_scale
    (dict(flags=_qflags("fp4_e2m1", "mx32"), scale=FAKE + 0x3000, ts=FAKE + 0x4000), L.RN_ERR_INVALID_ARG),
    (dict(flags=L.make_flags("bf16", "bf16", "bf16", "fp8_e4m3fn", False)), L.RN_ERR_INVALID_ARG),  # no scale
    (dict(eps=float("nan")), L.RN_ERR_INVALID_ARG),
    (dict(out=P1, flags=L.make_flags("bf16", "bf16", "bf16", "fp8_e4m3fn", False), scale=FAKE + 0x3000),
     L.RN_ERR_INVALID_ARG),  # in place over a partial of another width
    (dict(out=P0, flags=L.make_flags("bf16", "f32", "bf16", "f32", False)), L.RN_ERR_INVALID_ARG),
])
def test_partials_reject_before_any_hip_call(lib, kw, status):
    assert _pfwd(lib, **kw) == status
    assert lib.rn_last_error().decode() != ""


def test_partials_rows_zero_is_a_noop(lib):
    assert lib.rmsnorm_fwd_partials(None, 3, None, None, None, None, None, None, None, 0, 1024, 1e-6, L.make_flags(
        "bf16", None, "bf16", "bf16", False), None) == L.RN_OK
    # the count is still checked
    assert lib.rmsnorm_fwd_partials(None, 0, None, None, None, None, None, None, None, 0, 1024, 1e-6, BF, None) \
        == L.RN_ERR_INVALID_ARG


def test_partials_selector():
    # at most 2 vectors per lane for more than one partial; the single-input
    # tables do not apply to them
    for x, vec, hmax in (("bf16", 8, 16384), ("f32", 4, 8192)):
        for n in (2, 3, 4, 5, 8):
            for hidden in list(range(vec, 4096 + 1, vec * 13)) + [7168, 8192, hmax]:
                if hidden > hmax:
                    continue
                for rows in (1, 64, 256, 257, 2048, 16384):
                    c = R.query_partials_config(rows, hidden, n, x_dtype=x, res_dtype="f32",
                                                out_dtype="bf16", w_dtype="bf16")
                    W, NV = c["waves_per_row"], c["vecs_per_lane"]
                    assert NV in (1, 2) and 1 <= W <= 16 and 64 * W * NV * vec >= hidden, (x, n, hidden, rows, c)
                    assert c["grid"] == rows
    # the rule (no table), the same for every output type: the exact fit at
    # one vector per lane, except 9-15 waves that are not a multiple of 4,
    # past 2 rows per CU, as 8 x 2
    def shape(rows, hidden, n, **kw):
        c = R.query_partials_config(rows, hidden, n, res_dtype="f32", num_cus=256, **kw)
        return c["waves_per_row"], c["vecs_per_lane"]

    for kw in ({}, {"out_dtype": "fp8_e4m3fn"}, {"out_dtype": "fp8_e4m3fn", "scale_scheme": "group128"},
               {"out_dtype": "fp8_e4m3fn", "scale_scheme": "mx32"}, {"out_dtype": "fp4_e2m1", "scale_scheme": "mx32"},
               {"out_dtype": "fp4_e2m1", "scale_scheme": "nv16"}):
        assert shape(2048, 8192, 8, **kw) == (16, 1), kw
        assert shape(5120, 8192, 2, **kw) == (16, 1), kw
        assert shape(3840, 8192, 4, **kw) == (16, 1), kw
        assert shape(3072, 7168, 7, **kw) == (8, 2), kw    # 14 x 1 runs behind
        assert shape(513, 7168, 2, **kw) == (8, 2), kw
        assert shape(512, 7168, 4, **kw) == (14, 1), kw   # up to 2 rows per CU: the exact fit
        assert shape(4096, 6144, 8, **kw) == (12, 1), kw  # 12 x 1 runs level or ahead
        assert shape(4096, 5120, 8, **kw) == (8, 2), kw   # 10 waves
        assert shape(256, 4096, 4, **kw) == (8, 1), kw
        assert shape(4096, 4096, 8, **kw) == (8, 1), kw
        assert shape(32, 8192, 8, **kw) == (16, 1), kw    # decode: up to 16 waves
        assert shape(64, 16384, 8, **kw) == (16, 2), kw
        assert shape(2048, 12288, 8, **kw) == (12, 2), kw
    assert shape(8, 2048, 2) == (4, 1)
    assert shape(2048, 8192, 8, out_dtype="fp8_e4m3fn") == (16, 1)
    # one partial is the single-input kernel and its tables
    assert R.query_partials_config(8192, 7168, 1, res_dtype="bf16", out_dtype="fp8_e4m3fn") == \
        R.query_config(8192, 7168, res_dtype="bf16", out_dtype="fp8_e4m3fn")


def test_partials_explicit_config_is_checked(lib):
    cfg = L.LaunchConfig()
    cfg.kernel, cfg.waves_per_row, cfg.vecs_per_lane, cfg.grid = 0, 2, 4, 4  # 4 vectors per lane: not built
    arr = _parts_ptrs(P0, P1, P2)
    st = lib.rmsnorm_fwd_partials_config(arr, 3, FAKE, FAKE, FAKE + 0x1000, FAKE + 0x2000, None, None, None, 4,
                                         1024, 1e-6, BF, ctypes.byref(cfg), None)
    assert st == L.RN_ERR_INVALID_ARG
    st = lib.rmsnorm_fwd_partials_config(arr, 3, FAKE, FAKE, FAKE + 0x1000, FAKE + 0x2000, None, None, None, 4,
                                         1024, 1e-6, BF, None, None)
    assert st == L.RN_ERR_INVALID_ARG
