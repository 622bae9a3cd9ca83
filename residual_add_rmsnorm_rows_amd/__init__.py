"""MI355X-native (gfx950) row kernels: fused residual add + RMSNorm (with x
given whole or as a sum of up to 8 partials), per-head QK-norm and SwiGLU
(SiLU-and-mul), with bf16 / f32 outputs or quantized ones
(fp8 e4m3fn with a per-row or per-128 scale, MXFP8 / MXFP4 with E8M0 scales per
32, NVFP4 with E4M3FN scales per 16 and a tensor scale).

Thin torch-facing binding over the C ABI in include/rmsnorm_rows.h: it checks
tensors, allocates outputs with torch, and passes raw device pointers and the
current HIP stream to the library.  Every step of the computation runs in the
library's HIP kernels; nothing here computes, and nothing falls back to the CPU.
"""

from __future__ import annotations

import ctypes
from typing import NamedTuple, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import LaunchConfig, RNError, check, lib, make_flags

__all__ = [
    "NormOutput",
    "fused_add_rmsnorm",
    "fused_partials_add_rmsnorm",
    "prepare_fused_add_rmsnorm",
    "PreparedCall",
    "rmsnorm",
    "qk_norm",
    "silu_mul",
    "query_silu_mul_config",
    "query_config",
    "query_partials_config",
    "query_qknorm_config",
    "RNError",
    "LaunchConfig",
    "lib",
]

_NAMES = {torch.bfloat16: "bf16", torch.float32: "f32", torch.float8_e4m3fn: "fp8_e4m3fn",
          torch.float4_e2m1fn_x2: "fp4_e2m1"}
_GROUP = {"row": None, "group128": 128, "mx32": 32, "nv16": 16}
_SCALE_DTYPE = {"row": torch.float32, "group128": torch.float32, "mx32": torch.float8_e8m0fnu,
                "nv16": torch.float8_e4m3fn}
_TORCH = {v: k for k, v in _NAMES.items()}


class NormOutput(NamedTuple):
    out: torch.Tensor
    residual_out: Optional[torch.Tensor]
    scale: Optional[torch.Tensor]  # quantized output: float32 [rows] / [rows, H/128], E8M0 [rows, H/32]
                                   # or E4M3FN [rows, H/16] (NVFP4)
    amax: Optional[torch.Tensor]   # quantized output when requested: float32, one per scale


def _name(dtype: torch.dtype, what: str) -> str:
    if dtype not in _NAMES:
        raise TypeError(f"{what}: unsupported dtype {dtype}")
    return _NAMES[dtype]


def _dev_tensor(t: torch.Tensor, what: str, device: torch.device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a tensor")
    if t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _quant_buffers(od: str, scale_scheme: str, rows: int, n: int, device: torch.device, return_amax: bool,
                   tensor_scale) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Scale (and amax) outputs of a quantized output, and the NVFP4 tensor scale
    as a one-element float32 device tensor."""
    if scale_scheme not in _GROUP:
        raise ValueError(f"scale_scheme must be one of {sorted(_GROUP)}")
    if (scale_scheme == "nv16") != (tensor_scale is not None):
        raise ValueError("tensor_scale is given exactly for scale_scheme='nv16'")
    ts = None
    if tensor_scale is not None:
        if isinstance(tensor_scale, torch.Tensor):
            _dev_tensor(tensor_scale, "tensor_scale", device)
            if tensor_scale.dtype != torch.float32 or tensor_scale.numel() != 1:
                raise ValueError("tensor_scale must be a one-element float32 tensor")
            ts = tensor_scale
        else:
            ts = torch.tensor([float(tensor_scale)], dtype=torch.float32, device=device)
    scale = amax = None
    if od in ("fp8_e4m3fn", "fp4_e2m1"):
        g = _GROUP[scale_scheme]
        nscale = (rows,) if g is None else (rows, n // g if n % g == 0 else 0)
        scale = torch.empty(nscale, dtype=_SCALE_DTYPE[scale_scheme], device=device)
        if return_amax:
            amax = torch.empty(nscale, dtype=torch.float32, device=device)
    return scale, amax, ts


def _rows_setup(x: torch.Tensor, residual: Optional[torch.Tensor], weight: torch.Tensor,
                weight_plus_one: bool, out_dtype: Optional[torch.dtype], out: Optional[torch.Tensor],
                residual_out: Optional[torch.Tensor], return_amax: bool, scale_scheme: str, tensor_scale):
    """Checks of a rows call (x stands for the shape and dtype of the input);
    allocates the outputs that were not given.  Returns (rows, H, out,
    residual_out, scale, amax, tensor_scale, flags)."""
    device = x.device
    if device.type != "cuda":
        raise ValueError("x must be a device tensor")
    _dev_tensor(x, "x", device)
    H = x.shape[-1]
    rows = x.numel() // H if H else 0
    xd = _name(x.dtype, "x")
    rd = None
    if residual is not None:
        _dev_tensor(residual, "residual", device)
        if residual.shape != x.shape:
            raise ValueError(f"residual shape {tuple(residual.shape)} != x shape {tuple(x.shape)}")
        rd = _name(residual.dtype, "residual")
    _dev_tensor(weight, "weight", device)
    if weight.shape != (H,):
        raise ValueError(f"weight shape {tuple(weight.shape)} != ({H},)")
    wd = _name(weight.dtype, "weight")
    od_t = out_dtype if out_dtype is not None else (out.dtype if out is not None else x.dtype)
    od = _name(od_t, "out")
    out_shape = x.shape if od != "fp4_e2m1" else (*x.shape[:-1], H // 2)
    if od == "fp4_e2m1" and H % 2:
        raise ValueError("fp4 output needs an even hidden size")
    if out is None:
        out = torch.empty(out_shape, dtype=od_t, device=device)
    else:
        _dev_tensor(out, "out", device)
        if tuple(out.shape) != tuple(out_shape) or out.dtype != od_t:
            raise ValueError("out has the wrong shape or dtype")
    if residual is not None:
        if residual_out is None:
            residual_out = torch.empty_like(residual)
        else:
            _dev_tensor(residual_out, "residual_out", device)
            if residual_out.shape != residual.shape or residual_out.dtype != residual.dtype:
                raise ValueError("residual_out must match residual's shape and dtype")
    elif residual_out is not None:
        raise ValueError("residual_out given without residual")
    scale, amax, ts = _quant_buffers(od, scale_scheme, rows, H, device, return_amax, tensor_scale)
    flags = make_flags(xd, rd, wd, od, weight_plus_one, scale_scheme)
    return rows, H, out, residual_out, scale, amax, ts, flags


def fused_add_rmsnorm(x: torch.Tensor, residual: Optional[torch.Tensor], weight: torch.Tensor,
                      eps: float, *, weight_plus_one: bool = False,
                      out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                      residual_out: Optional[torch.Tensor] = None, return_amax: bool = False,
                      scale_scheme: str = "row", tensor_scale=None,
                      config: Optional[LaunchConfig] = None) -> NormOutput:
    """``residual_out = x + residual``; ``out = RMSNorm(residual_out) * (w [+ 1])``.

    ``x`` is [..., H] (bf16 or f32), ``residual`` the same shape (x dtype or
    f32) or None, ``weight`` [H].  ``out_dtype`` is bf16, f32,
    ``torch.float8_e4m3fn`` or ``torch.float4_e2m1fn_x2`` (two codes per byte,
    [..., H/2]).  Quantized outputs carry scales per ``scale_scheme``:
    ``"row"`` (fp8; float32 [rows]), ``"group128"`` (fp8; float32
    [rows, H/128]), ``"mx32"`` (fp8 or fp4; E8M0 ``torch.float8_e8m0fnu``
    [rows, H/32]) or ``"nv16"`` (fp4; E4M3FN ``torch.float8_e4m3fn``
    [rows, H/16], with the per-tensor float32 ``tensor_scale``: a
    one-element device tensor, or a number copied to the device).
    ``out=x`` (when out has x's dtype width) and ``residual_out=residual`` are
    allowed (in place).  ``config`` forces a launch configuration.
    """
    rows, H, out, residual_out, scale, amax, ts, flags = _rows_setup(
        x, residual, weight, weight_plus_one, out_dtype, out, residual_out, return_amax, scale_scheme, tensor_scale)
    L = lib()
    if config is not None:
        st = L.rmsnorm_fwd_config(_p(x), _p(residual), _p(weight), _p(out), _p(residual_out), _p(scale),
                                  _p(amax), _p(ts), rows, H, eps, flags, ctypes.byref(config), _stream(x.device))
    else:
        st = L.rmsnorm_fwd_ex(_p(x), _p(residual), _p(weight), _p(out), _p(residual_out), _p(scale),
                              _p(amax), _p(ts), rows, H, eps, flags, _stream(x.device))
    check(st)
    return NormOutput(out, residual_out, scale, amax)


class PreparedCall:
    """One C-ABI call with every argument marshalled once.

    For decode-sized calls issued many times on the same buffers (a serving
    loop outside graph capture): the tensors, flags, sizes and stream are
    written into the library's call record (``rn_rmsnorm_call``) when the
    object is built, so a call is a single foreign-function call with one
    argument, and no tensor inspection, output allocation or stream lookup.
    ``result`` holds the output tensors, which every call overwrites.  The
    object keeps its tensors alive.
    """

    __slots__ = ("_fn", "_arg", "result", "_keep")

    def __init__(self, fn, arg, result, keep):
        self._fn = fn
        self._arg = arg
        self.result = result
        self._keep = keep

    def __call__(self):
        st = self._fn(self._arg)
        if st:
            check(st)
        return self.result


def prepare_fused_add_rmsnorm(x: torch.Tensor, residual: Optional[torch.Tensor], weight: torch.Tensor,
                              eps: float, *, weight_plus_one: bool = False,
                              out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                              residual_out: Optional[torch.Tensor] = None, return_amax: bool = False,
                              scale_scheme: str = "row", tensor_scale=None,
                              stream: Optional[torch.cuda.Stream] = None) -> PreparedCall:
    """``fused_add_rmsnorm`` over fixed buffers, prepared once and called many
    times: ``call = prepare_fused_add_rmsnorm(...); call()`` launches it on
    ``stream`` (default: the current stream when prepared) and returns the
    ``NormOutput`` it writes.  The arguments and checks are those of
    ``fused_add_rmsnorm``; the library re-checks them on every call."""
    rows, H, out, residual_out, scale, amax, ts, flags = _rows_setup(
        x, residual, weight, weight_plus_one, out_dtype, out, residual_out, return_amax, scale_scheme, tensor_scale)
    s = stream.cuda_stream if stream is not None else _stream(x.device)
    rec = _lib.RmsnormCall(_p(x), _p(residual), _p(weight), _p(out), _p(residual_out), _p(scale), _p(amax), _p(ts),
                           rows, H, eps, flags, s)
    # the entry point called through a prototype whose argument is already of
    # the declared type: no conversion per call
    fn = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.POINTER(_lib.RmsnormCall))(
        ctypes.cast(lib().rmsnorm_fwd_call, ctypes.c_void_p).value)
    result = NormOutput(out, residual_out, scale, amax)
    call = PreparedCall(fn, ctypes.pointer(rec), result, (x, residual, weight, ts, rec))
    call()  # a first call: any argument error is raised here
    return call


def fused_partials_add_rmsnorm(partials: Sequence[torch.Tensor], residual: Optional[torch.Tensor],
                               weight: torch.Tensor, eps: float, *, weight_plus_one: bool = False,
                               out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                               residual_out: Optional[torch.Tensor] = None, return_amax: bool = False,
                               scale_scheme: str = "row", tensor_scale=None,
                               config: Optional[LaunchConfig] = None) -> NormOutput:
    """``fused_add_rmsnorm`` with ``x = partials[0] + partials[1] + ...``: the
    kernel takes the exact sum of the partials (and the residual) and rounds it
    once, to the residual dtype (or float32 without a residual).

    ``partials`` holds 1..8 tensors of one shape and dtype (bf16 or f32): the
    partial outputs of a row-parallel projection, or the branch outputs of a
    parallel residual block.  Outputs, scale schemes and ``tensor_scale`` are
    those of ``fused_add_rmsnorm``.  ``out`` may be one of the partials (in
    place) when it has the partials' dtype width.
    """
    parts = list(partials)
    if not 1 <= len(parts) <= _lib.MAX_PARTIALS:
        raise ValueError(f"1..{_lib.MAX_PARTIALS} partials expected, got {len(parts)}")
    x = parts[0]
    for i, p in enumerate(parts):
        _dev_tensor(p, f"partials[{i}]", x.device)
        if p.shape != x.shape or p.dtype != x.dtype:
            raise ValueError(f"partials[{i}] has shape {tuple(p.shape)} / {p.dtype}, "
                             f"partials[0] has {tuple(x.shape)} / {x.dtype}")
    rows, H, out, residual_out, scale, amax, ts, flags = _rows_setup(
        x, residual, weight, weight_plus_one, out_dtype, out, residual_out, return_amax, scale_scheme, tensor_scale)
    ptrs = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    L = lib()
    if config is not None:
        st = L.rmsnorm_fwd_partials_config(ptrs, len(parts), _p(residual), _p(weight), _p(out), _p(residual_out),
                                           _p(scale), _p(amax), _p(ts), rows, H, eps, flags, ctypes.byref(config),
                                           _stream(x.device))
    else:
        st = L.rmsnorm_fwd_partials(ptrs, len(parts), _p(residual), _p(weight), _p(out), _p(residual_out),
                                    _p(scale), _p(amax), _p(ts), rows, H, eps, flags, _stream(x.device))
    check(st)
    return NormOutput(out, residual_out, scale, amax)


def rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float, **kw) -> NormOutput:
    """RMSNorm over the last dimension, no residual (see ``fused_add_rmsnorm``)."""
    return fused_add_rmsnorm(x, None, weight, eps, **kw)


def _head_view(t: torch.Tensor, what: str, device: torch.device) -> Tuple[int, int, int, int]:
    if t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")
    if t.dim() != 3:
        raise ValueError(f"{what} must be [tokens, heads, head_dim]")
    T, nh, D = t.shape
    if t.stride(2) != 1 or (nh > 1 and t.stride(1) != D):
        raise ValueError(f"{what}: heads must be contiguous inside a token")
    stride = t.stride(0) if T > 1 else nh * D
    return T, nh, D, stride


def _qk_flags(dtype: str, w_dtype: str, weight_plus_one: bool) -> int:
    f = (_lib.DTYPE_CODES[dtype] << _lib.RN_FLAGS_X_SHIFT) | (_lib.DTYPE_CODES[w_dtype] << _lib.RN_FLAGS_W_SHIFT)
    return f | (_lib.RN_FLAG_WEIGHT_PLUS_ONE if weight_plus_one else 0)


def qk_norm(q: torch.Tensor, k: Optional[torch.Tensor], q_weight: torch.Tensor,
            k_weight: Optional[torch.Tensor], eps: float, *, weight_plus_one: bool = False,
            inplace: bool = True, config: Optional[LaunchConfig] = None
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Per-head RMSNorm of ``q`` [T, nq, D] and ``k`` [T, nk, D] over D (64, 128 or 256).

    Views with a token stride (e.g. slices of a fused QKV buffer) are accepted.
    ``inplace=True`` (the page's form) overwrites q and k; otherwise new
    tensors with the same layout are returned.  ``config`` forces a launch
    configuration (rows_per_lane, block_threads).
    """
    device = q.device
    if device.type != "cuda":
        raise ValueError("q must be a device tensor")
    T, nq, D, qs = _head_view(q, "q", device)
    td = _name(q.dtype, "q")
    nk, ks = 0, 0
    if k is not None:
        Tk, nk, Dk, ks = _head_view(k, "k", device)
        if Tk != T or Dk != D or k.dtype != q.dtype:
            raise ValueError("k must have q's tokens, head_dim and dtype")
        if k_weight is None:
            raise ValueError("k_weight is required with k")
    _dev_tensor(q_weight, "q_weight", device)
    if q_weight.shape != (D,):
        raise ValueError("q_weight must be [head_dim]")
    wd = _name(q_weight.dtype, "q_weight")
    if k is not None:
        _dev_tensor(k_weight, "k_weight", device)
        if k_weight.shape != (D,) or k_weight.dtype != q_weight.dtype:
            raise ValueError("k_weight must be [head_dim] with q_weight's dtype")
    if inplace:
        q_out, k_out = q, k
    else:
        q_out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=device)
        k_out = None if k is None else torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=device)
    flags = _qk_flags(td, wd, weight_plus_one)
    args = (_p(q), _p(k), _p(q_weight), _p(k_weight if k is not None else None), _p(q_out), _p(k_out),
            T, nq, nk, D, qs, ks, eps, flags)
    if config is not None:
        st = lib().qknorm_fwd_config(*args, ctypes.byref(config), _stream(device))
    else:
        st = lib().qknorm_fwd(*args, _stream(device))
    check(st)
    return q_out, k_out


def query_config(rows: int, hidden: int, *, x_dtype: str = "bf16", res_dtype: Optional[str] = None,
                 w_dtype: str = "bf16", out_dtype: str = "bf16", weight_plus_one: bool = False,
                 scale_scheme: str = "row", num_cus: int = 256) -> dict:
    """The launch configuration the selector picks (host only with an explicit
    ``num_cus``; ``num_cus=0`` queries the current device)."""
    cfg = LaunchConfig()
    flags = make_flags(x_dtype, res_dtype, w_dtype, out_dtype, weight_plus_one, scale_scheme)
    check(lib().rmsnorm_query_config(rows, hidden, flags, int(res_dtype is not None), num_cus,
                                     ctypes.byref(cfg)))
    return cfg.as_dict()


def query_partials_config(rows: int, hidden: int, num_partials: int, *, x_dtype: str = "bf16",
                          res_dtype: Optional[str] = None, w_dtype: str = "bf16", out_dtype: str = "bf16",
                          weight_plus_one: bool = False, scale_scheme: str = "row", num_cus: int = 256) -> dict:
    """The launch configuration ``fused_partials_add_rmsnorm`` would use."""
    cfg = LaunchConfig()
    flags = make_flags(x_dtype, res_dtype, w_dtype, out_dtype, weight_plus_one, scale_scheme)
    check(lib().rmsnorm_partials_query_config(rows, hidden, num_partials, flags, int(res_dtype is not None),
                                              num_cus, ctypes.byref(cfg)))
    return cfg.as_dict()


def query_qknorm_config(tokens: int, num_q_heads: int, num_k_heads: int, head_dim: int, *,
                        dtype: str = "bf16", w_dtype: str = "bf16", num_cus: int = 256) -> dict:
    cfg = LaunchConfig()
    flags = _qk_flags(dtype, w_dtype, False)
    check(lib().qknorm_query_config(tokens, num_q_heads, num_k_heads, head_dim, flags, num_cus,
                                    ctypes.byref(cfg)))
    return cfg.as_dict()


def silu_mul(x: torch.Tensor, *, out_dtype: Optional[torch.dtype] = None, scale_scheme: str = "row",
             return_amax: bool = False, out: Optional[torch.Tensor] = None, tensor_scale=None,
             config: Optional[LaunchConfig] = None) -> NormOutput:
    """SwiGLU: ``silu(x[..., :d]) * x[..., d:]`` for ``x`` [..., 2 d] (bf16 or f32).

    Outputs as for ``fused_add_rmsnorm`` (bf16, f32, fp8 e4m3fn with per-row /
    per-128 / MX scales, fp4 e2m1 with MX or NVFP4 scales); ``residual_out``
    is None.
    """
    device = x.device
    if device.type != "cuda":
        raise ValueError("x must be a device tensor")
    _dev_tensor(x, "x", device)
    if x.shape[-1] % 2:
        raise ValueError("the last dimension of x must be 2 d (gate, then up)")
    d = x.shape[-1] // 2
    rows = x.numel() // x.shape[-1] if x.shape[-1] else 0
    xd = _name(x.dtype, "x")
    od_t = out_dtype if out_dtype is not None else (out.dtype if out is not None else x.dtype)
    od = _name(od_t, "out")
    out_shape = (*x.shape[:-1], d // 2 if od == "fp4_e2m1" else d)
    if out is None:
        out = torch.empty(out_shape, dtype=od_t, device=device)
    else:
        _dev_tensor(out, "out", device)
        if tuple(out.shape) != tuple(out_shape) or out.dtype != od_t:
            raise ValueError("out has the wrong shape or dtype")
    scale, amax, ts = _quant_buffers(od, scale_scheme, rows, d, device, return_amax, tensor_scale)
    flags = (_lib.DTYPE_CODES[xd] << _lib.RN_FLAGS_X_SHIFT) | (_lib.DTYPE_CODES[od] << _lib.RN_FLAGS_OUT_SHIFT)
    flags |= _lib.SCALE_SCHEMES[scale_scheme] << _lib.RN_FLAGS_SCALE_SHIFT
    L = lib()
    if config is not None:
        st = L.silu_mul_fwd_config(_p(x), _p(out), _p(scale), _p(amax), _p(ts), rows, d, flags,
                                   ctypes.byref(config), _stream(device))
    else:
        st = L.silu_mul_fwd(_p(x), _p(out), _p(scale), _p(amax), _p(ts), rows, d, flags, _stream(device))
    check(st)
    return NormOutput(out, None, scale, amax)


def query_silu_mul_config(rows: int, d: int, *, x_dtype: str = "bf16", out_dtype: str = "bf16",
                          scale_scheme: str = "row", num_cus: int = 256) -> dict:
    """The launch configuration silu_mul picks (host only with an explicit
    ``num_cus``; ``num_cus=0`` queries the current device)."""
    cfg = LaunchConfig()
    flags = (_lib.DTYPE_CODES[x_dtype] << _lib.RN_FLAGS_X_SHIFT) | (_lib.DTYPE_CODES[out_dtype] << _lib.RN_FLAGS_OUT_SHIFT)
    flags |= _lib.SCALE_SCHEMES[scale_scheme] << _lib.RN_FLAGS_SCALE_SHIFT
    check(lib().silu_mul_query_config(rows, d, flags, num_cus, ctypes.byref(cfg)))
    return cfg.as_dict()
