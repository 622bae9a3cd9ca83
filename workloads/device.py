"""Moving the generator's arrays to the device and results back.

Storage conversions only (bf16 bit patterns, float32 values, 8-bit codes);
no arithmetic of the method.  Used by the tests, the smoke check and the
benchmark alike.
"""

from __future__ import annotations

import numpy as np
import torch

TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8_e4m3fn": torch.float8_e4m3fn,
                "fp4_e2m1": torch.float4_e2m1fn_x2}


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """A generator array (bf16 bits as uint16, or float32 values) as a device tensor of ``dtype``."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    raise ValueError(dtype)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Stored bits/values: bf16 -> uint16 bits, f32 -> float32, fp8 / fp4 pairs / E8M0 -> uint8."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.float4_e2m1fn_x2, torch.float8_e8m0fnu):
        return t.view(torch.uint8).cpu().numpy()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    raise ValueError(t.dtype)
