"""FP8 (E4M3) KV-cache values for the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name FP8 for attention without fixing a format: the FlashAttention
capstone (§2.2, the FA-3 paragraph) describes FP8 operands with fp32
accumulation and scaling factors that keep values in range, and the CUTLASS
Split KV article (§5.8) raises FP8 for split-KV decode. The reading taken
here: a cache element is stored as an 8-bit code in the OCP FP8 E4M3 format
(1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
encodes subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN; largest
finite magnitude 448), and the value attention sees is that code's value
times a per-KV-head float32 scale, one scale for K and one for V.

``e4m3_value`` writes the format's definition out for one code; everything
else maps codes through it. Arithmetic is float64.
"""

from __future__ import annotations

import math

import numpy as np

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def e4m3_value(code: int) -> float:
    """The real number an E4M3 code stands for (NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """Float64 values of an array of E4M3 codes (uint8 array, or a torch
    float8_e4m3fn / uint8 tensor, read bit for bit)."""
    if torch is not None and isinstance(codes, torch.Tensor):
        codes = codes.detach().to("cpu").contiguous().view(torch.uint8).numpy()
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def is_fp8(x) -> bool:
    """Whether ``x`` is a tensor of E4M3 codes."""
    return torch is not None and isinstance(x, torch.Tensor) and x.dtype == getattr(torch, "float8_e4m3fn", None)
