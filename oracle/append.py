"""Appending a decode step's new tokens to a paged KV cache, with rotary
position embedding (RoPE) applied to the new keys and the queries.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: the CUTLASS Split KV article (§5.3) requires RoPE to be
applied to the current step's K (and the queries) in a separate step before
the split-KV kernel reads the cache, which must not change while it runs; the
FlashAttention capstone (§4.1) stores the cache in fixed 16-token physical
blocks addressed through a per-request block table, a new block being taken
every 16 tokens. The pages do not print RoPE's formula; the reading here is the
rotary embedding as published with RoFormer: dimension pair i of a head
vector is rotated by the angle pos * theta_i with theta_i = base^(-2i/d), for
i < d/2. Two pairings are in use and both are provided: ``interleaved`` pairs
dimensions (2i, 2i+1), ``half`` pairs (i, i + d/2).

Positions follow the multi-query reading of the decode path: with the
sequence lengths *after* the append (L_b) and n new tokens per sequence, new
token j sits at position L_b - n + j, i.e. in block table entry
(L_b - n + j) // 16, slot (L_b - n + j) % 16.

Stored values are the exact rotation divided by the head's scale (1 when no
scales are given) and rounded once to the cache's format, round-to-nearest-
even (``round_to_format``); an FP8 cache stores the E4M3 code, saturated to
the largest finite magnitude (448).
Arithmetic is float64.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import as_f64
from .fp8 import decode_e4m3

try:
    import torch
except Exception:  # pragma: no cover
    torch = None

# (mantissa bits, smallest normal exponent, largest finite value) per format
FORMATS = {
    "f16": (10, -14, 65504.0),
    "bf16": (7, -126, float.fromhex("0x1.fep127")),
    "e4m3": (3, -6, 448.0),
}


def round_to_format(x, fmt: str, saturate: bool = False) -> np.ndarray:
    """Round float64 values to the nearest value of a binary floating-point
    format (ties to even mantissa), with its subnormals. Overflow gives +-inf,
    or the largest finite magnitude when ``saturate``. NaN stays NaN."""
    mbits, emin, fmax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat, res = x.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat):
        if v != v or v == 0.0 or math.isinf(v):
            res[i] = v
            continue
        _, E = math.frexp(v)        # |v| = m * 2^E with 0.5 <= m < 1
        e = max(E - 1, emin)        # the exponent of v's binade (subnormals share emin)
        quantum = math.ldexp(1.0, e - mbits)
        n = v / quantum             # exact: division by a power of two
        r = math.floor(n)
        frac = n - r
        if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
            r += 1
        val = math.copysign(r * quantum, v)  # a tiny negative rounds to -0
        if abs(val) > fmax:
            val = math.copysign(fmax if saturate else math.inf, v)
        res[i] = val
    return out


def e4m3_code(value: float) -> int:
    """The E4M3 code of a value the format represents exactly."""
    if value != value:
        return 0x7F
    sign = 0x80 if math.copysign(1.0, value) < 0 else 0
    a = abs(value)
    if a < 2.0 ** -6:
        mant = a / 2.0 ** -9
        assert mant == int(mant)
        return sign | int(mant)
    _, E = math.frexp(a)
    e = E - 1
    mant = (a / 2.0 ** e - 1.0) * 8
    assert mant == int(mant) and -6 <= e <= 8
    return sign | ((e + 7) << 3) | int(mant)


def rope_angles(pos: int, d: int, base: float) -> np.ndarray:
    """pos * theta_i for the d/2 pairs, theta_i = base^(-2i/d)."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    return float(pos) * theta


def rope_pairs(d: int, style: str):
    """Index arrays (a, b): pair i rotates dimensions a[i] and b[i]."""
    i = np.arange(d // 2)
    if style == "interleaved":
        return 2 * i, 2 * i + 1
    if style == "half":
        return i, i + d // 2
    raise ValueError(f"unknown RoPE style {style!r}")


def rope_rotate(x, pos: int, base: float, style: str) -> np.ndarray:
    """Rotate each pair (x_a, x_b) of the last axis by the pair's angle:
    (x_a cos - x_b sin, x_a sin + x_b cos). ``style`` None leaves x as is."""
    x = as_f64(x).copy()
    if style is None:
        return x
    d = x.shape[-1]
    a, b = rope_pairs(d, style)
    ang = rope_angles(pos, d, base)
    c, s = np.cos(ang), np.sin(ang)
    xa, xb = x[..., a].copy(), x[..., b].copy()
    x[..., a] = xa * c - xb * s
    x[..., b] = xa * s + xb * c
    return x


def _cache_fmt(dtype) -> str:
    return {torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "e4m3"}[dtype]


def _store(values: np.ndarray, dtype, scale: float = 1.0):
    """float64 values -> a CPU tensor of the cache dtype, rounded once (RNE)."""
    fmt = _cache_fmt(dtype)
    if fmt == "e4m3":
        r = round_to_format(values / scale, "e4m3", saturate=True)
        codes = np.array([e4m3_code(v) for v in r.reshape(-1)], dtype=np.uint8).reshape(r.shape)
        return torch.from_numpy(codes).view(torch.float8_e4m3fn)
    r = round_to_format(values / scale, fmt)
    return torch.from_numpy(r).to(dtype)  # exact: r is representable


def append_kv(k_cache, v_cache, block_table, seq_lens, k_new, v_new, q=None, *, rope_style=None,
              rope_base: float = 10000.0, k_scale=None, v_scale=None, page_size: int = 16):
    """The cache after the append, and the rotated queries.

    k_cache, v_cache: [P, page_size, Hkv, d] (CPU tensors, any cache dtype);
    k_new, v_new: [B, n, Hkv, d]; q: [B, n, Hq, d] or None; seq_lens: lengths
    after the append. Returns (k_cache', v_cache', q') as new tensors: new
    token j of sequence b goes to position L_b - n + j; K and q are rotated
    at that position, K/V divided by the head's scale and rounded to the cache
    format. Every other slot keeps its bytes.
    """
    kc, vc = k_cache.clone(), v_cache.clone()
    B, n, hkv, d = k_new.shape
    lens = [int(x) for x in (seq_lens.tolist() if hasattr(seq_lens, "tolist") else seq_lens)]
    table = block_table.cpu().numpy() if hasattr(block_table, "cpu") else np.asarray(block_table)
    ks = as_f64(k_scale) if k_scale is not None else np.ones(hkv)
    vs = as_f64(v_scale) if v_scale is not None else np.ones(hkv)
    qr = None
    if q is not None:
        qr = np.empty(tuple(q.shape))
    for b in range(B):
        for j in range(n):
            pos = lens[b] - n + j
            if pos < 0:
                raise ValueError("a sequence is shorter than its new tokens")
            page, slot = int(table[b, pos // page_size]), pos % page_size
            kr = rope_rotate(k_new[b, j], pos, rope_base, rope_style)   # [Hkv, d]
            vv = as_f64(v_new[b, j])
            for g in range(hkv):
                kc[page, slot, g] = _store(kr[g], kc.dtype, float(ks[g]))
                vc[page, slot, g] = _store(vv[g], vc.dtype, float(vs[g]))
            if q is not None:
                qr[b, j] = rope_rotate(q[b, j], pos, rope_base, rope_style)
    q_out = None
    if q is not None:
        q_out = _store(qr, q.dtype)
    return kc, vc, q_out


def cache_values(cache, scale=None) -> np.ndarray:
    """float64 values of a cache tensor (codes decoded, times the head scale)."""
    x = as_f64(cache)
    if scale is not None:
        x = x * as_f64(scale)[None, None, :, None]
    return x


__all__ = ["append_kv", "cache_values", "decode_e4m3", "e4m3_code", "rope_angles", "rope_pairs",
           "rope_rotate", "round_to_format"]
