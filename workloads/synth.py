"""Seeded synthetic KV caches shaped like the decode workloads on the pages.

Shapes follow the pages' decode examples: batch 1 with 32 heads of
dimension 128 (the CUTLASS Split KV article, §2), 128K-token contexts (same
article, §2), grouped-query heads (FlashAttention 全景演进 capstone, §4.2) and
16-token KV pages (same capstone, §4.1). Values are N(0, 1) drawn in fp32
and rounded once to fp16/bf16 with round-to-nearest-even.

Every random draw comes from ``numpy.random.default_rng`` under a
``SeedSequence`` whose children are taken in a fixed order
(lengths, q, K, V, spike rows, page permutation). Large tensors are drawn in
fixed-size chunks, each with its own child seed, so the result does not depend
on how many threads generate it.

FP8 caches (``quantize_kv_fp8``) store each K/V element as an OCP E4M3 code of
the drawn value divided by a per-KV-head scale (the head's largest magnitude
over 448, the format's largest finite value), rounded by torch's cast.

Nothing here computes attention: the module draws numbers and places them in
the cache layouts. Slots that no valid token occupies are filled with NaN so
that any read past a sequence's end shows up in the output.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence, Union

import numpy as np
import torch

_CHUNK = 1 << 23  # elements per independently seeded chunk
_WORKERS = max(1, min(16, os.cpu_count() or 1))

CONFIG_NAMES = {
    1: "tiny_mha_b1_h8_d64_L1024_f16_splits4",
    2: "mha_b1_h32_d128_L32768_f16",
    3: "mha_b1_h32_d128_L131072_f16_spikes",
    4: "gqa_b16_hq32_hkv8_d128_L1024-16384_bf16_varlen",
    5: "paged_gqa_b64_hq64_hkv8_d128_L512-32768_bf16_page16",
}


def poison_value() -> float:
    """The value written into cache slots no valid token occupies."""
    return float("nan")


@dataclass
class Workload:
    """One decode-attention problem: a query token per sequence and its KV cache.

    Layouts (all row-major, contiguous):
      q            [B, Hq, d], or [B, q_len, Hq, d] with several query tokens
      k, v         contiguous: [sum(L_b) + pad_rows, Hkv, d]; sequence b
                   occupies rows [start_b, start_b + L_b), start_b the sum of
                   the lengths before it; the pad rows hold NaN.
                   paged: [P, page_size, Hkv, d] pools.
      seq_lens     int32 [B]
      block_table  int32 [B, max_pages_per_seq] (paged only); entries past a
                   sequence's last page point at a NaN-filled spare page.
      k_scale, v_scale  float32 [Hkv] for an FP8 cache (element value =
                   scale[g] * code value), else None.
    ``dtype`` is q's dtype; ``kv_dtype`` the cache's.
    """

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: torch.dtype
    scale: float
    page_size: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    seq_lens: torch.Tensor
    block_table: Optional[torch.Tensor] = None
    max_pages_per_seq: int = 0
    force_num_splits: int = 0
    pad_rows: int = 0
    seed: int = 0
    meta: dict = field(default_factory=dict)
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    @property
    def kv_dtype(self) -> torch.dtype:
        return self.k.dtype

    @property
    def q_len(self) -> int:
        return 1 if self.q.dim() == 3 else int(self.q.shape[1])

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def lens(self) -> list:
        return [int(x) for x in self.seq_lens.tolist()]

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lens))

    @property
    def paged(self) -> bool:
        return self.page_size > 0

    def seq_starts(self) -> list:
        """Row where each sequence begins in the packed contiguous layout."""
        starts, acc = [], 0
        for n in self.lens:
            starts.append(acc)
            acc += n
        return starts


# ---------------------------------------------------------------- drawing


def _child(ss: np.random.SeedSequence, *key: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(entropy=ss.entropy, spawn_key=tuple(ss.spawn_key) + tuple(key))


def _normal_into(out: torch.Tensor, ss: np.random.SeedSequence) -> None:
    """Fill ``out`` (fp16/bf16, contiguous) with N(0,1) drawn in fp32 chunks."""
    flat = out.view(-1)
    n = flat.numel()
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        rng = np.random.default_rng(_child(ss, c))
        buf = np.empty(hi - lo, dtype=np.float32)
        rng.standard_normal(out=buf, dtype=np.float32)
        flat[lo:hi].copy_(torch.from_numpy(buf).to(out.dtype))

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_WORKERS) as ex:
            list(ex.map(work, range(nchunks)))


def _draw_lengths(spec, batch: int, ss: np.random.SeedSequence) -> list:
    rng = np.random.default_rng(ss)
    if isinstance(spec, (list, tuple)) and spec and isinstance(spec[0], str):
        kind, lo, hi = spec
        if kind == "uniform":
            lens = rng.integers(lo, hi + 1, size=batch)
        elif kind == "loguniform":
            u = rng.uniform(math.log(lo), math.log(hi), size=batch)
            lens = np.clip(np.rint(np.exp(u)), lo, hi)
        else:
            raise ValueError(f"unknown length distribution {kind!r}")
        return [int(x) for x in lens]
    lens = [int(x) for x in spec]
    if len(lens) != batch:
        raise ValueError("need one length per sequence")
    return lens


def _scatter_pages(packed: torch.Tensor, lens: Sequence[int], page_size: int,
                   table: np.ndarray, num_pages: int) -> torch.Tensor:
    """Copy packed token rows into a page pool following ``table``.

    Layout only: row t of sequence b goes to pool[table[b, t // page], t % page].
    Every pool slot no token lands in holds NaN.
    """
    hkv, d = packed.shape[1], packed.shape[2]
    pool = torch.full((num_pages, page_size, hkv, d), poison_value(), dtype=packed.dtype)
    start = 0
    for b, n in enumerate(lens):
        full, rem = divmod(n, page_size)
        for p in range(full + (1 if rem else 0)):
            rows = page_size if p < full else rem
            src = packed[start + p * page_size: start + p * page_size + rows]
            pool[int(table[b, p]), :rows].copy_(src)
        start += n
    return pool


def make_workload(
    *,
    name: str = "custom",
    batch: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    seq_lens: Union[Sequence[int], tuple],
    dtype: torch.dtype = torch.float16,
    page_size: int = 0,
    seed: int = 0,
    scale: Optional[float] = None,
    spike_fraction: float = 0.0,
    spike_factor: float = 4.0,
    force_num_splits: int = 0,
    pad_rows: int = 16,
    spare_pages: int = 8,
    permute_pages: bool = True,
    max_pages_per_seq: Optional[int] = None,
    q_len: int = 1,
) -> Workload:
    """Draw one workload. ``seq_lens`` is a list of lengths, or a tuple
    ``("uniform", lo, hi)`` (integers, both ends included) or
    ``("loguniform", lo, hi)`` (rounded, clamped to [lo, hi]). With
    ``q_len`` > 1, q is [B, q_len, Hq, d]: the queries of the last q_len
    tokens of each cache."""
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    root = np.random.SeedSequence(seed)
    ss_len, ss_q, ss_k, ss_v, ss_spike, ss_page = root.spawn(6)

    lens = _draw_lengths(seq_lens, batch, ss_len)
    total = int(sum(lens))

    q_shape = (batch, num_q_heads, head_dim) if q_len == 1 else (batch, q_len, num_q_heads, head_dim)
    q = torch.empty(q_shape, dtype=dtype)
    _normal_into(q, ss_q)
    k = torch.empty((total + pad_rows, num_kv_heads, head_dim), dtype=dtype)
    v = torch.empty((total + pad_rows, num_kv_heads, head_dim), dtype=dtype)
    _normal_into(k[:total], ss_k)
    _normal_into(v[:total], ss_v)
    if pad_rows:
        k[total:] = poison_value()
        v[total:] = poison_value()

    meta = {"spike_rows": None}
    if spike_fraction > 0:
        rng = np.random.default_rng(ss_spike)
        nspike = int(round(spike_fraction * total))
        rows = np.sort(rng.choice(total, size=nspike, replace=False))
        idx = torch.from_numpy(rows.astype(np.int64))
        k[idx] = k[idx] * spike_factor  # a power of two: exact in fp16/bf16
        meta["spike_rows"] = rows

    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)

    wl = Workload(
        name=name, batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, dtype=dtype, scale=float(scale), page_size=0,
        q=q, k=k, v=v, seq_lens=torch.tensor(lens, dtype=torch.int32),
        force_num_splits=force_num_splits, pad_rows=pad_rows, seed=seed, meta=meta,
    )
    if page_size:
        wl = to_paged(wl, page_size, ss_page, spare_pages=spare_pages,
                      permute=permute_pages, max_pages_per_seq=max_pages_per_seq)
    return wl


def to_paged(wl: Workload, page_size: int, ss_page=None, *, spare_pages: int = 8,
             permute: bool = True, max_pages_per_seq: Optional[int] = None) -> Workload:
    """Move a contiguous workload's tokens into a page pool with a block table.

    Pages are dealt to sequences in order from a seeded permutation of the
    pool (or in pool order when ``permute`` is False). The first spare page is
    the one unused table entries point at; all spare pages hold NaN.
    """
    if wl.paged:
        raise ValueError("already paged")
    lens = wl.lens
    npages = [(n + page_size - 1) // page_size for n in lens]
    used = int(sum(npages))
    spare = max(1, spare_pages)
    num_pages = used + spare
    if permute:
        if ss_page is None:
            ss_page = np.random.SeedSequence(wl.seed).spawn(6)[5]
        order = np.random.default_rng(ss_page).permutation(num_pages)
    else:
        order = np.arange(num_pages)
    mp = max(npages) if max_pages_per_seq is None else int(max_pages_per_seq)
    if mp < max(npages):
        raise ValueError("max_pages_per_seq too small for the longest sequence")
    filler = int(order[used])  # a spare, NaN-filled page
    table = np.full((wl.batch, mp), filler, dtype=np.int32)
    off = 0
    for b, n in enumerate(npages):
        table[b, :n] = order[off: off + n]
        off += n
    total = wl.total_tokens
    kp = _scatter_pages(wl.k[:total], lens, page_size, table, num_pages)
    vp = _scatter_pages(wl.v[:total], lens, page_size, table, num_pages)
    meta = dict(wl.meta)
    meta["filler_page"] = filler
    return Workload(
        name=wl.name, batch=wl.batch, num_q_heads=wl.num_q_heads,
        num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim, dtype=wl.dtype,
        scale=wl.scale, page_size=page_size, q=wl.q, k=kp, v=vp,
        seq_lens=wl.seq_lens, block_table=torch.from_numpy(table),
        max_pages_per_seq=mp, force_num_splits=wl.force_num_splits, pad_rows=0,
        seed=wl.seed, meta=meta, k_scale=wl.k_scale, v_scale=wl.v_scale,
    )


_FP8_MAX = 448.0  # largest finite E4M3 magnitude


def _fp8_codes(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """E4M3 codes of x / scale (per KV head, the second-to-last axis), cast
    in token chunks to bound host memory. NaN stays NaN (code 0x7F)."""
    out = torch.empty(x.shape, dtype=torch.float8_e4m3fn)
    step = max(1, _CHUNK // max(1, x[0].numel()))
    shape = (1,) * (x.dim() - 2) + (scale.numel(), 1)
    inv = (1.0 / scale.float()).view(shape)
    for lo in range(0, x.shape[0], step):
        out[lo:lo + step] = (x[lo:lo + step].float() * inv).to(torch.float8_e4m3fn)
    return out


def _head_amax(x: torch.Tensor) -> torch.Tensor:
    """Largest finite magnitude per KV head (the second-to-last axis)."""
    hkv = x.shape[-2]
    flat = x.reshape(-1, hkv, x.shape[-1])
    amax = torch.zeros(hkv, dtype=torch.float32)
    step = max(1, _CHUNK // max(1, flat[0].numel()))
    for lo in range(0, flat.shape[0], step):
        blk = flat[lo:lo + step].float().abs()
        blk = torch.nan_to_num(blk, nan=0.0)
        amax = torch.maximum(amax, blk.amax(dim=(0, 2)))
    return amax


def quantize_kv_fp8(wl: Workload) -> Workload:
    """The same workload with an FP8 (OCP E4M3) cache: per KV head, scale =
    amax / 448 and code = e4m3(x / scale), separately for K and V. q stays in
    its 16-bit type. Poisoned (NaN) slots stay NaN."""
    def quant(x):
        amax = _head_amax(x)
        scale = torch.where(amax > 0, amax / _FP8_MAX, torch.ones_like(amax)).to(torch.float32)
        return _fp8_codes(x, scale), scale

    kq, ks = quant(wl.k)
    vq, vs = quant(wl.v)
    meta = dict(wl.meta)
    return Workload(
        name=wl.name + "_fp8", batch=wl.batch, num_q_heads=wl.num_q_heads,
        num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim, dtype=wl.dtype,
        scale=wl.scale, page_size=wl.page_size, q=wl.q, k=kq, v=vq,
        seq_lens=wl.seq_lens, block_table=wl.block_table, max_pages_per_seq=wl.max_pages_per_seq,
        force_num_splits=wl.force_num_splits, pad_rows=wl.pad_rows, seed=wl.seed, meta=meta,
        k_scale=ks, v_scale=vs,
    )


def make_config(i: int, seed: Optional[int] = None, q_len: int = 1, kv_fp8: bool = False) -> Workload:
    """The five decode workloads, numbered 1..5 (tiny MHA, 32K MHA, 128K MHA
    with key spikes, GQA varlen, paged GQA). Seeds default to 1000 + i. With
    q_len > 1 each sequence carries that many query tokens (its last q_len
    cache positions); the name gets a ``_q<q_len>`` suffix. ``kv_fp8`` stores
    the cache as E4M3 codes with per-head scales (``quantize_kv_fp8``)."""
    s = 1000 + i if seed is None else seed
    if kv_fp8:
        return quantize_kv_fp8(make_config(i, seed, q_len))
    if q_len > 1:
        wl = make_config(i, seed, 1)
        q = torch.empty((wl.batch, q_len, wl.num_q_heads, wl.head_dim), dtype=wl.dtype)
        _normal_into(q, np.random.SeedSequence([s, q_len]))
        wl.q = q
        wl.name = f"{wl.name}_q{q_len}"
        return wl
    name = CONFIG_NAMES[i]
    if i == 1:
        return make_workload(name=name, batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64,
                             seq_lens=[1024], dtype=torch.float16, seed=s, force_num_splits=4)
    if i == 2:
        return make_workload(name=name, batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128,
                             seq_lens=[32768], dtype=torch.float16, seed=s)
    if i == 3:
        return make_workload(name=name, batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128,
                             seq_lens=[131072], dtype=torch.float16, seed=s,
                             spike_fraction=0.01, spike_factor=4.0)
    if i == 4:
        return make_workload(name=name, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             seq_lens=("uniform", 1024, 16384), dtype=torch.bfloat16, seed=s)
    if i == 5:
        return make_workload(name=name, batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128,
                             seq_lens=("loguniform", 512, 32768), dtype=torch.bfloat16, seed=s,
                             page_size=16, max_pages_per_seq=32768 // 16)
    raise ValueError(f"no config {i}")


PREFILL_NAME = "prefill_gqa_b1_hq32_hkv8_d128_L8192_bf16_causal"


def make_prefill(seed: int = 2000, length: int = 8192, dtype: torch.dtype = torch.bfloat16) -> Workload:
    """Causal prefill of one 8192-token prompt: every token is a query
    (q [1, L, 32, 128]), 8 KV heads (group 4), d = 128, N(0,1) values."""
    wl = make_workload(name=PREFILL_NAME if (length, dtype) == (8192, torch.bfloat16) else
                       f"prefill_gqa_b1_hq32_hkv8_d128_L{length}_{str(dtype).split('.')[-1]}_causal",
                       batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=[length], dtype=dtype,
                       seed=seed, q_len=length)
    wl.q = wl.q.reshape(1, length, 32, 128)
    return wl


APPEND_NAME = "append_rope_half_b1_hq32_hkv8_d128_n8192_bf16_paged"


def make_append(seed: int = 2100, length: int = 8192, dtype: torch.dtype = torch.bfloat16):
    """The KV append before a prefill: one 8192-token prompt's new keys and
    values (k_new, v_new [1, L, 8, 128], N(0,1)) to be written, rotated, into a
    16-token paged pool whose pages are a seeded permutation (the pool's old
    contents are N(0,1) too, spare pages NaN), and its queries (q [1, L, 32,
    128]) rotated in place. Returns (workload, k_new, v_new); the workload's
    lengths are those after the append."""
    wl = make_workload(name=APPEND_NAME if (length, dtype) == (8192, torch.bfloat16) else
                       f"append_rope_half_b1_hq32_hkv8_d128_n{length}_{str(dtype).split('.')[-1]}_paged",
                       batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=[length], dtype=dtype,
                       seed=seed, q_len=length)
    wl = to_paged(wl, 16, spare_pages=2)
    wl.q = wl.q.reshape(1, length, 32, 128)
    ss = np.random.SeedSequence(seed + 1)
    k_new = torch.empty((1, length, 8, 128), dtype=dtype)
    v_new = torch.empty((1, length, 8, 128), dtype=dtype)
    _normal_into(k_new, _child(ss, 0))
    _normal_into(v_new, _child(ss, 1))
    return wl, k_new, v_new
