"""Plain fp64 decode attention and the split/merge algebra it is built from.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources, by page title and section:
  * FlashAttention 全景演进与大模型 Token 生成全链路性能优化实战 (the
    FlashAttention capstone): §1.1 defines attention as softmax(QK^T/sqrt(d))V;
    §1.2 gives the safe softmax (subtract the row max), the worked example with
    blocks [2, 4] and [3, 5], and the proof that two blocks' (max, sum) merge
    exactly; §2.3 (FlashDecoding) splits the KV sequence of a single decode
    query into chunks, computes a local softmax and output per chunk and
    merges the chunks with the online-softmax identity; §4.1 maps logical
    token positions to fixed 16-token physical blocks through a per-request
    block table; §4.2 lets a group of query heads share one KV head (GQA).
  * 注意力算子、算子融合与 CUDA Graph: "Decode 的注意力是另一种形状" states the
    same split-along-KV-length method and that the merged result equals the
    one-shot computation exactly.
  * The lpnh.cn memory-wall article, §2.2: the tile-by-tile running max m and
    running sum l, with the old statistics rescaled by exp(m_old - m_new)
    before each new tile is added, and a single division at the end.

Readings where the pages leave a step open:
  * several query tokens per sequence (the verification pass of speculative
    decoding, FlashAttention capstone §4.5: the target model scores K draft
    tokens appended to the input in one pass) are the last q_len positions
    of the cache; query i attends to tokens 0 .. L - q_len + i (causal);
  * a split that holds no token a query may see has statistics m = -inf,
    l = 0, O = 0 (the max and sum over an empty set);
  * merging finished partials rescales both sides: O = sum_s e^{m_s-M} O_s,
    l = sum_s e^{m_s-M} l_s (the capstone's two-block identity applied to
    every split);
  * LSE is the natural log of the sum of exp over the *scaled* scores;
  * query head h reads KV head h // (Hq / Hkv) (contiguous groups);
  * tokens at or past a sequence's length never contribute (masking, not
    padding with copies of the last token);
  * a zero-length sequence has no defined output and is rejected;
  * an FP8 cache holds OCP E4M3 codes; the value attention sees is the code's
    value times a per-KV-head scale, one for K and one for V (``oracle.fp8``).

Arithmetic is float64 throughout; inputs (fp16/bf16 tensors or arrays) are
converted exactly. Library primitives used as steps: matrix-vector products,
``numpy.exp``/``numpy.log`` and ``max``/``sum`` reductions.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .fp8 import decode_e4m3, is_fp8

try:  # torch is only used to read bf16 tensors exactly
    import torch
except Exception:  # pragma: no cover
    torch = None


# ------------------------------------------------------------------ inputs


def as_f64(x) -> np.ndarray:
    """Exact conversion of an fp16/bf16/fp32 array or CPU tensor to float64;
    E4M3 code tensors are decoded by the format's definition."""
    if is_fp8(x):
        return decode_e4m3(x)
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _lens(seq_lens) -> List[int]:
    if torch is not None and isinstance(seq_lens, torch.Tensor):
        return [int(t) for t in seq_lens.tolist()]
    return [int(t) for t in seq_lens]


def logical_kv(k, v, seq_lens, b: int, g: int, block_table=None, page_size: int = 0,
               k_scale=None, v_scale=None):
    """Rows 0..L_b-1 of KV head ``g`` of sequence ``b``, as float64 [L_b, d].

    Contiguous caches pack the sequences one after another along the token
    axis. Paged caches find token t in physical block ``block_table[b, t //
    page_size]`` at slot ``t % page_size`` (FlashAttention capstone, §4.1).
    ``k_scale`` / ``v_scale`` (one value per KV head, or None for 1) multiply
    the rows of head ``g``.
    """
    lens = _lens(seq_lens)
    L = lens[b]
    if L <= 0:
        raise ValueError("a sequence needs at least one token")
    if page_size:
        npg = (L + page_size - 1) // page_size
        row = block_table[b, :npg]
        if torch is not None and isinstance(row, torch.Tensor):
            row = row.cpu().numpy()
        table = np.asarray(row, dtype=np.int64)
        idx = table if torch is None or not isinstance(k, torch.Tensor) else torch.from_numpy(table)
        kr = k[idx].reshape(npg * page_size, k.shape[2], k.shape[3])[:L, g, :]
        vr = v[idx].reshape(npg * page_size, v.shape[2], v.shape[3])[:L, g, :]
    else:
        start = sum(lens[:b])
        kr = k[start:start + L, g, :]
        vr = v[start:start + L, g, :]
    K, V = as_f64(kr), as_f64(vr)
    if k_scale is not None:
        K = K * float(as_f64(k_scale)[g])
    if v_scale is not None:
        V = V * float(as_f64(v_scale)[g])
    return K, V


# ------------------------------------------------------- the plain definition


def attention_row(q, K, V, scale: float):
    """softmax(scale * K q) V for one query row, with its log-sum-exp.

    Steps follow the FlashAttention capstone §1.1 (definition) and §1.2 (safe
    softmax in three passes: row max, sum of exp(x - max), divide):
      s_t = scale * <q, K_t>;  m = max_t s_t;  e_t = exp(s_t - m);  l = sum e_t
      o = sum_t e_t V_t / l;   lse = m + ln l
    Returns (o [d], lse, m, l).
    """
    q = as_f64(q)
    K = as_f64(K)
    V = as_f64(V)
    if K.shape[0] == 0:
        raise ValueError("a sequence needs at least one token")
    s = (K @ q) * scale
    m = float(np.max(s))
    e = np.exp(s - m)
    l = float(np.sum(e))
    o = (e @ V) / l
    return o, m + math.log(l), m, l


def block_stats(x) -> Tuple[float, float]:
    """(m, l) of a block of scores: its max and sum of exp(x - max).

    The per-block statistics of the FlashAttention capstone §1.2 worked example.
    """
    x = as_f64(x)
    m = float(np.max(x))
    return m, float(np.sum(np.exp(x - m)))


def merge_two(mA: float, lA: float, OA, mB: float, lB: float, OB):
    """Merge two blocks' unnormalised statistics into those of their union.

    FlashAttention capstone §1.2 formal proof: with m = max(mA, mB),
    l = lA e^{mA-m} + lB e^{mB-m}; the output accumulator is rescaled the same
    way, O = OA e^{mA-m} + OB e^{mB-m} (both sides rescaled, since both are
    finished partials).
    """
    m = max(mA, mB)
    a = math.exp(mA - m)
    b = math.exp(mB - m)
    return m, lA * a + lB * b, as_f64(OA) * a + as_f64(OB) * b


def merge_partials(O_s, m_s, l_s):
    """Normalised output and LSE from per-split (O_s, m_s, l_s).

    The cross-chunk reduce of FlashDecoding (FlashAttention capstone §2.3):
    M = max_s m_s; w_s = exp(m_s - M); l = sum_s w_s l_s;
    o = sum_s w_s O_s / l; lse = M + ln l.
    ``O_s`` is [S, d] unnormalised (O_s = sum over the split of e^{s_t - m_s} V_t).
    """
    O_s = as_f64(O_s)
    m_s = as_f64(m_s)
    l_s = as_f64(l_s)
    M = float(np.max(m_s))
    w = np.exp(m_s - M)
    l = float(np.sum(w * l_s))
    o = (w @ O_s) / l
    return o, M + math.log(l)


def online_softmax_row(q, K, V, scale: float, tile: int):
    """One query row by the running-statistics recurrence over tiles of K/V.

    The lpnh.cn memory-wall article §2.2 (and the FlashAttention capstone's
    lab 1 walk-through): start from m = -inf, l = 0, O = 0; for each tile of
    scores S: m_new = max(m, max S); P = exp(S - m_new); rescale the old
    statistics by alpha = exp(m - m_new): l = alpha l + sum P,
    O = alpha O + P V_tile; m = m_new. Divide O by l once after the last tile.
    Returns (o, lse, m, l).
    """
    q = as_f64(q)
    K = as_f64(K)
    V = as_f64(V)
    n = K.shape[0]
    if n == 0:
        raise ValueError("a sequence needs at least one token")
    m = -math.inf
    l = 0.0
    O = np.zeros(V.shape[1])
    for j in range(0, n, tile):
        S = (K[j:j + tile] @ q) * scale
        m_new = max(m, float(np.max(S)))
        P = np.exp(S - m_new)
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        l = alpha * l + float(np.sum(P))
        O = alpha * O + P @ V[j:j + tile]
        m = m_new
    return O / l, m + math.log(l), m, l


# ------------------------------------------------------------ split / merge


def split_bounds(L: int, chunk: int) -> List[Tuple[int, int]]:
    """Token ranges of the splits of a length-L sequence with chunk size C.

    FlashDecoding cuts the KV sequence into consecutive chunks
    (FlashAttention capstone §2.3): split s covers [s C, min((s+1) C, L)),
    for s < ceil(L / C), so every split holds at least one token.
    """
    if L <= 0 or chunk <= 0:
        raise ValueError("L and chunk must be positive")
    return [(s, min(s + chunk, L)) for s in range(0, L, chunk)]


def _split_partial(q, K, V, scale: float):
    """(O_s unnormalised, m_s, l_s) of one split: its local softmax statistics."""
    s = (K @ q) * scale
    m = float(np.max(s))
    e = np.exp(s - m)
    return e @ V, m, float(np.sum(e))


# ------------------------------------------------------------------ batches


def _pairs(batch: int, hq: int, pairs: Optional[Iterable[Tuple[int, int]]]):
    if pairs is None:
        return [(b, h) for b in range(batch) for h in range(hq)]
    return [(int(b), int(h)) for b, h in pairs]


def decode_attention(q, k, v, seq_lens, scale: float, block_table=None, page_size: int = 0,
                     pairs: Optional[Sequence[Tuple[int, int]]] = None, k_scale=None, v_scale=None):
    """Exact decode attention for a batch: out [B, Hq, d] and lse [B, Hq] (fp64).

    For each sequence b and query head h, with KV head g = h // (Hq / Hkv)
    (FlashAttention capstone §4.2, contiguous groups), ``attention_row`` over
    the sequence's logical rows. ``pairs`` restricts the work to some (b, h);
    entries not computed are NaN. ``k_scale`` / ``v_scale``: per-KV-head
    dequantisation scales (see ``logical_kv``).
    """
    qf = as_f64(q)
    B, hq, d = qf.shape
    hkv = k.shape[-2]
    G = hq // hkv
    out = np.full((B, hq, d), np.nan)
    lse = np.full((B, hq), np.nan)
    todo = {}
    for b, h in _pairs(B, hq, pairs):
        todo.setdefault((b, h // G), []).append(h)
    for (b, g), heads in sorted(todo.items()):
        K, V = logical_kv(k, v, seq_lens, b, g, block_table, page_size, k_scale, v_scale)
        for h in heads:
            o, ls, _, _ = attention_row(qf[b, h], K, V, scale)
            out[b, h] = o
            lse[b, h] = ls
    return out, lse


def decode_attention_multi(q, k, v, seq_lens, scale: float, block_table=None, page_size: int = 0,
                           k_scale=None, v_scale=None, rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Several query tokens per sequence: q [B, q_len, Hq, d] -> out
    [B, q_len, Hq, d], lse [B, q_len, Hq] (fp64).

    Query i of sequence b is the token at position L_b - q_len + i and
    attends to tokens 0 .. L_b - q_len + i (causal among the new tokens;
    FlashAttention capstone §4.5). Each query is ``attention_row`` over its
    visible prefix. With q_len = L_b this is causal attention over the whole
    sequence (prefill). ``rows`` restricts the work to some (b, i, h); entries
    not computed are NaN.
    """
    qf = as_f64(q)
    B, ql, hq, d = qf.shape
    hkv = k.shape[-2]
    G = hq // hkv
    lens = _lens(seq_lens)
    out = np.full((B, ql, hq, d), np.nan)
    lse = np.full((B, ql, hq), np.nan)
    todo = {}
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(ql) for h in range(hq)]
    for b, i, h in rows:
        todo.setdefault((int(b), int(h) // G), []).append((int(i), int(h)))
    for (b, g), items in sorted(todo.items()):
        if lens[b] < ql:
            raise ValueError("every sequence must hold its q_len new tokens")
        K, V = logical_kv(k, v, seq_lens, b, g, block_table, page_size, k_scale, v_scale)
        for i, h in items:
            n = lens[b] - ql + i + 1
            o, ls, _, _ = attention_row(qf[b, i, h], K[:n], V[:n], scale)
            out[b, i, h] = o
            lse[b, i, h] = ls
    return out, lse


def _splits_of(lens: List[int], chunk: Optional[int], bounds) -> List[List[Tuple[int, int]]]:
    """Token ranges of every sequence's splits: consecutive chunks of ``chunk``
    tokens, or the ranges ``bounds[b]`` a caller gives (any cut of [0, L_b)
    into consecutive ranges; the statistics of each range follow the same
    definition)."""
    if bounds is None:
        return [split_bounds(L, chunk) for L in lens]
    out = [[(int(lo), int(hi)) for lo, hi in bounds[b]] for b in range(len(lens))]
    for b, rs in enumerate(out):
        if not rs or rs[0][0] != 0 or rs[-1][1] != lens[b] or any(
                lo >= hi or (i and rs[i - 1][1] != lo) for i, (lo, hi) in enumerate(rs)):
            raise ValueError(f"bounds of sequence {b} do not cut [0, {lens[b]}) into consecutive ranges")
    return out


def decode_partials(q, k, v, seq_lens, scale: float, chunk: Optional[int], block_table=None,
                    page_size: int = 0, max_splits: Optional[int] = None,
                    pairs: Optional[Sequence[Tuple[int, int]]] = None, k_scale=None, v_scale=None,
                    bounds=None):
    """Per-split statistics for every (b, h): O [B, Hq, S, d] (unnormalised),
    m [B, Hq, S] and l [B, Hq, S], S = max_b ceil(L_b / chunk). Splits a
    sequence does not have are NaN. ``bounds`` (a list of (lo, hi) token
    ranges per sequence) replaces the chunk cut.

    With several queries per sequence (q [B, q_len, Hq, d]) the row index is
    i * Hq + h and each query sees its causal prefix; a split past that
    prefix has m = -inf, l = 0, O = 0."""
    qf = as_f64(q)
    cuts = _splits_of(_lens(seq_lens), chunk, bounds)
    if qf.ndim == 4:
        B, ql, hq, d = qf.shape
        return _decode_partials_multi(qf, k, v, seq_lens, scale, cuts, block_table, page_size, max_splits,
                                      k_scale, v_scale)
    B, hq, d = qf.shape
    hkv = k.shape[-2]
    G = hq // hkv
    lens = _lens(seq_lens)
    S = max(len(c) for c in cuts) if max_splits is None else max_splits
    O = np.full((B, hq, S, d), np.nan)
    m = np.full((B, hq, S), np.nan)
    l = np.full((B, hq, S), np.nan)
    todo = {}
    for b, h in _pairs(B, hq, pairs):
        todo.setdefault((b, h // G), []).append(h)
    for (b, g), heads in sorted(todo.items()):
        K, V = logical_kv(k, v, seq_lens, b, g, block_table, page_size, k_scale, v_scale)
        for si, (lo, hi) in enumerate(cuts[b]):
            for h in heads:
                O[b, h, si], m[b, h, si], l[b, h, si] = _split_partial(qf[b, h], K[lo:hi], V[lo:hi], scale)
    return O, m, l


def _decode_partials_multi(qf, k, v, seq_lens, scale, cuts, block_table, page_size, max_splits,
                           k_scale=None, v_scale=None):
    B, ql, hq, d = qf.shape
    hkv = k.shape[-2]
    G = hq // hkv
    lens = _lens(seq_lens)
    S = max(len(c) for c in cuts) if max_splits is None else max_splits
    O = np.full((B, ql * hq, S, d), np.nan)
    m = np.full((B, ql * hq, S), np.nan)
    l = np.full((B, ql * hq, S), np.nan)
    for b in range(B):
        for g in range(hkv):
            K, V = logical_kv(k, v, seq_lens, b, g, block_table, page_size, k_scale, v_scale)
            for si, (lo, hi) in enumerate(cuts[b]):
                for i in range(ql):
                    top = min(hi, lens[b] - ql + i + 1)
                    for h in range(g * G, (g + 1) * G):
                        r = i * hq + h
                        if top <= lo:
                            O[b, r, si], m[b, r, si], l[b, r, si] = 0.0, -math.inf, 0.0
                        else:
                            O[b, r, si], m[b, r, si], l[b, r, si] = _split_partial(qf[b, i, h], K[lo:top], V[lo:top], scale)
    return O, m, l
