"""Planted mistakes in the oracle must fail at least one pin.

Each mutant is a copy of one oracle function with one plausible error (a
flipped sign, a dropped term, a wrong index). It is swapped in with
monkeypatch, on the CPU, and the pins of ``test_oracle.py`` that cover that
function are run; at least one must fail.
"""

import math

import numpy as np
import pytest

import oracle.attention as A
import oracle.append as AP
import oracle.fp8 as F
import tests.test_oracle as P
import tests.test_oracle_append as PA


def _merge_two_flipped_sign(mA, lA, OA, mB, lB, OB):
    m = max(mA, mB)
    a, b = math.exp(m - mA), math.exp(m - mB)
    return m, lA * a + lB * b, A.as_f64(OA) * a + A.as_f64(OB) * b


def _merge_partials_unweighted_l(O_s, m_s, l_s):
    O_s, m_s, l_s = A.as_f64(O_s), A.as_f64(m_s), A.as_f64(l_s)
    M = float(np.max(m_s))
    w = np.exp(m_s - M)
    l = float(np.sum(l_s))
    return (w @ O_s) / l, M + math.log(l)


def _attention_row_no_scale(q, K, V, scale):
    q, K, V = A.as_f64(q), A.as_f64(K), A.as_f64(V)
    s = K @ q
    m = float(np.max(s))
    e = np.exp(s - m)
    l = float(np.sum(e))
    return (e @ V) / l, m + math.log(l), m, l


def _attention_row_unsafe(q, K, V, scale):
    q, K, V = A.as_f64(q), A.as_f64(K), A.as_f64(V)
    s = (K @ q) * scale
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(s)
        l = float(np.sum(e))
        return (e @ V) / l, math.log(l) if l > 0 else float("nan"), float(np.max(s)), l


def _attention_row_lse_log2(q, K, V, scale):
    q, K, V = A.as_f64(q), A.as_f64(K), A.as_f64(V)
    s = (K @ q) * scale
    m = float(np.max(s))
    e = np.exp(s - m)
    l = float(np.sum(e))
    return (e @ V) / l, m + math.log2(l), m, l


def _online_flipped_alpha(q, K, V, scale, tile):
    q, K, V = A.as_f64(q), A.as_f64(K), A.as_f64(V)
    m, l, O = -math.inf, 0.0, np.zeros(V.shape[1])
    for j in range(0, K.shape[0], tile):
        S = (K[j:j + tile] @ q) * scale
        m_new = max(m, float(np.max(S)))
        P = np.exp(S - m_new)
        alpha = math.exp(m_new - m) if m != -math.inf else 0.0
        l = alpha * l + float(np.sum(P))
        O = alpha * O + P @ V[j:j + tile]
        m = m_new
    return O / l, m + math.log(l), m, l


def _online_no_rescale_of_o(q, K, V, scale, tile):
    q, K, V = A.as_f64(q), A.as_f64(K), A.as_f64(V)
    m, l, O = -math.inf, 0.0, np.zeros(V.shape[1])
    for j in range(0, K.shape[0], tile):
        S = (K[j:j + tile] @ q) * scale
        m_new = max(m, float(np.max(S)))
        P = np.exp(S - m_new)
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        l = alpha * l + float(np.sum(P))
        O = O + P @ V[j:j + tile]
        m = m_new
    return O / l, m + math.log(l), m, l


_orig_decode = A.decode_attention


def _decode_head_mod_mapping(q, k, v, seq_lens, scale, block_table=None, page_size=0, pairs=None):
    qf = A.as_f64(q)
    B, hq, d = qf.shape
    hkv = k.shape[-2]
    out = np.full((B, hq, d), np.nan)
    lse = np.full((B, hq), np.nan)
    for b, h in A._pairs(B, hq, pairs):
        K, V = A.logical_kv(k, v, seq_lens, b, h % hkv, block_table, page_size)
        out[b, h], lse[b, h], _, _ = A.attention_row(qf[b, h], K, V, scale)
    return out, lse


_orig_logical = A.logical_kv


def _logical_kv_slot_reversed(k, v, seq_lens, b, g, block_table=None, page_size=0, k_scale=None, v_scale=None):
    if not page_size:
        return _orig_logical(k, v, seq_lens, b, g, block_table, page_size)
    L = A._lens(seq_lens)[b]
    npg = (L + page_size - 1) // page_size
    import torch
    table = block_table[b, :npg].long()
    kk = k[table].flip(1).reshape(npg * page_size, k.shape[2], k.shape[3])[:L, g, :]
    vv = v[table].flip(1).reshape(npg * page_size, v.shape[2], v.shape[3])[:L, g, :]
    return A.as_f64(kk), A.as_f64(vv)


def _split_bounds_drops_tail(L, chunk):
    return [(s, s + chunk) for s in range(0, L - chunk + 1, chunk)] or [(0, L)]


def _multi_causal_off_by_one(q, k, v, seq_lens, scale, block_table=None, page_size=0):
    qf = A.as_f64(q)
    B, ql, hq, d = qf.shape
    hkv = k.shape[-2]
    G = hq // hkv
    lens = A._lens(seq_lens)
    out = np.full((B, ql, hq, d), np.nan)
    lse = np.full((B, ql, hq), np.nan)
    for b in range(B):
        for g in range(hkv):
            K, V = A.logical_kv(k, v, seq_lens, b, g, block_table, page_size)
            for i in range(ql):
                n = max(1, lens[b] - ql + i)
                for h in range(g * G, (g + 1) * G):
                    out[b, i, h], lse[b, i, h], _, _ = A.attention_row(qf[b, i, h], K[:n], V[:n], scale)
    return out, lse


def _e4m3_bias_8(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, mnt = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and mnt == 0x7:
        return math.nan
    if e == 0:
        return sign * (mnt / 8.0) * 2.0 ** (1 - 8)
    return sign * (1.0 + mnt / 8.0) * 2.0 ** (e - 8)


_logical_kv_orig = A.logical_kv


def _logical_kv_scales_swapped(k, v, seq_lens, b, g, block_table=None, page_size=0, k_scale=None, v_scale=None):
    return _logical_kv_orig(k, v, seq_lens, b, g, block_table, page_size, v_scale, k_scale)


def _rope_rotate_flipped(x, pos, base, style):
    x = A.as_f64(x).copy()
    if style is None:
        return x
    a, b = AP.rope_pairs(x.shape[-1], style)
    ang = AP.rope_angles(pos, x.shape[-1], base)
    c, s = np.cos(ang), np.sin(ang)
    xa, xb = x[..., a].copy(), x[..., b].copy()
    x[..., a] = xa * c + xb * s
    x[..., b] = -xa * s + xb * c
    return x


def _rope_angles_wrong_exponent(pos, d, base):
    return float(pos) * np.power(float(base), -1.0 * np.arange(d // 2) / d)


def _round_ties_away(x, fmt, saturate=False):
    mbits, emin, fmax = AP.FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for i, v in enumerate(x.reshape(-1)):
        if v != v or v == 0.0 or math.isinf(v):
            out.reshape(-1)[i] = v
            continue
        e = max(math.frexp(v)[1] - 1, emin)
        q = math.ldexp(1.0, e - mbits)
        val = math.copysign(math.floor(abs(v) / q + 0.5) * q, v)
        if abs(val) > fmax:
            val = math.copysign(fmax if saturate else math.inf, v)
        out.reshape(-1)[i] = val
    return out


_append_orig = AP.append_kv


def _append_position_off_by_one(k_cache, v_cache, block_table, seq_lens, k_new, v_new, q=None, **kw):
    lens = [int(x) + 1 for x in seq_lens.tolist()]
    return _append_orig(k_cache, v_cache, block_table, lens, k_new, v_new, q, **kw)


MUTANTS = [
    ("append:rope_rotate", _rope_rotate_flipped,
     [lambda: PA.test_rope_interleaved_is_complex_multiplication_and_half_is_a_permutation()]),
    ("append:rope_angles", _rope_angles_wrong_exponent,
     [lambda: PA.test_rope_interleaved_is_complex_multiplication_and_half_is_a_permutation()]),
    ("append:round_to_format", _round_ties_away, [PA.test_rounding_ties_and_saturation_closed_forms,
                                                  PA.test_round_to_f16_matches_numpy_float64_cast]),
    ("append:append_kv", _append_position_off_by_one, [lambda: PA.test_append_writes_only_the_new_tokens_slots(1)]),
    ("fp8:e4m3_value", _e4m3_bias_8, [P.test_e4m3_codes_match_torch_float8_e4m3fn, P.test_e4m3_format_closed_forms]),
    ("logical_kv", _logical_kv_scales_swapped, [P.test_fp8_scales_apply_per_kv_head]),
    ("decode_attention_multi", _multi_causal_off_by_one, [lambda: P.test_multi_query_matches_torch_causal_masked_softmax(4)]),
    ("merge_two", _merge_two_flipped_sign,
     [P.test_worked_example_printed_values, lambda: P.test_every_split_merges_to_the_full_row(17)]),
    ("merge_partials", _merge_partials_unweighted_l,
     [P.test_worked_example_closed_form_and_attention_row, lambda: P.test_every_split_merges_to_the_full_row(17)]),
    ("attention_row", _attention_row_no_scale,
     [lambda: P.test_uniform_keys_give_mean_of_v(7, 16), lambda: P.test_matches_torch_float64_softmax(1)]),
    ("attention_row", _attention_row_unsafe, [P.test_large_scores_stay_finite]),
    ("attention_row", _attention_row_lse_log2,
     [P.test_worked_example_closed_form_and_attention_row, lambda: P.test_matches_torch_float64_softmax(2)]),
    ("online_softmax_row", _online_flipped_alpha, [lambda: P.test_running_max_rising_and_falling("rising")]),
    ("online_softmax_row", _online_no_rescale_of_o, [lambda: P.test_online_recurrence_equals_full_softmax(64, 7)]),
    ("decode_attention", _decode_head_mod_mapping, [P.test_gqa_equals_mha_with_repeated_kv_heads]),
    ("logical_kv", _logical_kv_slot_reversed, [P.test_paged_equals_contiguous_for_identity_and_permuted_tables]),
    ("split_bounds", _split_bounds_drops_tail, [lambda: P.test_every_split_merges_to_the_full_row(17)]),
]


@pytest.mark.parametrize("idx", range(len(MUTANTS)), ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, idx):
    name, fn, pins = MUTANTS[idx]
    mod = A
    if name.startswith("fp8:"):
        mod, name = F, name[4:]
    elif name.startswith("append:"):
        mod, name = AP, name[7:]
    monkeypatch.setattr(mod, name, fn)
    caught = 0
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError, ZeroDivisionError):
            caught += 1
    assert caught >= 1, f"no pin caught the planted mistake in {name}"
