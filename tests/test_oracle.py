"""Pins for the CPU oracle: facts fixed outside its own code.

Each test checks the oracle against something other than itself: the worked
example printed on the FlashAttention capstone page (§1.2), closed forms
(uniform keys, one dominant key, a single token), brute force over every split
of tiny rows, reductions (GQA equals MHA with repeated KV heads; paged equals
contiguous), invariances (token order, linearity in V) and an independent
library (torch's float64 softmax and logsumexp). ``test_oracle_mutants.py``
plants mistakes in the oracle and checks that these pins catch them.

The functions are looked up on the module at call time so the mutant tests
can swap them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.attention as A
from workloads import make_workload
from workloads.synth import to_paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "online_softmax_worked_example.json")


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ printed values


def test_worked_example_printed_values():
    """Capstone §1.2 tiny calculator: every value the page prints."""
    g = json.load(open(GOLDEN, encoding="utf-8"))
    p = g["printed"]
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-12
    mA, lA = A.block_stats(g["block_A"])
    mB, lB = A.block_stats(g["block_B"])
    assert mA == p["m_A"] and mB == p["m_B"]
    assert abs(lA - p["l_A"]) <= tol and abs(lB - p["l_B"]) <= tol
    m, l, _ = A.merge_two(mA, lA, np.zeros(1), mB, lB, np.zeros(1))
    assert m == p["m_new"]
    assert abs(l - p["l_new"]) <= tol
    assert abs(math.exp(mA - m) - p["rescale_A"]) <= tol
    # the page's intermediate product l_A * e^{-1}: its own printed inputs
    # (1.1353 x 0.3679) round to 0.4177, the exact value is 0.41766...
    assert abs(lA * math.exp(mA - m) - p["l_A_rescaled"]) <= 2 * tol
    mf, lf = A.block_stats(g["block_A"] + g["block_B"])
    assert mf == p["m_new"] and abs(lf - p["l_truth"]) <= tol
    terms = np.exp(np.array(g["block_A"] + g["block_B"], dtype=float) - mf)
    assert np.all(np.abs(terms - np.array(p["full_row_terms"])) <= tol)


def test_worked_example_closed_form_and_attention_row():
    """The same example at full precision: l_A = e^-2 + 1, l = e^-3 + e^-1 + e^-2 + 1,
    and as attention with d = 1, q = [1], scale 1, K = [2, 4, 3, 5]."""
    lA_exact = math.exp(-2) + 1.0
    l_exact = math.exp(-3) + math.exp(-1) + math.exp(-2) + 1.0
    mA, lA = A.block_stats([2, 4])
    mB, lB = A.block_stats([3, 5])
    assert abs(lA - lA_exact) < 1e-15 and abs(lB - lA_exact) < 1e-15
    V = np.array([[1.0], [10.0], [100.0], [1000.0]])
    q = np.array([1.0])
    K = np.array([[2.0], [4.0], [3.0], [5.0]])
    o, lse, m, l = A.attention_row(q, K, V, 1.0)
    assert m == 5.0 and abs(l - l_exact) < 1e-15
    assert abs(lse - (5.0 + math.log(l_exact))) < 1e-14
    o_exact = (math.exp(-3) * 1 + math.exp(-1) * 10 + math.exp(-2) * 100 + 1000) / l_exact
    assert abs(o[0] - o_exact) < 1e-12
    # split at the page's block boundary and merge
    O_s, m_s, l_s = [], [], []
    for lo, hi in A.split_bounds(4, 2):
        Os, ms, ls = A._split_partial(q, K[lo:hi], V[lo:hi], 1.0)
        O_s.append(Os); m_s.append(ms); l_s.append(ls)
    assert m_s == [4.0, 5.0]
    assert abs(l_s[0] - lA_exact) < 1e-15 and abs(l_s[1] - lA_exact) < 1e-15
    om, lsem = A.merge_partials(np.array(O_s), np.array(m_s), np.array(l_s))
    assert abs(om[0] - o_exact) < 1e-12 and abs(lsem - (5.0 + math.log(l_exact))) < 1e-14


# ------------------------------------------------------------- closed forms


@pytest.mark.parametrize("L,d", [(1, 8), (7, 16), (64, 64), (300, 128)])
def test_uniform_keys_give_mean_of_v(L, d):
    r = _rng(L * 31 + d)
    q = r.standard_normal(d)
    krow = r.standard_normal(d)
    K = np.tile(krow, (L, 1))
    V = r.standard_normal((L, d))
    scale = 1 / math.sqrt(d)
    o, lse, _, _ = A.attention_row(q, K, V, scale)
    s = scale * float(np.dot(q, krow))
    assert np.allclose(o, V.mean(axis=0), rtol=0, atol=1e-13)
    assert abs(lse - (s + math.log(L))) < 1e-12
    # q = 0 makes every score zero
    o0, lse0, _, _ = A.attention_row(np.zeros(d), r.standard_normal((L, d)), V, scale)
    assert np.allclose(o0, V.mean(axis=0), rtol=0, atol=1e-13)
    assert abs(lse0 - math.log(L)) < 1e-12


@pytest.mark.parametrize("L,tstar", [(2, 0), (50, 17), (1000, 999)])
def test_dominant_key_selects_its_value_row(L, tstar):
    r = _rng(L + tstar)
    d = 32
    q = r.standard_normal(d)
    q /= np.linalg.norm(q)
    K = r.standard_normal((L, d)) * 0.1
    K[tstar] = q * 60.0  # score 60 against |others| < ~1
    V = r.standard_normal((L, d))
    o, lse, m, _ = A.attention_row(q, K, V, 1.0)
    assert m == pytest.approx(60.0, abs=1e-12)
    assert np.allclose(o, V[tstar], rtol=0, atol=1e-15 * L + 1e-20)
    assert abs(lse - 60.0) < 1e-15 * 60 * 4 + L * math.exp(-55)


def test_single_token():
    r = _rng(3)
    q, k, v = r.standard_normal(64), r.standard_normal((1, 64)), r.standard_normal((1, 64))
    o, lse, m, l = A.attention_row(q, k, v, 0.125)
    assert np.array_equal(o, v[0])
    assert lse == 0.125 * float(k[0] @ q) and l == 1.0


# ----------------------------------------------------------- brute force


@pytest.mark.parametrize("L", [1, 2, 3, 5, 17, 64])
def test_every_split_merges_to_the_full_row(L):
    r = _rng(100 + L)
    d = 8
    q = r.standard_normal(d) * 3
    K = r.standard_normal((L, d))
    V = r.standard_normal((L, d))
    o_ref, lse_ref, _, _ = A.attention_row(q, K, V, 0.7)
    for chunk in range(1, L + 1):
        parts = [A._split_partial(q, K[lo:hi], V[lo:hi], 0.7) for lo, hi in A.split_bounds(L, chunk)]
        o, lse = A.merge_partials(np.array([p[0] for p in parts]), np.array([p[1] for p in parts]),
                                  np.array([p[2] for p in parts]))
        assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-14)
        assert abs(lse - lse_ref) < 1e-12
    # every two-block cut, merged pairwise with the two-block identity
    for cut in range(1, L):
        pa = A._split_partial(q, K[:cut], V[:cut], 0.7)
        pb = A._split_partial(q, K[cut:], V[cut:], 0.7)
        m, l, O = A.merge_two(pa[1], pa[2], pa[0], pb[1], pb[2], pb[0])
        assert np.allclose(O / l, o_ref, rtol=1e-12, atol=1e-14)
        assert abs(m + math.log(l) - lse_ref) < 1e-12


@pytest.mark.parametrize("L,tile", [(1, 1), (10, 3), (64, 1), (64, 7), (256, 64), (1000, 128)])
def test_online_recurrence_equals_full_softmax(L, tile):
    r = _rng(L * 7 + tile)
    d = 16
    q = r.standard_normal(d) * 2
    K = r.standard_normal((L, d))
    V = r.standard_normal((L, d))
    o_ref, lse_ref, m_ref, l_ref = A.attention_row(q, K, V, 0.5)
    o, lse, m, l = A.online_softmax_row(q, K, V, 0.5, tile)
    assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    assert abs(lse - lse_ref) < 1e-12 and m == m_ref and abs(l - l_ref) <= 1e-12 * l_ref


@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_running_max_rising_and_falling(direction):
    """Scores that raise the running max at every tile, and ones that never do
    (the memory-wall article §4.2 names the sign of exp(m_old - m_new) as the
    usual bug)."""
    L, d = 40, 4
    q = np.array([1.0, 0, 0, 0])
    s = np.arange(L, dtype=float) * 0.5
    if direction == "falling":
        s = s[::-1].copy()
    K = np.zeros((L, d)); K[:, 0] = s
    V = np.eye(L, d, dtype=float) + np.arange(L)[:, None] * 0.01
    w = np.exp(s - s.max()); w /= w.sum()
    for tile in (1, 3, 8):
        o, lse, m, _ = A.online_softmax_row(q, K, V, 1.0, tile)
        assert np.allclose(o, w @ V, rtol=1e-12, atol=1e-15)
        assert m == s.max()
        assert abs(lse - (s.max() + math.log(np.exp(s - s.max()).sum()))) < 1e-12


# ------------------------------------------------ independent library routine


@pytest.mark.parametrize("seed", range(5))
def test_matches_torch_float64_softmax(seed):
    r = _rng(seed)
    L = int(r.integers(1, 400))
    d = int(r.choice([1, 8, 64, 128]))
    scale = float(r.uniform(0.05, 2.0))
    q, K, V = r.standard_normal(d), r.standard_normal((L, d)) * 2, r.standard_normal((L, d))
    o, lse, _, _ = A.attention_row(q, K, V, scale)
    tq, tK, tV = (torch.from_numpy(x) for x in (q, K, V))
    logits = (tK @ tq) * scale
    o_t = torch.softmax(logits, dim=0) @ tV
    lse_t = torch.logsumexp(logits, dim=0)
    assert np.allclose(o, o_t.numpy(), rtol=1e-12, atol=1e-14)
    assert abs(lse - float(lse_t)) < 1e-12


# ------------------------------------------------- reductions and invariants


def _wl(**kw):
    base = dict(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=[5, 40, 17],
                dtype=torch.float16, seed=7)
    base.update(kw)
    return make_workload(**base)


def test_gqa_equals_mha_with_repeated_kv_heads():
    wl = _wl()
    G = wl.group_size
    out, lse = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    k_rep = wl.k.repeat_interleave(G, dim=1)
    v_rep = wl.v.repeat_interleave(G, dim=1)
    out2, lse2 = A.decode_attention(wl.q, k_rep, v_rep, wl.seq_lens, wl.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    # and each head against the definition on its own KV head
    qf = A.as_f64(wl.q)
    start = 0
    for b, L in enumerate(wl.lens):
        for h in range(wl.num_q_heads):
            Kr = A.as_f64(wl.k[start:start + L, h // G])
            Vr = A.as_f64(wl.v[start:start + L, h // G])
            o, ls, _, _ = A.attention_row(qf[b, h], Kr, Vr, wl.scale)
            assert np.array_equal(o, out[b, h]) and ls == lse[b, h]
        start += L


def test_paged_equals_contiguous_for_identity_and_permuted_tables():
    wl = _wl(seq_lens=[1, 16, 17, 33, 100], batch=5, dtype=torch.bfloat16)
    ref = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    for permute in (False, True):
        pw = to_paged(wl, 16, permute=permute, spare_pages=3)
        got = A.decode_attention(pw.q, pw.k, pw.v, pw.seq_lens, pw.scale, pw.block_table, 16)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        assert np.isfinite(got[0]).all()


def test_token_permutation_invariance_and_linearity_in_v():
    r = _rng(11)
    L, d = 123, 32
    q, K, V1, V2 = r.standard_normal(d), r.standard_normal((L, d)), r.standard_normal((L, d)), r.standard_normal((L, d))
    o, lse, _, _ = A.attention_row(q, K, V1, 0.3)
    perm = r.permutation(L)
    op, lsep, _, _ = A.attention_row(q, K[perm], V1[perm], 0.3)
    assert np.allclose(o, op, rtol=1e-12, atol=1e-14) and abs(lse - lsep) < 1e-12
    o2, _, _, _ = A.attention_row(q, K, V2, 0.3)
    o12, _, _, _ = A.attention_row(q, K, V1 + 2.5 * V2, 0.3)
    assert np.allclose(o12, o + 2.5 * o2, rtol=1e-12, atol=1e-13)


def test_decode_partials_merge_to_decode_attention():
    wl = _wl(seq_lens=[300, 64, 1], num_q_heads=4, num_kv_heads=4)
    out, lse = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    for chunk in (1, 7, 64, 300):
        O, m, l = A.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, chunk)
        for b, L in enumerate(wl.lens):
            S = len(A.split_bounds(L, chunk))
            assert np.isnan(m[b, :, S:]).all()
            for h in range(wl.num_q_heads):
                o, ls = A.merge_partials(O[b, h, :S], m[b, h, :S], l[b, h, :S])
                assert np.allclose(o, out[b, h], rtol=1e-12, atol=1e-14)
                assert abs(ls - lse[b, h]) < 1e-12


def test_decode_partials_over_given_cuts_merge_to_decode_attention():
    """Any cut of [0, L) into consecutive ranges merges to the full result
    (the split-invariance of capstone §2.3, for cuts that are not a fixed
    chunk: the balanced tile list cuts sequences at arbitrary tile offsets);
    malformed cuts are refused."""
    wl = _wl(seq_lens=[300, 64, 1], num_q_heads=4, num_kv_heads=2)
    out, lse = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    rng = np.random.default_rng(11)
    for _ in range(3):
        cuts = []
        for L in wl.lens:
            inner = sorted(rng.choice(np.arange(1, L), size=min(L - 1, int(rng.integers(0, 5))), replace=False)) \
                if L > 1 else []
            edges = [0, *[int(x) for x in inner], L]
            cuts.append(list(zip(edges[:-1], edges[1:])))
        O, m, l = A.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, None, bounds=cuts)
        for b, rs in enumerate(cuts):
            S = len(rs)
            assert np.isnan(m[b, :, S:]).all()
            for h in range(wl.num_q_heads):
                o, ls = A.merge_partials(O[b, h, :S], m[b, h, :S], l[b, h, :S])
                assert np.allclose(o, out[b, h], rtol=1e-12, atol=1e-14)
                assert abs(ls - lse[b, h]) < 1e-12
    for bad in ([[(0, 150), (151, 300)], [(0, 64)], [(0, 1)]],    # gap
                [[(0, 300)], [(0, 64)], [(0, 2)]],                # past L
                [[(0, 300)], [(0, 32), (32, 32), (32, 64)], [(0, 1)]]):  # empty range
        with pytest.raises(ValueError):
            A.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, None, bounds=bad)


def test_sampled_pairs_match_full_batch():
    wl = _wl()
    out, lse = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    pairs = [(0, 3), (2, 7), (1, 0)]
    o2, l2 = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, pairs=pairs)
    for b, h in pairs:
        assert np.array_equal(o2[b, h], out[b, h]) and l2[b, h] == lse[b, h]
    assert np.isnan(l2[0, 0])


def test_zero_length_is_rejected():
    with pytest.raises(ValueError):
        A.attention_row(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    with pytest.raises(ValueError):
        A.split_bounds(0, 4)


def test_large_scores_stay_finite():
    """The safe softmax subtracts the row max so exp never overflows
    (capstone §1.2): scores near 800 are beyond exp's fp64 range."""
    r = _rng(5)
    d, L = 16, 50
    q = np.ones(d)
    K = 50.0 + r.standard_normal((L, d))
    V = r.standard_normal((L, d))
    o, lse, m, l = A.attention_row(q, K, V, 1.0)
    assert m > 750 and np.isfinite(o).all() and np.isfinite(lse)
    s = K @ q
    w = np.exp(s - s.max()); w /= w.sum()
    assert np.allclose(o, w @ V, rtol=1e-12, atol=1e-14)
    o2, lse2, _, _ = A.online_softmax_row(q, K, V, 1.0, 7)
    assert np.allclose(o2, o, rtol=1e-12, atol=1e-14) and abs(lse2 - lse) < 1e-9



# ------------------------------------------------------- several query tokens


def test_multi_query_with_one_query_is_single_query_decode():
    wl = _wl(seq_lens=[5, 40, 17])
    out, lse = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    o2, l2 = A.decode_attention_multi(wl.q[:, None], wl.k, wl.v, wl.seq_lens, wl.scale)
    assert np.array_equal(o2[:, 0], out) and np.array_equal(l2[:, 0], lse)


@pytest.mark.parametrize("q_len", [2, 4, 7])
def test_multi_query_matches_torch_causal_masked_softmax(q_len):
    """Query i sees tokens 0 .. L - q_len + i: checked against torch's softmax
    over the full row with -inf past each query's limit (an independent
    library and a different way to express the mask)."""
    wl = make_workload(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=[q_len, 50, 130],
                       dtype=torch.bfloat16, seed=q_len, q_len=q_len)
    out, lse = A.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    G = wl.group_size
    start = 0
    for b, L in enumerate(wl.lens):
        K = wl.k[start:start + L].double()
        V = wl.v[start:start + L].double()
        for i in range(q_len):
            for h in range(wl.num_q_heads):
                logits = (K[:, h // G] @ wl.q[b, i, h].double()) * wl.scale
                logits[L - q_len + i + 1:] = -float("inf")
                o = torch.softmax(logits, 0) @ V[:, h // G]
                assert np.allclose(out[b, i, h], o.numpy(), rtol=1e-12, atol=1e-14)
                assert abs(lse[b, i, h] - float(torch.logsumexp(logits, 0))) < 1e-12
        start += L


def test_multi_query_split_statistics_merge_to_the_result():
    wl = make_workload(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=32, seq_lens=[9, 70],
                       dtype=torch.float16, seed=3, q_len=4)
    out, lse = A.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    for chunk in (1, 3, 8, 70):
        O, m, l = A.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, chunk)
        for b, L in enumerate(wl.lens):
            S = -(-L // chunk)
            for i in range(4):
                for h in range(4):
                    r = i * 4 + h
                    # splits past a query's causal limit hold the empty statistics
                    for si in range(S):
                        if si * chunk > L - 4 + i:
                            assert m[b, r, si] == -np.inf and l[b, r, si] == 0 and not O[b, r, si].any()
                    ms = m[b, r, :S]
                    keep = ms > -np.inf
                    o, ls = A.merge_partials(O[b, r, :S][keep], ms[keep], l[b, r, :S][keep])
                    assert np.allclose(o, out[b, i, h], rtol=1e-12, atol=1e-14) and abs(ls - lse[b, i, h]) < 1e-12


def test_multi_query_rejects_short_caches():
    wl = make_workload(batch=1, num_q_heads=2, num_kv_heads=2, head_dim=16, seq_lens=[3], seed=1, q_len=4)
    with pytest.raises(ValueError):
        A.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)


# ------------------------------------------------------------ FP8 KV cache

import oracle.fp8 as F  # noqa: E402


def test_e4m3_codes_match_torch_float8_e4m3fn():
    """Every one of the 256 codes against torch's float8_e4m3fn -> float64
    cast (an independent implementation of the OCP E4M3 format)."""
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([F.e4m3_value(c) for c in range(256)])
    assert np.array_equal(mine, ref, equal_nan=True)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.signbit(mine[fin]), np.signbit(ref[fin]))  # -0 included
    assert np.array_equal(F.decode_e4m3(codes), ref, equal_nan=True)
    assert np.array_equal(A.as_f64(codes.view(torch.float8_e4m3fn)), ref, equal_nan=True)


def test_e4m3_format_closed_forms():
    """Values the format's definition fixes: signed zeros, the smallest and
    largest subnormals (2^-9, 7 * 2^-9), the smallest normal (2^-6), 1, 1.5,
    -2, the largest finite magnitude 448, NaN only at S.1111.111, and the
    positive codes in increasing order."""
    v = F.e4m3_value
    assert v(0x00) == 0.0 and v(0x80) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9 and v(0x08) == 2.0 ** -6
    assert v(0x38) == 1.0 and v(0x3C) == 1.5 and v(0xC0) == -2.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert [c for c in range(256) if math.isnan(v(c))] == [0x7F, 0xFF]
    pos = [v(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))


def _fp8_wl(**kw):
    from workloads import quantize_kv_fp8
    return quantize_kv_fp8(_wl(**kw))


def test_fp8_cache_with_unit_scales_equals_the_same_values_in_fp16():
    """Every E4M3 value is exact in fp16, so an FP8 cache read with scales of
    1 gives the fp16 cache of the same values (torch's cast) bit for bit."""
    wl = _fp8_wl()
    k16, v16 = wl.k.to(torch.float16), wl.v.to(torch.float16)
    a = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    b = A.decode_attention(wl.q, k16, v16, wl.seq_lens, wl.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.isfinite(a[0]).all()


def test_fp8_scales_apply_per_kv_head():
    """A K scale c on KV head g acts as a softmax scale c times larger for
    the query heads of group g only; a V scale c on head g multiplies their
    outputs by c and leaves their lse alone (powers of two: exact)."""
    wl = _fp8_wl()
    G = wl.group_size
    base = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    half = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale * 0.5)
    o, lse = A.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale,
                                k_scale=torch.tensor([1.0, 0.5]), v_scale=torch.tensor([1.0, 4.0]))
    assert np.array_equal(o[:, :G], base[0][:, :G]) and np.array_equal(lse[:, :G], base[1][:, :G])
    assert np.array_equal(o[:, G:], 4.0 * half[0][:, G:]) and np.array_equal(lse[:, G:], half[1][:, G:])
    # the same through the split statistics
    O, m, l = A.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, 8,
                                k_scale=torch.tensor([1.0, 0.5]), v_scale=torch.tensor([1.0, 4.0]))
    for b, L in enumerate(wl.lens):
        S = (L + 7) // 8
        for h in range(wl.num_q_heads):
            ob, lb = A.merge_partials(O[b, h, :S], m[b, h, :S], l[b, h, :S])
            assert np.allclose(ob, o[b, h], rtol=1e-12, atol=1e-13) and abs(lb - lse[b, h]) < 1e-12


# ------------------------------------------------------------------ prefill


def test_prefill_is_torch_causal_sdpa():
    """q_len = L (every token of the sequence is a query): causal self-attention,
    checked against torch's scaled_dot_product_attention(is_causal=True) in
    float64 on the CPU (an independent implementation), GQA heads repeated."""
    wl = make_workload(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=32, seq_lens=[37, 37],
                       dtype=torch.bfloat16, seed=21, q_len=37)
    out, lse = A.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    G = wl.group_size
    for b in range(2):
        q = wl.q[b].double().permute(1, 0, 2)                                   # [Hq, L, d]
        kk = wl.k[37 * b: 37 * b + 37].double().permute(1, 0, 2).repeat_interleave(G, 0)
        vv = wl.v[37 * b: 37 * b + 37].double().permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True, scale=wl.scale)
        assert np.allclose(out[b].transpose(1, 0, 2), ref.numpy(), rtol=1e-12, atol=1e-12)
        s = (q @ kk.transpose(1, 2)) * wl.scale
        s = s.masked_fill(torch.triu(torch.ones(37, 37, dtype=torch.bool), 1), float("-inf"))
        assert np.allclose(lse[b].T, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_sampled_query_rows_match_the_full_computation():
    wl = make_workload(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=16, seq_lens=[9, 30],
                       dtype=torch.float16, seed=22, q_len=5)
    full = A.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    rows = [(0, 4, 1), (1, 0, 3), (1, 2, 0)]
    part = A.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, rows=rows)
    for b, i, h in rows:
        assert np.array_equal(part[0][b, i, h], full[0][b, i, h]) and part[1][b, i, h] == full[1][b, i, h]
    assert np.isnan(part[1]).sum() == part[1].size - len(rows)
