"""GPU parity for fd_append_kv: the paged cache and the rotated queries after
an append, against the oracle's append on the same inputs.

Both sides compute the rotation in fp64 and round once to the storage format
(ties to even), so the stored bits agree except where the two sides' fp64
pow/sin/cos differ by an ulp and a result sits on a rounding boundary: such
elements may differ by one unit in the last place, and only in at most
1e-4 of the new elements. Slots the append does not own must keep their
bytes exactly (their NaN poison included).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.append import append_kv
from tests.test_parity_gpu import announce, parity
from workloads import make_workload
from workloads.synth import quantize_kv_fp8, to_paged

pytestmark = pytest.mark.gpu

CASES = [
    # (cache dtype, q dtype, rope style, d, Hq, Hkv, lens after the append, new tokens)
    (torch.float16, torch.float16, "interleaved", 128, 8, 2, [17, 32, 5, 1000], 1),
    (torch.bfloat16, torch.bfloat16, "half", 64, 4, 4, [3, 16, 300], 3),
    (torch.float8_e4m3fn, torch.float16, "half", 128, 32, 8, [100, 4000], 2),
    (torch.float8_e4m3fn, torch.bfloat16, "interleaved", 64, 8, 8, [1, 64, 65], 1),
    (torch.float16, torch.float16, None, 128, 4, 4, [15, 16, 17], 2),
    (torch.bfloat16, torch.bfloat16, "half", 128, 2, 1, [100000], 4),   # positions near 1e5
]


def _bits(t):
    t = t.contiguous()
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16)


def assert_same_storage(got, ref, what, changed_mask=None):
    """Bitwise equality, except one-ulp steps in at most 1e-4 of the elements
    under ``changed_mask`` (the slots the append wrote)."""
    gb, rb = _bits(got.cpu()).numpy().astype(np.int32), _bits(ref.cpu()).numpy().astype(np.int32)
    diff = gb != rb
    if changed_mask is not None:
        assert not diff[~changed_mask].any(), f"{what}: bytes outside the new tokens changed"
        n_new = int(changed_mask.sum())
    else:
        n_new = diff.size
    bad = np.argwhere(diff)
    announce(f"  {what}: {len(bad)} of {n_new} new elements differ")
    assert len(bad) <= max(1, int(1e-4 * n_new)), f"{what}: {len(bad)} elements differ"
    if len(bad):
        assert np.all(np.abs(gb[diff] - rb[diff]) == 1), f"{what}: a difference beyond one ulp"


def setup(case, seed):
    kvdt, qdt, style, d, hq, hkv, lens, n = case
    wl = make_workload(name="append", batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                       seq_lens=lens, dtype=qdt, seed=seed, q_len=n)
    wl = to_paged(wl, 16, spare_pages=4)
    wl.q = wl.q.reshape(len(lens), n, hq, d)
    if kvdt == torch.float8_e4m3fn:
        wl = quantize_kv_fp8(wl)
    g = torch.Generator().manual_seed(seed)
    k_new = (torch.randn(len(lens), n, hkv, d, generator=g) * 2).to(qdt)
    v_new = (torch.randn(len(lens), n, hkv, d, generator=g) * 2).to(qdt)
    return wl, k_new, v_new


@pytest.mark.parametrize("case", range(len(CASES)))
def test_append_matches_oracle(fd, case):
    kvdt, qdt, style, d, hq, hkv, lens, n = CASES[case]
    wl, k_new, v_new = setup(CASES[case], 900 + case)
    announce(f"append case {case}: cache {kvdt} q {qdt} rope {style} d={d} Hq={hq} Hkv={hkv} lens={lens} n={n}")
    dev = torch.device("cuda", 0)
    kc, vc, q = wl.k.to(dev), wl.v.to(dev), wl.q.to(dev).contiguous()
    ks = wl.k_scale.to(dev) if wl.k_scale is not None else None
    vs = wl.v_scale.to(dev) if wl.v_scale is not None else None
    prob = fd.make_problem(batch=wl.batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, kv_dtype=kvdt,
                           q_dtype=qdt, page_size=16, max_pages_per_seq=wl.max_pages_per_seq, q_len=n)
    fd.fd_append_kv(prob, k_new.to(dev), v_new.to(dev), q, kc, vc, wl.block_table.to(dev), wl.seq_lens.to(dev),
                    rope_style=style, rope_base=10000.0, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    rk, rv, rq = append_kv(wl.k, wl.v, wl.block_table, wl.seq_lens, k_new, v_new, wl.q, rope_style=style,
                           rope_base=10000.0, k_scale=wl.k_scale, v_scale=wl.v_scale)
    mask = np.zeros(tuple(wl.k.shape), dtype=bool)
    for b, L in enumerate(wl.lens):
        for j in range(n):
            pos = L - n + j
            mask[int(wl.block_table[b, pos // 16]), pos % 16] = True
    assert_same_storage(kc, rk, "K cache", mask)
    assert_same_storage(vc, rv, "V cache", mask)
    if style is None:
        assert torch.equal(q.cpu(), wl.q)
    else:
        assert_same_storage(q, rq, "q")


LOOP_CASES = [
    # a few hundred new tokens per sequence (chunks of a prompt), every token checked
    (torch.bfloat16, torch.bfloat16, "half", 128, 8, 2, [300, 500, 177], 150),
    (torch.float8_e4m3fn, torch.float16, "interleaved", 64, 4, 4, [700], 600),
    (torch.float16, torch.float16, None, 128, 4, 2, [400, 301], 300),
]


@pytest.mark.parametrize("case", range(len(LOOP_CASES)))
def test_append_many_new_tokens(fd, case):
    """Hundreds of new tokens per sequence (a prompt chunk) against the
    oracle: every token, rotated queries included."""
    kvdt, qdt, style, d, hq, hkv, lens, n = LOOP_CASES[case]
    wl, k_new, v_new = setup(LOOP_CASES[case], 990 + case)
    announce(f"append chunk case {case}: cache {kvdt} rope {style} d={d} Hq={hq} Hkv={hkv} lens={lens} n={n}")
    dev = torch.device("cuda", 0)
    kc, vc, q = wl.k.to(dev), wl.v.to(dev), wl.q.to(dev).contiguous()
    ks = wl.k_scale.to(dev) if wl.k_scale is not None else None
    vs = wl.v_scale.to(dev) if wl.v_scale is not None else None
    prob = fd.make_problem(batch=wl.batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, kv_dtype=kvdt,
                           q_dtype=qdt, page_size=16, max_pages_per_seq=wl.max_pages_per_seq, q_len=n)
    fd.fd_append_kv(prob, k_new.to(dev), v_new.to(dev), q, kc, vc, wl.block_table.to(dev), wl.seq_lens.to(dev),
                    rope_style=style, rope_base=10000.0, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    rk, rv, rq = append_kv(wl.k, wl.v, wl.block_table, wl.seq_lens, k_new, v_new, wl.q, rope_style=style,
                           rope_base=10000.0, k_scale=wl.k_scale, v_scale=wl.v_scale)
    mask = np.zeros(tuple(wl.k.shape), dtype=bool)
    for b, L in enumerate(wl.lens):
        for j in range(n):
            pos = L - n + j
            mask[int(wl.block_table[b, pos // 16]), pos % 16] = True
    assert_same_storage(kc, rk, "K cache", mask)
    assert_same_storage(vc, rv, "V cache", mask)
    if style is None:
        assert torch.equal(q.cpu(), wl.q)
    else:
        assert_same_storage(q, rq, "q")


def test_append_then_decode(fd):
    """The step a decoder runs: append with RoPE, then split-KV decode with the
    rotated queries, against the oracle doing the same two steps."""
    case = (torch.bfloat16, torch.bfloat16, "half", 128, 32, 8, [700, 5000, 33], 2)
    kvdt, qdt, style, d, hq, hkv, lens, n = case
    wl, k_new, v_new = setup(case, 950)
    dev = torch.device("cuda", 0)
    kc, vc, q = wl.k.to(dev), wl.v.to(dev), wl.q.to(dev).contiguous()
    bt, lens_dev = wl.block_table.to(dev), wl.seq_lens.to(dev)
    prob = fd.make_problem(batch=wl.batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, kv_dtype=kvdt,
                           page_size=16, max_pages_per_seq=wl.max_pages_per_seq, q_len=n)
    fd.fd_append_kv(prob, k_new.to(dev), v_new.to(dev), q, kc, vc, bt, lens_dev, rope_style=style)
    res = fd.decode_attention(q, kc, vc, wl.seq_lens, block_table=bt, page_size=16,
                              max_pages_per_seq=wl.max_pages_per_seq, scale=wl.scale)
    torch.cuda.synchronize()
    rk, rv, rq = append_kv(wl.k, wl.v, wl.block_table, wl.seq_lens, k_new, v_new, wl.q, rope_style=style)
    ref_out, ref_lse = oracle.decode_attention_multi(rq, rk, rv, wl.seq_lens, wl.scale, wl.block_table, 16)
    parity(res.out, res.lse, ref_out, ref_lse, what="append + decode")


def test_append_skips_positions_outside_the_table(fd):
    """A sequence shorter than its new tokens, or a page index outside the
    pool, writes nothing (checked on the device, nothing is trusted)."""
    wl, k_new, v_new = setup((torch.float16, torch.float16, "half", 64, 2, 2, [1, 40], 2), 960)
    dev = torch.device("cuda", 0)
    bt = wl.block_table.clone()
    bt[1, 2] = 10 ** 6          # position 38 and 39 of sequence 1 point outside the pool
    kc, vc = wl.k.to(dev), wl.v.to(dev)
    prob = fd.make_problem(batch=2, num_q_heads=2, num_kv_heads=2, head_dim=64, kv_dtype=torch.float16,
                           page_size=16, max_pages_per_seq=wl.max_pages_per_seq, q_len=2)
    fd.fd_append_kv(prob, k_new.to(dev), v_new.to(dev), None, kc, vc, bt.to(dev), wl.seq_lens.to(dev),
                    rope_style="half")
    torch.cuda.synchronize()
    # sequence 0: position -1 skipped, position 0 written; sequence 1: nothing written
    changed = (_bits(kc.cpu()) != _bits(wl.k)).reshape(wl.k.shape[0], 16, -1).any(-1)
    pages = torch.nonzero(changed).tolist()
    assert pages == [[int(wl.block_table[0, 0]), 0]]


def test_append_scaled_16bit_cache(fd):
    """A 16-bit cache with per-head scales stores value / scale (rounded once)."""
    case = (torch.bfloat16, torch.bfloat16, "interleaved", 128, 16, 4, [31, 32, 400], 3)
    kvdt, qdt, style, d, hq, hkv, lens, n = case
    wl, k_new, v_new = setup(case, 970)
    ks = torch.tensor([0.5, 3.0, 0.1, 1.0], dtype=torch.float32)
    vs = torch.tensor([2.0, 0.3, 1.0, 7.0], dtype=torch.float32)
    dev = torch.device("cuda", 0)
    kc, vc, q = wl.k.to(dev), wl.v.to(dev), wl.q.to(dev).contiguous()
    prob = fd.make_problem(batch=wl.batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, kv_dtype=kvdt,
                           page_size=16, max_pages_per_seq=wl.max_pages_per_seq, q_len=n)
    fd.fd_append_kv(prob, k_new.to(dev), v_new.to(dev), q, kc, vc, wl.block_table.to(dev), wl.seq_lens.to(dev),
                    rope_style=style, k_scale=ks.to(dev), v_scale=vs.to(dev))
    torch.cuda.synchronize()
    rk, rv, rq = append_kv(wl.k, wl.v, wl.block_table, wl.seq_lens, k_new, v_new, wl.q, rope_style=style,
                           k_scale=ks, v_scale=vs)
    mask = np.zeros(tuple(wl.k.shape), dtype=bool)
    for b, L in enumerate(wl.lens):
        for j in range(n):
            pos = L - n + j
            mask[int(wl.block_table[b, pos // 16]), pos % 16] = True
    assert_same_storage(kc, rk, "K cache (scaled)", mask)
    assert_same_storage(vc, rv, "V cache (scaled)", mask)
    assert_same_storage(q, rq, "q")


def test_append_full_size_sampled_tokens(fd):
    """The 8192-token prompt append the benchmark times (one call, 32 query /
    8 KV heads, bf16, half pairing, permuted pages): 64 sampled tokens,
    including the first and last and both sides of page edges, each checked
    against the oracle appending that token alone at its position; slots the
    append does not own keep their bytes."""
    from workloads import make_append
    wl, k_new, v_new = make_append()
    n = wl.q.shape[1]
    dev = torch.device("cuda", 0)
    kc, vc, q = wl.k.to(dev), wl.v.to(dev), wl.q.to(dev).contiguous()
    prob = fd.make_problem(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype=torch.bfloat16,
                           page_size=16, max_pages_per_seq=wl.max_pages_per_seq, q_len=n)
    announce(f"append full size: {wl.name}")
    fd.fd_append_kv(prob, k_new.to(dev), v_new.to(dev), q, kc, vc, wl.block_table.to(dev), wl.seq_lens.to(dev),
                    rope_style="half")
    torch.cuda.synchronize()
    got_k, got_v, got_q = kc.cpu(), vc.cpu(), q.cpu()
    r = np.random.default_rng(11)
    js = sorted(set([0, 1, 15, 16, 17, 4095, 4096, n - 17, n - 16, n - 1] + [int(x) for x in r.integers(0, n, 54)]))
    table = wl.block_table[0:1].repeat(len(js), 1)
    rk, rv, rq = append_kv(wl.k, wl.v, table, [j + 1 for j in js], k_new[0, js][:, None], v_new[0, js][:, None],
                           wl.q[0, js][:, None], rope_style="half")
    for i, j in enumerate(js):
        pg, sl = int(wl.block_table[0, j // 16]), j % 16
        assert_same_storage(got_k[pg, sl], rk[pg, sl], f"K token {j}")
        assert_same_storage(got_v[pg, sl], rv[pg, sl], f"V token {j}")
        assert_same_storage(got_q[0, j], rq[i, 0], f"q token {j}")
    # the spare pages (NaN) keep their bytes
    used = set(int(p) for p in wl.block_table[0, : n // 16])
    spare = [p for p in range(wl.k.shape[0]) if p not in used]
    assert spare and all(torch.equal(_bits(got_k[p]), _bits(wl.k[p])) for p in spare)
