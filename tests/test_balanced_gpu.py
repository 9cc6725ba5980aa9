"""GPU parity for the balanced split mode (fd_plan.split_mode 1).

The tiles of every sequence form one list that is dealt out in equal work
items across sequence boundaries; a work-group then runs the shares of
several sequences one after the other. The result must match the oracle and
the per-sequence mode on the same inputs, the per-split statistics must be
the oracle's over the ranges the partition rule gives, and a plan made for
upper-bound lengths must serve shorter device lengths (the items then start
at other tiles of each sequence).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.split_cuts import plan_cuts
from tests.test_parity_fp8_gpu import reference_fp8, run_fp8
from tests.test_parity_gpu import O_MAX_ABS, announce, parity, run
from workloads import make_config, make_workload
from workloads.synth import quantize_kv_fp8, to_paged

pytestmark = pytest.mark.gpu


def _tiny_and_long(B, seed):
    """Lengths mixing single tokens, page edges and long sequences, so one
    work item holds shares of many sequences and some sequences span many
    items."""
    rng = np.random.default_rng(seed)
    pool = [1, 2, 15, 16, 17, 31, 33, 257, 600, 5000, 8000]
    return [int(x) for x in rng.choice(pool, size=B)]


CASES = [
    # (name, workload maker, oracle pairs sampled per call or None for all)
    ("GQA varlen: 16 sequences of 1024-16384 tokens, 32/8 heads", lambda: make_config(4), None),
    ("paged GQA: 64 sequences of 512-32768 tokens, 64/8 heads", lambda: make_config(5), 96),
    ("G8 paged, 200 mixed sequences", lambda: to_paged(make_workload(
        name="bal200", batch=200, num_q_heads=64, num_kv_heads=8, head_dim=128, seq_lens=_tiny_and_long(200, 3),
        dtype=torch.bfloat16, seed=1600), 16), 128),
    ("G4 fp16 contiguous, one long among tiny", lambda: make_workload(
        name="bal-long", batch=5, num_q_heads=16, num_kv_heads=4, head_dim=128, seq_lens=[1, 3, 100000, 7, 2],
        dtype=torch.float16, seed=1601), None),
    ("G2 q_len 4 paged", lambda: to_paged(make_workload(
        name="bal-mq", batch=6, num_q_heads=16, num_kv_heads=8, head_dim=128, seq_lens=[4, 900, 31, 5000, 17, 64],
        dtype=torch.bfloat16, seed=1602, q_len=4), 16), None),
    ("G4 q_len 4 contiguous (16 rows)", lambda: make_workload(
        name="bal-mq16", batch=7, num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_lens=[4, 3000, 17, 700, 64, 9000, 5], dtype=torch.bfloat16, seed=1604, q_len=4), None),
    ("G8 q_len 8 paged (64 rows, 4 column tiles)", lambda: to_paged(make_workload(
        name="bal-mq64", batch=5, num_q_heads=64, num_kv_heads=8, head_dim=128, seq_lens=[8, 2500, 33, 700, 4100],
        dtype=torch.bfloat16, seed=1605, q_len=8), 16), None),
    ("G4 q_len 4 fp8 paged", lambda: quantize_kv_fp8(to_paged(make_workload(
        name="bal-mq-fp8", batch=6, num_q_heads=16, num_kv_heads=4, head_dim=128, seq_lens=[4, 1500, 20, 3000, 64, 9],
        dtype=torch.float16, seed=1606, q_len=4), 16)), None),
    ("G8 fp8 paged", lambda: quantize_kv_fp8(to_paged(make_workload(
        name="bal-fp8", batch=40, num_q_heads=64, num_kv_heads=8, head_dim=128, seq_lens=_tiny_and_long(40, 4),
        dtype=torch.bfloat16, seed=1603), 16)), 64),
]


def _pairs(wl, n, seed):
    if n is None:
        return None
    rng = np.random.default_rng(seed)
    bs = rng.integers(0, wl.batch, size=n)
    hs = rng.integers(0, wl.num_q_heads, size=n)
    return sorted({(int(b), int(h)) for b, h in zip(bs, hs)} | {(int(np.argmax(wl.lens)), 0), (0, 0)})


def _run(fd, wl):
    return run_fp8(fd, wl, num_splits=0) if wl.kv_dtype == torch.float8_e4m3fn else run(fd, wl, num_splits=0)


def _reference(wl, pairs):
    if wl.kv_dtype == torch.float8_e4m3fn:
        assert pairs is None or wl.q_len == 1
        if pairs is not None:
            return oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table, wl.page_size,
                                           pairs=pairs, k_scale=wl.k_scale, v_scale=wl.v_scale)
        return reference_fp8(wl)
    if wl.q_len > 1:
        return oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table, wl.page_size)
    return oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table, wl.page_size,
                                   pairs=pairs)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_balanced_matches_oracle_and_per_sequence_mode(fd, monkeypatch, case):
    name, mk, npairs = CASES[case]
    wl = mk()
    monkeypatch.delenv("FD_SPLIT_MODE", raising=False)
    bal = _run(fd, wl)
    assert bal.plan.split_mode == 1, bal.plan.as_dict()
    monkeypatch.setenv("FD_SPLIT_MODE", "0")
    seq = _run(fd, wl)
    assert seq.plan.split_mode == 0
    pairs = _pairs(wl, npairs, 1610 + case)
    ref_out, ref_lse = _reference(wl, pairs)
    tol = O_MAX_ABS
    parity(bal.out, bal.lse, ref_out, ref_lse, o_tol=tol, what=f"balanced {name} plan={bal.plan.as_dict()}")
    parity(seq.out, seq.lse, ref_out, ref_lse, o_tol=tol, what=f"per-sequence {name}")
    # the two modes differ only in where the splits are cut: fp32 rounding apart
    d = (bal.out.double() - seq.out.double()).abs().max().item()
    assert d <= tol, d


def test_balanced_split_statistics_match_oracle(fd):
    """Each (sequence, split) slot of the workspace holds the oracle's
    statistics over the token range the partition rule gives; the work items
    cut sequences at tile offsets that are not chunk multiples."""
    wl = to_paged(make_workload(name="bal-stats", batch=9, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                seq_lens=[1, 17, 700, 16, 4000, 33, 2500, 3, 1200], dtype=torch.bfloat16,
                                seed=1620), 16)
    res = run(fd, wl, num_splits=0)
    plan = res.plan
    assert plan.split_mode == 1
    cuts = plan_cuts(wl.lens, plan)
    assert max(len(c) for c in cuts) <= plan.max_splits
    assert any(len(c) > 1 and c[0][1] % plan.chunk_tokens for c in cuts)  # a cut off the chunk grid
    prob = fd.make_problem(batch=wl.batch, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype=torch.bfloat16,
                           page_size=16, max_pages_per_seq=wl.max_pages_per_seq)
    O_s, m_s, l_s = (x.double().cpu().numpy() for x in fd.workspace_views(prob, plan, res.workspace))
    Oo, mo, lo = oracle.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, None, wl.block_table, 16,
                                        max_splits=plan.max_splits, bounds=cuts)
    for b, c in enumerate(cuts):
        S = len(c)
        assert np.allclose(m_s[b, :, :S], mo[b, :, :S], rtol=0, atol=1e-5)
        assert np.allclose(l_s[b, :, :S], lo[b, :, :S], rtol=1e-5, atol=0)
        scale = np.abs(Oo[b, :, :S]).max()
        assert np.max(np.abs(O_s[b, :, :S] - Oo[b, :, :S])) <= 1e-5 * max(1.0, scale) * 8


@pytest.mark.parametrize("page", [0, 16])
def test_balanced_plan_for_upper_bound_lengths(fd, page):
    """A balanced plan made for upper-bound lengths, run on shorter device
    lengths: the items start at other tiles of each sequence, and every
    sequence's splits still fit the plan's S_max."""
    final = [5000, 17, 3000, 800, 64, 12000, 1]
    wl = make_workload(name="bal-ub", batch=len(final), num_q_heads=32, num_kv_heads=8, head_dim=128,
                       seq_lens=final, dtype=torch.bfloat16, seed=1630)
    if page:
        wl = to_paged(wl, 16, spare_pages=2)
    dev = torch.device("cuda", 0)
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    bt = wl.block_table.to(dev) if page else None
    prob = fd.make_problem(batch=wl.batch, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype=torch.bfloat16,
                           scale=wl.scale, page_size=page, max_pages_per_seq=wl.max_pages_per_seq if page else 0)
    plan = fd.fd_plan_splits(prob, final)
    assert plan.split_mode == 1
    announce(f"balanced upper-bound plan page={page}: {plan.as_dict()}")
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    out = torch.empty((wl.batch, 32, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.batch, 32), dtype=torch.float32, device=dev)
    for lens in ([5000, 17, 3000, 800, 64, 12000, 1], [1, 17, 2999, 800, 1, 11000, 1], [4000, 1, 1, 1, 64, 3, 1]):
        if not page:
            # a packed cache is packed by the device lengths: rebuild it for this step
            sub = make_workload(name="bal-ub-step", batch=wl.batch, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                seq_lens=lens, dtype=torch.bfloat16, seed=1631)
            sub.q = wl.q
            # sized for the plan's lengths (the binding checks that), NaN past this step's rows
            k_use = torch.full((sum(final) + 16, 8, 128), float("nan"), dtype=torch.bfloat16, device=dev)
            v_use = torch.full_like(k_use, float("nan"))
            k_use[: sum(lens)] = sub.k[: sum(lens)].to(dev)
            v_use[: sum(lens)] = sub.v[: sum(lens)].to(dev)
            ref_wl = sub
        else:
            k_use, v_use, ref_wl = k, v, wl
        lens_dev = torch.tensor(lens, dtype=torch.int32, device=dev)
        fd.fd_decode_partial(prob, plan, q, k_use, v_use, bt, lens_dev, ws)
        fd.fd_combine(prob, plan, lens_dev, ws, out, lse)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle.decode_attention(ref_wl.q, ref_wl.k, ref_wl.v, lens, wl.scale,
                                                   ref_wl.block_table if page else None, page)
        parity(out, lse, ref_out, ref_lse, what=f"upper-bound plan, lengths {lens}")


def _random_case(seed):
    """A seeded ragged batch: group size, query tokens, cache type and layout,
    and a length mix of single tokens, page edges and long sequences."""
    r = np.random.default_rng(seed)
    G = int(r.choice([4, 8]))
    hkv = int(r.choice([1, 2, 4, 8]))
    ql = int(r.choice([1, 1, 2, 4, 8]))
    if ql * G > 64:
        ql = 64 // G
    B = int(r.integers(2, 160))
    pool = [1, 2, 15, 16, 17, 33, 100, 257, 1000, 3000, 9000]
    lens = [max(ql, int(x)) for x in r.choice(pool, size=B)]
    if len(set(lens)) == 1:  # equal lengths keep per-sequence chunks
        lens[-1] += 1
    dt = torch.float16 if r.random() < 0.5 else torch.bfloat16
    wl = make_workload(name=f"bal-rand{seed}", batch=B, num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=128,
                       seq_lens=lens, dtype=dt, seed=seed, q_len=ql)
    if r.random() < 0.5:
        wl = to_paged(wl, 16, spare_pages=2)
    if ql == 1 and r.random() < 0.3:
        wl = quantize_kv_fp8(wl)
    return wl


@pytest.mark.parametrize("seed", range(1650, 1662))
def test_balanced_random_ragged_batches(fd, monkeypatch, seed):
    """Seeded random ragged batches on the balanced list against the oracle,
    every query row of a sampled set of (sequence, head) pairs. Odd seeds
    force the matrix-core kernel with one work-group per column tile (kernel
    1); even seeds take the planner's choice."""
    if seed % 2:
        monkeypatch.setenv("FD_PARTIAL_KERNEL", "1")
    wl = _random_case(seed)
    res = _run(fd, wl)
    assert res.plan.split_mode == 1, res.plan.as_dict()
    r = np.random.default_rng(seed + 1)
    bs = sorted({int(x) for x in r.integers(0, wl.batch, size=24)} | {0, wl.batch - 1, int(np.argmax(wl.lens))})
    tol = O_MAX_ABS
    if wl.q_len > 1:
        rows = [(b, i, h) for b in bs for i in range(wl.q_len) for h in range(wl.num_q_heads)]
        ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                                         wl.page_size, rows=rows)
    else:
        pairs = [(b, h) for b in bs for h in range(wl.num_q_heads)]
        ref_out, ref_lse = _reference(wl, pairs)
    parity(res.out, res.lse, ref_out, ref_lse, o_tol=tol,
           what=f"random ragged seed={seed} B={wl.batch} G={wl.num_q_heads // wl.num_kv_heads} "
                f"q_len={wl.q_len} {wl.kv_dtype} page={wl.page_size} plan={res.plan.as_dict()}")


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
def test_balanced_low_precision_outputs_and_fused(fd, out_dtype):
    """16-bit outputs on the balanced list, through the combine and through the
    fused merge (three calls in a row on one workspace), against the oracle
    with the output's own rounding added to the bar."""
    wl = to_paged(make_workload(name="bal-out", batch=12, num_q_heads=32, num_kv_heads=4, head_dim=128,
                                seq_lens=[1, 700, 33, 5000, 16, 2600, 3, 129, 9000, 64, 1500, 17],
                                dtype=torch.bfloat16, seed=1670), 16)
    res = run(fd, wl, num_splits=0, out_dtype=out_dtype)
    assert res.plan.split_mode == 1
    ref_out, ref_lse = oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table, 16)
    rnd = 2.0 ** -11 if out_dtype == torch.float16 else 2.0 ** -8
    bar = O_MAX_ABS + rnd * float(np.abs(ref_out).max())
    o = res.out.double().cpu().numpy()
    assert np.max(np.abs(o - ref_out)) <= bar
    assert np.max(np.abs(res.lse.double().cpu().numpy() - ref_lse)) <= 1e-4
    dev = torch.device("cuda", 0)
    q, k, v, bt = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), wl.block_table.to(dev)
    lens = wl.seq_lens.to(dev)
    prob = fd.make_problem(batch=wl.batch, num_q_heads=32, num_kv_heads=4, head_dim=128, kv_dtype=torch.bfloat16,
                           out_dtype=out_dtype, scale=wl.scale, page_size=16, max_pages_per_seq=wl.max_pages_per_seq)
    plan = fd.fd_plan_splits(prob, wl.lens)
    assert plan.split_mode == 1
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    fd.fd_workspace_init(prob, plan, ws)
    for _ in range(3):
        out = torch.full(tuple(wl.q.shape), float("nan"), dtype=out_dtype, device=dev)
        lse = torch.full(tuple(wl.q.shape[:-1]), float("nan"), dtype=torch.float32, device=dev)
        fd.fd_decode_fused(prob, plan, q, k, v, bt, lens, ws, out, lse)
        torch.cuda.synchronize()
        of = out.double().cpu().numpy()
        assert np.isfinite(of).all()
        assert np.max(np.abs(of - ref_out)) <= bar
        assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) <= 1e-4


def test_balanced_upper_bound_plan_multi_query(fd):
    """Four query tokens per sequence on a balanced plan made for longer
    lengths: each step's shorter device lengths move the cuts and every
    query's causal limit with them."""
    final = [900, 40, 3000, 17, 5000, 260]
    wl = to_paged(make_workload(name="bal-ub-mq", batch=len(final), num_q_heads=32, num_kv_heads=8, head_dim=128,
                                seq_lens=final, dtype=torch.bfloat16, seed=1680, q_len=4), 16, spare_pages=2)
    dev = torch.device("cuda", 0)
    q, k, v, bt = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), wl.block_table.to(dev)
    prob = fd.make_problem(batch=wl.batch, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype=torch.bfloat16,
                           scale=wl.scale, page_size=16, max_pages_per_seq=wl.max_pages_per_seq, q_len=4)
    plan = fd.fd_plan_splits(prob, final)
    assert plan.split_mode == 1 and plan.partial_kernel in (1, 4)
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    out = torch.empty(tuple(wl.q.shape), dtype=torch.float32, device=dev)
    lse = torch.empty(tuple(wl.q.shape[:-1]), dtype=torch.float32, device=dev)
    for lens in (final, [4, 40, 2999, 5, 4000, 260], [900, 4, 7, 17, 33, 100]):
        lens_dev = torch.tensor(lens, dtype=torch.int32, device=dev)
        fd.fd_decode_partial(prob, plan, q, k, v, bt, lens_dev, ws)
        fd.fd_combine(prob, plan, lens_dev, ws, out, lse)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, lens, wl.scale, wl.block_table, 16)
        parity(out, lse, ref_out, ref_lse, what=f"multi-query upper-bound plan, lengths {lens}")
