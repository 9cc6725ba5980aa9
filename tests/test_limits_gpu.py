"""GPU parity at the edges of the supported shapes: a million-token context,
thousands of tiny sequences in one batch, many query heads, every split
count, and lengths on both sides of page and chunk boundaries."""

import numpy as np
import pytest
import torch

import oracle
from tests.test_parity_gpu import parity, reference, run
from workloads import make_workload
from workloads.synth import to_paged

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hq,hkv,dt", [(4, 2, torch.float16), (8, 1, torch.bfloat16)])
def test_million_token_context(fd, hq, hkv, dt):
    """2^20 tokens (the split count and the work list at their largest for one
    sequence); every head against the oracle."""
    wl = make_workload(name="ctx1m", batch=1, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                       seq_lens=[1 << 20], dtype=dt, seed=1400 + hq)
    res = run(fd, wl)
    assert res.plan.max_splits > 64
    ref_out, ref_lse = reference(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"1M tokens plan={res.plan.as_dict()}")


def test_thousands_of_tiny_paged_sequences(fd):
    """4096 sequences of 1..40 tokens in a paged cache: more sequences than the
    work list's 64-lane scans cover at once, most sequences a single split."""
    r = np.random.default_rng(7)
    lens = [int(x) for x in r.integers(1, 41, 4096)]
    wl = make_workload(name="tiny4096", batch=4096, num_q_heads=8, num_kv_heads=2, head_dim=128, seq_lens=lens,
                       dtype=torch.bfloat16, seed=1410)
    wl = to_paged(wl, 16, spare_pages=2)
    res = run(fd, wl)
    pairs = [(int(b), int(h)) for b, h in zip(r.integers(0, 4096, 400), r.integers(0, 8, 400))]
    ref_out, ref_lse = oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table, 16,
                                               pairs=pairs)
    parity(res.out, res.lse, ref_out, ref_lse, what="4096 tiny paged sequences (400 sampled pairs)")


@pytest.mark.parametrize("kernel", [0, 1, 4])
def test_many_query_heads(fd, monkeypatch, kernel):
    """128 query heads over 16 KV heads (group 8)."""
    monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    wl = make_workload(name="h128", batch=2, num_q_heads=128, num_kv_heads=16, head_dim=128, seq_lens=[5000, 333],
                       dtype=torch.bfloat16, seed=1420)
    res = run(fd, wl)
    assert res.plan.partial_kernel == kernel
    ref_out, ref_lse = reference(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"128 query heads kernel {kernel}")


@pytest.mark.parametrize("L", [15, 16, 17, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049])
def test_lengths_around_page_and_chunk_edges(fd, L):
    """Lengths one short of, at and one past page (16), minimum-chunk (256)
    and head-rows chunk (1024, 2048) boundaries, contiguous and paged."""
    wl = make_workload(name=f"edge{L}", batch=2, num_q_heads=8, num_kv_heads=8, head_dim=128, seq_lens=[L, L + 1],
                       dtype=torch.float16, seed=1430 + L)
    for w in (wl, to_paged(wl, 16, spare_pages=1)):
        for splits in (0, 2):
            res = run(fd, w, num_splits=splits)
            ref_out, ref_lse = reference(w)
            parity(res.out, res.lse, ref_out, ref_lse, what=f"L={L} paged={w.paged} splits={splits}")


@pytest.mark.parametrize("kernel", [0, 1, 2, 4])
def test_out_of_pool_page_indices_read_page_zero(fd, monkeypatch, kernel):
    """With the pool size known (the binding passes it), a table entry outside
    [0, num_pages) reads page 0 instead of memory outside the pool: the result
    is the oracle's on the table with those entries replaced by 0."""
    monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    wl = to_paged(make_workload(name="badpages", batch=2, num_q_heads=16, num_kv_heads=8, head_dim=128,
                                seq_lens=[3000, 700], dtype=torch.bfloat16, seed=1440), 16, spare_pages=1,
                  permute=False)  # page 0 is then the first (full) page of sequence 0, no NaN poison
    bad = wl.block_table.clone()
    bad[0, 5] = 10 ** 6
    bad[0, 100] = -7
    bad[1, 3] = wl.k.shape[0]          # one past the last page
    fixed = bad.clone()
    fixed[(bad < 0) | (bad >= wl.k.shape[0])] = 0
    dev = torch.device("cuda", 0)
    prob = fd.make_problem(batch=2, num_q_heads=16, num_kv_heads=8, head_dim=128, kv_dtype=torch.bfloat16,
                           scale=wl.scale, page_size=16, max_pages_per_seq=wl.max_pages_per_seq)
    plan = fd.fd_plan_splits(prob, wl.lens, 256)
    assert plan.partial_kernel == kernel
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    out = torch.empty((2, 16, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((2, 16), dtype=torch.float32, device=dev)
    lens = wl.seq_lens.to(dev)
    fd.fd_decode_partial(prob, plan, wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), bad.to(dev), lens, ws)
    fd.fd_combine(prob, plan, lens, ws, out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, fixed, 16)
    parity(out, lse, ref_out, ref_lse, what=f"out-of-pool pages, kernel {kernel}")
