"""The seeded input generator: determinism, layouts and poison placement."""

import math

import numpy as np
import torch

from workloads import make_config, make_workload
from workloads.synth import to_paged


def test_same_seed_same_inputs_and_thread_independence():
    a = make_workload(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, seq_lens=[3000, 70000],
                      dtype=torch.bfloat16, seed=3)
    b = make_workload(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, seq_lens=[3000, 70000],
                      dtype=torch.bfloat16, seed=3)
    assert torch.equal(a.q, b.q)
    assert torch.equal(a.k[:a.total_tokens], b.k[:b.total_tokens])
    assert torch.equal(a.v[:a.total_tokens], b.v[:b.total_tokens])
    c = make_workload(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, seq_lens=[3000, 70000],
                      dtype=torch.bfloat16, seed=4)
    assert not torch.equal(a.q, c.q)


def test_contiguous_layout_and_tail_poison():
    wl = make_workload(batch=3, num_q_heads=6, num_kv_heads=3, head_dim=128, seq_lens=[5, 1, 9],
                       dtype=torch.float16, seed=1, pad_rows=16)
    assert wl.k.shape == (15 + 16, 3, 128) and wl.q.shape == (3, 6, 128)
    assert wl.seq_starts() == [0, 5, 6]
    assert torch.isfinite(wl.k[:15].float()).all() and torch.isnan(wl.k[15:].float()).all()
    assert torch.isnan(wl.v[15:].float()).all()
    assert wl.seq_lens.dtype == torch.int32 and wl.group_size == 2


def test_values_are_standard_normal_rounded_once():
    wl = make_workload(batch=1, num_q_heads=8, num_kv_heads=8, head_dim=128, seq_lens=[4096],
                       dtype=torch.float16, seed=9)
    x = wl.k[:4096].float()
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1) < 0.01
    # already representable: a second rounding changes nothing
    assert torch.equal(wl.k[:4096], x.to(torch.float16))


def test_length_distributions():
    wl = make_workload(batch=200, num_q_heads=2, num_kv_heads=1, head_dim=64,
                       seq_lens=("uniform", 10, 20), seed=2, pad_rows=0)
    assert min(wl.lens) >= 10 and max(wl.lens) <= 20 and len(set(wl.lens)) > 5
    wl = make_workload(batch=300, num_q_heads=2, num_kv_heads=1, head_dim=64,
                       seq_lens=("loguniform", 8, 512), seed=2, pad_rows=0)
    assert min(wl.lens) >= 8 and max(wl.lens) <= 512
    logs = np.log(np.array(wl.lens, dtype=float))
    assert abs(logs.mean() - (math.log(8) + math.log(512)) / 2) < 0.3


def test_spike_rows():
    wl = make_workload(batch=1, num_q_heads=2, num_kv_heads=2, head_dim=64, seq_lens=[1000],
                       dtype=torch.float16, seed=5, spike_fraction=0.01, spike_factor=4.0)
    rows = wl.meta["spike_rows"]
    assert len(rows) == 10 and len(set(rows.tolist())) == 10
    base = make_workload(batch=1, num_q_heads=2, num_kv_heads=2, head_dim=64, seq_lens=[1000],
                         dtype=torch.float16, seed=5)
    assert torch.equal(wl.k[rows], base.k[rows] * 4)
    mask = np.ones(1000, bool); mask[rows] = False
    assert torch.equal(wl.k[:1000][torch.from_numpy(mask)], base.k[:1000][torch.from_numpy(mask)])


def test_paged_layout():
    wl = make_workload(batch=4, num_q_heads=4, num_kv_heads=2, head_dim=64, seq_lens=[1, 16, 17, 40],
                       dtype=torch.bfloat16, seed=8)
    pw = to_paged(wl, 16, spare_pages=2)
    npages = [1, 1, 2, 3]
    assert pw.k.shape == (sum(npages) + 2, 16, 2, 64)
    t = pw.block_table.numpy()
    used = np.concatenate([t[b, :n] for b, n in enumerate(npages)])
    assert len(set(used.tolist())) == len(used)  # each page dealt once
    filler = pw.meta["filler_page"]
    assert filler not in used.tolist()
    assert torch.isnan(pw.k[filler].float()).all()
    for b, n in enumerate(npages):
        assert (t[b, n:] == filler).all()
    # token t of sequence b sits at pool[table[b, t // 16], t % 16]
    starts = wl.seq_starts()
    for b, L in enumerate(wl.lens):
        for tok in range(L):
            assert torch.equal(pw.k[t[b, tok // 16], tok % 16], wl.k[starts[b] + tok])
        rem = L % 16
        if rem:
            assert torch.isnan(pw.v[t[b, L // 16], rem:].float()).all()


def test_config_shapes_small_ones():
    c1 = make_config(1)
    assert (c1.batch, c1.num_q_heads, c1.num_kv_heads, c1.head_dim) == (1, 8, 8, 64)
    assert c1.lens == [1024] and c1.force_num_splits == 4 and c1.dtype == torch.float16
    assert c1.scale == 1 / 8
    c4 = make_config(4)
    assert c4.group_size == 4 and c4.dtype == torch.bfloat16 and c4.batch == 16
    assert all(1024 <= n <= 16384 for n in c4.lens)
