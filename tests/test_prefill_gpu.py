"""GPU parity for prefill attention (fd_prefill_attention, the FA-2 forward
pass): every query row against the oracle's causal multi-query attention, at
sizes the oracle finishes in seconds, and on sampled rows at the full
8192-token workload. Tolerances are the decode path's.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_parity_gpu import announce, parity
from workloads import make_workload
from workloads.synth import to_paged

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, Hq, Hkv, lens, q_len, page)
    (torch.float16, 4, 4, [200], 200, 0),              # one ragged block of rows, MHA
    (torch.bfloat16, 8, 2, [300, 300], 300, 0),        # GQA, two sequences
    (torch.bfloat16, 8, 8, [1000, 700], 257, 0),       # a chunk at the end of longer caches
    (torch.float16, 16, 2, [129, 500], 129, 16),       # paged
    (torch.bfloat16, 4, 1, [1], 1, 0),                 # a single token
    (torch.float16, 2, 2, [3000], 3000, 0),            # many tiles
    (torch.bfloat16, 32, 8, [33, 64, 95], 33, 16),     # short paged sequences, G = 4
]


def _wl(case, seed):
    dt, hq, hkv, lens, ql, page = case
    wl = make_workload(name="prefill", batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                       seq_lens=lens, dtype=dt, seed=seed, q_len=ql)
    wl.q = wl.q.reshape(len(lens), ql, hq, 128)
    if page:
        wl = to_paged(wl, 16, spare_pages=2)
    return wl


def _run(fd, wl, out_dtype=torch.float32):
    dev = torch.device("cuda", 0)
    bt = wl.block_table.to(dev) if wl.paged else None
    announce(f"prefill B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} lens={wl.lens[:4]} "
             f"q_len={wl.q.shape[1]} {wl.dtype} page={wl.page_size} seed={wl.seed}")
    out, lse = fd.prefill_attention(wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), wl.seq_lens, block_table=bt,
                                    page_size=wl.page_size, max_pages_per_seq=wl.max_pages_per_seq,
                                    scale=wl.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_matches_oracle(fd, case):
    wl = _wl(CASES[case], 1100 + case)
    out, lse = _run(fd, wl)
    ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                                     wl.page_size)
    parity(out, lse, ref_out, ref_lse, what=f"prefill case {case}")


def test_prefill_low_precision_output(fd):
    wl = _wl(CASES[1], 1150)
    out, lse = _run(fd, wl, out_dtype=torch.bfloat16)
    ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    # bf16 rounding of O adds up to half an ulp (2^-9 relative) per element
    # on top of the fp32 output's bar (O max-abs 2e-3)
    o = out.double().cpu().numpy()
    assert np.all(np.abs(o - ref_out) <= 2 ** -8 * np.abs(ref_out) + 2e-3)
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) < 1e-4


def test_prefill_full_size_sampled_rows(fd):
    """The 8192-token GQA prefill the benchmark times (B=1, 32 query / 8 KV
    heads, bf16): 256 sampled rows, including the first and last rows and
    both sides of every 128-row block edge near the start and the end."""
    wl = make_workload(name="prefill_full", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
                       seq_lens=[8192], dtype=torch.bfloat16, seed=1200, q_len=8192)
    wl.q = wl.q.reshape(1, 8192, 32, 128)
    out, lse = _run(fd, wl)
    r = np.random.default_rng(5)
    pick = sorted(set([0, 1, 127, 128, 255, 256, 8063, 8064, 8191] + list(r.integers(0, 8192, 200))))
    rows = [(0, int(i), int(r.integers(0, 32))) for i in pick]
    ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, rows=rows)
    parity(out, lse, ref_out, ref_lse, what="prefill 8192 sampled rows")


def test_prefill_bf16_values_beyond_fp16_range(fd):
    """bf16 V tiles holding values past fp16's largest (2^17, 2^20, 2^40) are
    scaled by a power of two before their fp16 products; tiles with tiny
    values (2^-30) too. Checked against the oracle relative to the output's
    magnitude (fp32 accumulation of values near 2^40 has no absolute 2e-3
    bar), LSE (independent of V) at the usual bar."""
    wl = make_workload(name="prefill_big_v", batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128,
                       seq_lens=[400], dtype=torch.bfloat16, seed=1160, q_len=400)
    wl.q = wl.q.reshape(1, 400, 4, 128)
    v = wl.v.float()
    v[64:128] *= 2.0 ** 20          # one whole 64-token tile far past fp16's range
    v[200] *= 2.0 ** 17              # a single row in an otherwise normal tile
    v[300:310] *= 2.0 ** -30         # tiny values: fp16 subnormal range and below
    v[399, 1, :4] = 2.0 ** 40        # the last row, one head
    wl.v = v.to(torch.bfloat16)
    out, lse = _run(fd, wl)
    ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale)
    o = out.double().cpu().numpy()
    assert np.isfinite(o).all()
    mag = np.max(np.abs(ref_out), axis=-1, keepdims=True)  # per row
    assert np.max(np.abs(o - ref_out) / mag) < 2e-3
    assert np.linalg.norm(o - ref_out) / np.linalg.norm(ref_out) < 1e-3
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) < 1e-4
