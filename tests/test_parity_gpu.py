"""GPU parity: the HIP path against the fp64 CPU oracle on identical seeded inputs.

Tolerances (fp32 accumulation over fp16/bf16 K/V, fp32 output): on O, max-abs
<= 2e-3 and relative RMS (||dO||_2 / ||O_ref||_2) <= 1e-3 over the whole
tensor; on LSE, abs <= 1e-4. Every call goes through the C ABI.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_config, make_workload
from workloads.synth import to_paged

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-3
O_REL_RMS = 1e-3
LSE_ABS = 1e-4


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu case] {msg}\n")
    sys.__stderr__.flush()


def to_dev(wl):
    dev = torch.device("cuda", 0)
    bt = wl.block_table.to(dev) if wl.paged else None
    return wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), bt


def run(fd, wl, num_splits=None, out_dtype=torch.float32, dev_tensors=None):
    q, k, v, bt = dev_tensors or to_dev(wl)
    ns = wl.force_num_splits if num_splits is None else num_splits
    announce(f"{wl.name} B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} d={wl.head_dim} "
             f"{wl.dtype} page={wl.page_size} splits={ns or 'auto'} seed={wl.seed}")
    res = fd.decode_attention(q, k, v, wl.seq_lens, block_table=bt, page_size=wl.page_size,
                              max_pages_per_seq=wl.max_pages_per_seq, scale=wl.scale,
                              out_dtype=out_dtype, num_splits=ns)
    torch.cuda.synchronize()
    return res


def reference(wl, pairs=None):
    return oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                   wl.page_size, pairs=pairs)


def parity(out, lse, ref_out, ref_lse, o_tol=O_MAX_ABS, what=""):
    o = out.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    mask = ~np.isnan(ref_lse)
    d_o = o[mask] - ref_out[mask]
    max_abs = float(np.max(np.abs(d_o)))
    rel_rms = float(np.linalg.norm(d_o) / np.linalg.norm(ref_out[mask]))
    lse_err = float(np.max(np.abs(ls[mask] - ref_lse[mask])))
    announce(f"  parity {what}: O max-abs {max_abs:.3e} rel-rms {rel_rms:.3e} LSE abs {lse_err:.3e}")
    assert np.isfinite(o[mask]).all() and np.isfinite(ls[mask]).all()
    assert max_abs <= o_tol, f"O max-abs {max_abs}"
    assert rel_rms <= O_REL_RMS, f"O rel-rms {rel_rms}"
    assert lse_err <= LSE_ABS, f"LSE abs {lse_err}"
    return max_abs, rel_rms, lse_err


# ------------------------------------------------------- the worked example


def test_worked_example_on_gpu(fd):
    """Capstone §1.2 tiny calculator embedded exactly in fp16 at d = 64:
    q = 8 e0, scale 1/8, K[:, 0] = [2, 4, 3, 5], two splits of two tokens.
    The split statistics must be the page's (m_A, l_A) = (4, 1.1353...) and
    (m_B, l_B) = (5, 1.1353...), and LSE = 5 + ln(1.5530...)."""
    d = 64
    q = torch.zeros(1, 1, d, dtype=torch.float16)
    q[0, 0, 0] = 8.0
    k = torch.zeros(4, 1, d, dtype=torch.float16)
    k[:, 0, 0] = torch.tensor([2.0, 4.0, 3.0, 5.0])
    g = torch.Generator().manual_seed(0)
    v = torch.randn(4, 1, d, generator=g).to(torch.float16)
    wl = make_workload(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=d, seq_lens=[4], pad_rows=0, seed=0)
    wl.q, wl.k, wl.v, wl.scale, wl.name = q, k, v, 1 / 8, "worked_example"
    res = run(fd, wl, num_splits=2)
    assert (res.plan.chunk_tokens, res.plan.max_splits) == (2, 2)
    O_s, m_s, l_s = fd.workspace_views(fd.make_problem(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=d,
                                                       kv_dtype=torch.float16), res.plan, res.workspace)
    m_s = m_s.double().cpu().numpy()[0, 0]
    l_s = l_s.double().cpu().numpy()[0, 0]
    lA = math.exp(-2) + 1.0
    assert np.allclose(m_s, [4.0, 5.0], rtol=0, atol=2e-6)
    assert np.allclose(l_s, [lA, lA], rtol=2e-6, atol=0)
    lse = float(res.lse.cpu()[0, 0])
    assert abs(lse - (5.0 + math.log(math.exp(-3) + math.exp(-1) + math.exp(-2) + 1.0))) < 2e-6
    ref_out, ref_lse = reference(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what="worked example")
    # the unnormalised split outputs against the oracle's split statistics
    Oo, mo, lo = oracle.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, 2)
    assert np.allclose(O_s.double().cpu().numpy()[0, 0], Oo[0, 0], rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------ the five configs


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity(fd, cfg):
    wl = make_config(cfg)
    res = run(fd, wl)
    ref_out, ref_lse = reference(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"config {cfg} plan={res.plan.as_dict()}")


# ------------------------------------------------------- shapes and splits


SHAPES = [
    # (d, dtype, Hq, Hkv, lens, page)
    (64, torch.float16, 8, 8, [1024], 0),
    (64, torch.bfloat16, 8, 2, [1, 17, 300, 2049], 0),
    (128, torch.float16, 4, 4, [1, 15, 16, 17, 63, 64, 65, 255], 0),
    (128, torch.bfloat16, 16, 2, [1000, 3001, 77], 0),
    (128, torch.float16, 8, 1, [4097, 5], 0),
    (128, torch.bfloat16, 32, 8, [513, 1, 2500], 16),
    (64, torch.float16, 4, 2, [16, 33, 700], 16),
    (128, torch.float16, 16, 16, [70000], 0),
]


@pytest.mark.parametrize("shape", range(len(SHAPES)))
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7, 64])
def test_shapes_and_forced_splits(fd, shape, splits):
    d, dt, hq, hkv, lens, page = SHAPES[shape]
    wl = make_workload(name=f"shape{shape}", batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                       seq_lens=lens, dtype=dt, seed=100 + shape, page_size=page)
    res = run(fd, wl, num_splits=splits)
    ref_out, ref_lse = reference(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"shape {shape} splits {splits}")


def test_split_count_invariance(fd):
    wl = make_workload(name="invariance", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[3000, 1111], dtype=torch.bfloat16, seed=21)
    ref_out, ref_lse = reference(wl)
    dev = to_dev(wl)
    outs = []
    for S in (1, 2, 3, 4, 7, 16, 64, 0):
        res = run(fd, wl, num_splits=S, dev_tensors=dev)
        parity(res.out, res.lse, ref_out, ref_lse, what=f"S={S}")
        outs.append(res.out.double().cpu().numpy())
    spread = max(float(np.max(np.abs(a - outs[0]))) for a in outs)
    assert spread <= O_MAX_ABS


@pytest.mark.parametrize("lens,kernel", [([1000, 257], None), ([4096, 1000], 2)])
def test_split_statistics_match_oracle(fd, monkeypatch, lens, kernel):
    """Each split's (O, m, l) against the oracle's statistics of the same token
    range. On the head-rows kernel with [4096, 1000] the 1024-token splits of
    the first sequence are whole multiples of the kernel's wave stages, so
    splits 1-3 walk their tokens from a rotated start: each must still cover
    exactly its own range."""
    if kernel is not None:
        monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    wl = make_workload(name="stats", batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128,
                       seq_lens=lens, dtype=torch.float16, seed=5)
    res = run(fd, wl, num_splits=4)
    if kernel is not None:
        assert res.plan.partial_kernel == kernel
    C = res.plan.chunk_tokens
    prob = fd.make_problem(batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128, kv_dtype=torch.float16)
    O_s, m_s, l_s = (x.double().cpu().numpy() for x in fd.workspace_views(prob, res.plan, res.workspace))
    Oo, mo, lo = oracle.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, C)
    for b, L in enumerate(wl.lens):
        S = -(-L // C)
        assert np.allclose(m_s[b, :, :S], mo[b, :, :S], rtol=0, atol=1e-5)
        assert np.allclose(l_s[b, :, :S], lo[b, :, :S], rtol=1e-5, atol=0)
        scale = np.abs(Oo[b, :, :S]).max()
        assert np.max(np.abs(O_s[b, :, :S] - Oo[b, :, :S])) <= 1e-5 * max(1.0, scale) * 8


# ------------------------------------------------------- paged and invariants


def test_paged_identity_permuted_and_contiguous_agree_bitwise(fd):
    base = make_workload(name="paged-eq", batch=5, num_q_heads=16, num_kv_heads=2, head_dim=128,
                         seq_lens=[1, 16, 17, 1500, 4096], dtype=torch.bfloat16, seed=31)
    res_c = run(fd, base, num_splits=3)
    outs = []
    for permute in (False, True):
        pw = to_paged(base, 16, permute=permute, spare_pages=4)
        pw.name = f"paged permute={permute}"
        res = run(fd, pw, num_splits=3)
        outs.append((res.out.cpu(), res.lse.cpu()))
    assert res.plan.chunk_tokens == res_c.plan.chunk_tokens
    for o, l in outs:
        assert torch.equal(o, res_c.out.cpu()) and torch.equal(l, res_c.lse.cpu())


def test_deterministic_across_runs(fd):
    wl = make_config(4)
    dev = to_dev(wl)
    a = run(fd, wl, dev_tensors=dev)
    b = run(fd, wl, dev_tensors=dev)
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
def test_low_precision_outputs(fd, out_dtype):
    wl = make_workload(name="outdtype", batch=2, num_q_heads=8, num_kv_heads=8, head_dim=128,
                       seq_lens=[5000, 64], dtype=torch.float16, seed=8)
    res = run(fd, wl, out_dtype=out_dtype)
    ref_out, ref_lse = reference(wl)
    o = res.out.double().cpu().numpy()
    ulp = 2.0 ** -11 if out_dtype == torch.float16 else 2.0 ** -8
    assert np.all(np.abs(o - ref_out) <= O_MAX_ABS + ulp * np.abs(ref_out))
    assert np.max(np.abs(res.lse.double().cpu().numpy() - ref_lse)) <= LSE_ABS


def test_one_shot_matches_split_api_and_checks_workspace(fd):
    wl = make_config(2)
    q, k, v, _ = to_dev(wl)
    res = run(fd, wl, num_splits=0, dev_tensors=(q, k, v, None))
    prob = fd.make_problem(batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128, kv_dtype=torch.float16,
                           scale=wl.scale)
    out = torch.empty_like(res.out)
    lse = torch.empty_like(res.lse)
    lens_dev = wl.seq_lens.cuda()
    announce("fd_decode_attention one-shot, config 2")
    fd.fd_decode_attention(prob, q, k, v, None, wl.lens, lens_dev, out, lse, res.workspace)
    torch.cuda.synchronize()
    assert torch.equal(out, res.out) and torch.equal(lse, res.lse)
    small = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(fd.FdError) as ei:
        fd.fd_decode_attention(prob, q, k, v, None, wl.lens, lens_dev, out, lse, small)
    assert ei.value.status == fd.FD_ERR_WORKSPACE_TOO_SMALL


def test_runs_on_a_side_stream(fd):
    wl = make_workload(name="stream", batch=3, num_q_heads=8, num_kv_heads=4, head_dim=64,
                       seq_lens=[100, 2000, 31], dtype=torch.float16, seed=44)
    q, k, v, _ = to_dev(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        res = fd.decode_attention(q, k, v, wl.seq_lens, scale=wl.scale)
    s.synchronize()
    ref_out, ref_lse = reference(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what="side stream")


GQA_CASES = [
    # (dtype, Hq, Hkv, lens, page)
    (torch.bfloat16, 32, 8, [1, 15, 16, 17, 100, 3000], 0),  # G = 4, ragged tails
    (torch.float16, 16, 2, [777, 4096], 0),                 # G = 8
    (torch.bfloat16, 4, 2, [33, 1024], 16),                 # G = 2, paged
    (torch.bfloat16, 64, 8, [5000, 31, 700], 16),           # G = 8, paged
    (torch.float16, 8, 2, [1, 2, 3, 64, 65], 16),           # G = 4, paged, tiny
]


# Kernel 4 needs a multiple of four KV heads (one per wave): its cases with
# two KV heads are not generated.
GQA_KERNEL_CASES = [(k, c) for c in range(len(GQA_CASES)) for k in (0, 1, 4) if k != 4 or GQA_CASES[c][2] % 4 == 0]


@pytest.mark.parametrize("kernel,case", GQA_KERNEL_CASES)
@pytest.mark.parametrize("splits", [0, 3])
def test_gqa_partial_kernels_agree_with_oracle(fd, monkeypatch, kernel, case, splits):
    """The vector-ALU (0) and both matrix-core (1: four waves share a head;
    4: each wave owns a head) partial kernels on the same GQA inputs."""
    dt, hq, hkv, lens, page = GQA_CASES[case]
    monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    wl = make_workload(name=f"gqa{case}-k{kernel}", batch=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                       head_dim=128, seq_lens=lens, dtype=dt, seed=300 + case, page_size=page)
    res = run(fd, wl, num_splits=splits)
    assert res.plan.partial_kernel == kernel
    ref_out, ref_lse = reference(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"gqa case {case} kernel {kernel} splits {splits}")


@pytest.mark.parametrize("kernel", [1, 4])
def test_mfma_split_statistics_match_oracle(fd, monkeypatch, kernel):
    monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    wl = make_workload(name="stats-mfma", batch=2, num_q_heads=32, num_kv_heads=4, head_dim=128,
                       seq_lens=[1000, 257], dtype=torch.bfloat16, seed=6)
    res = run(fd, wl, num_splits=4)
    assert res.plan.partial_kernel == kernel
    C = res.plan.chunk_tokens
    prob = fd.make_problem(batch=2, num_q_heads=32, num_kv_heads=4, head_dim=128, kv_dtype=torch.bfloat16)
    O_s, m_s, l_s = (x.double().cpu().numpy() for x in fd.workspace_views(prob, res.plan, res.workspace))
    Oo, mo, lo = oracle.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, C)
    for b, L in enumerate(wl.lens):
        S = -(-L // C)
        assert np.allclose(m_s[b, :, :S], mo[b, :, :S], rtol=0, atol=1e-5)
        assert np.allclose(l_s[b, :, :S], lo[b, :, :S], rtol=1e-5, atol=0)
        scale = np.abs(Oo[b, :, :S]).max()
        assert np.max(np.abs(O_s[b, :, :S] - Oo[b, :, :S])) <= 1e-5 * max(1.0, scale) * 8


@pytest.mark.parametrize("kernel", [0, 1, 4])
@pytest.mark.parametrize("page", [0, 16])
def test_large_batch_work_list(fd, monkeypatch, kernel, page):
    """More than 64 sequences: the work-list lookup scans the lengths in
    several 64-lane blocks; full and short splits interleave across blocks."""
    monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    g = np.random.default_rng(77)
    lens = [int(x) for x in g.integers(1, 700, size=150)] + [64, 128, 1]
    wl = make_workload(name=f"bigbatch-k{kernel}-p{page}", batch=len(lens), num_q_heads=16, num_kv_heads=4,
                       head_dim=128, seq_lens=lens, dtype=torch.bfloat16, seed=78, page_size=page)
    for splits in (0, 5):
        res = run(fd, wl, num_splits=splits)
        ref_out, ref_lse = reference(wl)
        parity(res.out, res.lse, ref_out, ref_lse, what=f"B={len(lens)} kernel {kernel} page {page} splits {splits}")


MHA_CASES = [
    # (d, dtype, Hq, Hkv, lens, page) -- Hkv a multiple of the rows one load covers
    (128, torch.float16, 8, 8, [1, 15, 16, 17, 2000], 0),
    (128, torch.bfloat16, 16, 8, [700, 3001], 0),       # G = 2
    (64, torch.float16, 16, 16, [5, 999, 4096], 0),     # d = 64: 8 heads per load
    (128, torch.float16, 32, 32, [1500, 33], 16),       # paged
    (64, torch.bfloat16, 8, 8, [17, 260], 16),          # paged, d = 64
    (64, torch.float16, 64, 64, [300, 2100], 0),        # d = 64, 64 heads: head columns apply
    (128, torch.bfloat16, 64, 32, [900, 64, 1], 16),    # G = 2, 32 KV heads, paged: head columns apply
]


# Head columns (kernel 3) need a multiple of 8 waves x the heads of one load:
# only the cases with enough KV heads run it.
MHA_KERNEL_CASES = [(k, c) for c in range(len(MHA_CASES)) for k in (0, 2, 3)
                    if k != 3 or MHA_CASES[c][3] % (8 * 64 // (MHA_CASES[c][0] // 8)) == 0]


@pytest.mark.parametrize("kernel,case", MHA_KERNEL_CASES)
@pytest.mark.parametrize("splits", [0, 3, 7])
def test_token_rows_and_head_rows_kernels_agree_with_oracle(fd, monkeypatch, kernel, case, splits):
    """The three vector-ALU partial kernels on the same inputs; forced split
    counts make paged splits start mid-page (per-token page lookups)."""
    d, dt, hq, hkv, lens, page = MHA_CASES[case]
    monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    wl = make_workload(name=f"mha{case}-k{kernel}", batch=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                       head_dim=d, seq_lens=lens, dtype=dt, seed=400 + case, page_size=page)
    res = run(fd, wl, num_splits=splits)
    assert res.plan.partial_kernel == kernel
    ref_out, ref_lse = reference(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"mha case {case} kernel {kernel} splits {splits}")


# ------------------------------------------------- several query tokens (n1)


MQ_CASES = [
    # (dtype, Hq, Hkv, q_len, lens, page)
    (torch.float16, 8, 8, 4, [4, 17, 1000], 0),       # MHA, 4 draft tokens
    (torch.bfloat16, 32, 8, 4, [600, 4096], 0),       # G = 4: 16 query rows
    (torch.bfloat16, 64, 8, 2, [100, 3000], 16),      # G = 8, paged
    (torch.float16, 4, 2, 8, [8, 9, 777], 16),        # G = 2, 8 tokens, paged
    (torch.float16, 16, 16, 16, [16, 2048], 0),       # MHA, 16 tokens
    (torch.bfloat16, 8, 8, 3, [5, 300], 0),           # 3 rows padded to 4
    (torch.bfloat16, 64, 8, 4, [100, 3000], 16),      # G = 8, 4 tokens: 32 rows, two column tiles
    (torch.bfloat16, 64, 8, 8, [8, 5000], 0),         # G = 8, 8 tokens: 64 rows, four column tiles
    (torch.float16, 8, 2, 10, [10, 700, 33], 16),     # G = 4, 10 tokens: 40 rows, a half-full last tile
    (torch.float16, 32, 32, 64, [64, 1500], 0),       # MHA, 64 tokens
]


@pytest.mark.parametrize("case", range(len(MQ_CASES)))
@pytest.mark.parametrize("splits", [0, 3, 64])
def test_multi_query_decode_matches_oracle(fd, case, splits):
    dt, hq, hkv, ql, lens, page = MQ_CASES[case]
    wl = make_workload(name=f"mq{case}", batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                       seq_lens=lens, dtype=dt, seed=500 + case, page_size=page, q_len=ql)
    res = run(fd, wl, num_splits=splits)
    assert res.plan.partial_kernel in (1, 4) and tuple(res.out.shape) == (len(lens), ql, hq, 128)
    ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                                     wl.page_size)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"multi-query case {case} splits {splits}")


@pytest.mark.parametrize("hq,hkv,ql", [(4, 2, 8), (16, 2, 5)])
def test_multi_query_split_statistics_include_empty_splits(fd, hq, hkv, ql):
    """Splits past a query's causal limit hold (m, l, O) = (-inf, 0, 0); with
    40 rows per KV head (three column tiles) the first tile's rows are all
    past their limits in the last splits."""
    wl = make_workload(name="mq-stats", batch=2, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seq_lens=[64, 30],
                       dtype=torch.bfloat16, seed=9, q_len=ql)
    res = run(fd, wl, num_splits=32)  # chunk 2: the last splits lie past the early queries' limits
    C = res.plan.chunk_tokens
    prob = fd.make_problem(batch=2, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, kv_dtype=torch.bfloat16,
                           q_len=ql)
    O_s, m_s, l_s = (x.double().cpu().numpy() for x in fd.workspace_views(prob, res.plan, res.workspace))
    Oo, mo, lo = oracle.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, C)
    for b, L in enumerate(wl.lens):
        S = -(-L // C)
        assert np.array_equal(np.isinf(m_s[b, :, :S]), np.isinf(mo[b, :, :S]))
        fin = np.isfinite(mo[b, :, :S])
        assert np.allclose(m_s[b, :, :S][fin], mo[b, :, :S][fin], rtol=0, atol=1e-5)
        assert np.allclose(l_s[b, :, :S], lo[b, :, :S], rtol=1e-5, atol=0)
        assert np.allclose(O_s[b, :, :S], Oo[b, :, :S], rtol=1e-5, atol=1e-5)


# ------------------------------------------------------- the four combine forms


@pytest.mark.parametrize("case", [
    # (d, dtype, Hq, Hkv, lens, page, q_len, out dtype)
    (128, torch.bfloat16, 64, 8, [7, 3000, 600, 17, 12000, 1] * 4, 16, 1, torch.float32),   # balanced list
    (64, torch.float16, 8, 2, [1, 300, 4097, 2, 900], 0, 1, torch.bfloat16),                # d = 64, bf16 out
    (128, torch.float16, 16, 16, [70000, 5], 0, 1, torch.float16),                          # many splits per row
    (128, torch.bfloat16, 32, 8, [40, 2500, 9, 800], 16, 4, torch.float32),                 # 4 query tokens
    (128, torch.float16, 3, 3, [5000, 17, 900], 0, 1, torch.float32),                       # odd rows: no pairs
    (128, torch.float16, 3, 3, [1 + (i * 37) % 700 for i in range(1500)], 0, 1, torch.float32),  # 4500 odd rows
    (128, torch.bfloat16, 2, 2, [900, 17, 3000, 1, 64], 0, 1, torch.float32),      # 10 rows: a part-filled last group
    (128, torch.float16, 4, 4, [600000, 3], 0, 1, torch.float32),                # hundreds of splits per row
])
def test_combine_forms_agree(fd, monkeypatch, case):
    """Four waves per (sequence, query row), one wave per row, two rows per
    wave and sixteen waves per row merge the same partials to the oracle's
    result; FD_COMBINE_FORM forces each."""
    d, dt, hq, hkv, lens, page, ql, od = case
    wl = make_workload(name="combine-forms", batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                       seq_lens=lens, dtype=dt, seed=1700 + d + hq + ql, q_len=ql)
    if page:
        wl = to_paged(wl, 16)
    dev = to_dev(wl)
    outs = {}
    for form in (0, 1, 2, 3):
        monkeypatch.setenv("FD_COMBINE_FORM", str(form))
        res = run(fd, wl, num_splits=0, out_dtype=od, dev_tensors=dev)
        outs[form] = res
    if ql > 1:
        ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                                         wl.page_size)
    else:
        ref_out, ref_lse = reference(wl)
    rnd = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}[od]
    for form, res in outs.items():
        o = res.out.double().cpu().numpy()
        assert np.isfinite(o).all()
        assert np.max(np.abs(o - ref_out)) <= O_MAX_ABS + rnd * np.abs(ref_out).max(), form
        assert np.max(np.abs(res.lse.double().cpu().numpy() - ref_lse)) <= LSE_ABS, form
    # the same partials: the forms differ by fp32 summation order (and one output rounding)
    for form in (1, 2, 3):
        diff = (outs[form].out.double() - outs[0].out.double()).abs().max().item()
        assert diff <= 1e-5 + 2 * rnd * float(outs[0].out.double().abs().max()), (form, diff)


@pytest.mark.parametrize("splits", [0, 5])
def test_bound_one_shot_call_matches_the_three_calls(fd, splits):
    """bind_decode_attention's callable (the one-shot C call with its
    arguments converted once; with a forced split count, the three C calls
    with theirs) gives, bit for bit, what plan + partial + combine give
    through the binding, on every call (16-bit and FP8, contiguous and
    paged)."""
    from workloads import quantize_kv_fp8
    dev = torch.device("cuda", 0)
    for fp8, page in ((False, 0), (True, 16)):
        wl = make_workload(name="bound", batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128,
                           seq_lens=[700, 3000, 65], dtype=torch.bfloat16, seed=1201, page_size=page)
        if fp8:
            wl = quantize_kv_fp8(wl)
        announce(f"bound one-shot call fp8={fp8} page={page}")
        q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
        bt = wl.block_table.to(dev) if wl.paged else None
        lens_dev = wl.seq_lens.to(dev)
        ks = wl.k_scale.to(dev) if fp8 else None
        vs = wl.v_scale.to(dev) if fp8 else None
        prob = fd.make_problem(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128, kv_dtype=wl.kv_dtype,
                               q_dtype=torch.bfloat16, out_dtype=torch.float32, scale=wl.scale,
                               page_size=page, max_pages_per_seq=wl.max_pages_per_seq)
        plan = fd.fd_plan_splits(prob, wl.lens, 0, splits)
        if splits:
            assert plan.max_splits == splits
        ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
        o1 = torch.empty(tuple(wl.q.shape), dtype=torch.float32, device=dev)
        l1 = torch.empty(tuple(wl.q.shape[:-1]), dtype=torch.float32, device=dev)
        fd.fd_decode_partial(prob, plan, q, k, v, bt, lens_dev, ws, None, ks, vs)
        fd.fd_combine(prob, plan, lens_dev, ws, o1, l1)
        o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
        run = fd.bind_decode_attention(prob, q, k, v, bt, wl.lens, lens_dev, o2, l2, ws, None, ks, vs,
                                       num_splits=splits)
        for _ in range(3):
            o2.fill_(float("nan"))
            run()
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2)
