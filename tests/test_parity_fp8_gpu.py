"""GPU parity for FP8 (OCP E4M3) KV caches with per-KV-head scales.

The oracle decodes every code by the format's definition and multiplies by
the head's scale in fp64; the kernels widen the codes exactly and fold the
scales into the score scale and the split outputs. The values attention sees
are the same, so the tolerances are those of the 16-bit caches.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_parity_gpu import announce, parity
from workloads import make_config, make_workload, quantize_kv_fp8

pytestmark = pytest.mark.gpu


def run_fp8(fd, wl, num_splits=None, out_dtype=torch.float32):
    dev = torch.device("cuda", 0)
    bt = wl.block_table.to(dev) if wl.paged else None
    ns = wl.force_num_splits if num_splits is None else num_splits
    announce(f"{wl.name} B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} d={wl.head_dim} q={wl.dtype} "
             f"kv={wl.kv_dtype} q_len={wl.q_len} page={wl.page_size} splits={ns or 'auto'} seed={wl.seed}")
    res = fd.decode_attention(wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), wl.seq_lens, block_table=bt,
                              page_size=wl.page_size, max_pages_per_seq=wl.max_pages_per_seq, scale=wl.scale,
                              out_dtype=out_dtype, num_splits=ns, k_scale=wl.k_scale.to(dev),
                              v_scale=wl.v_scale.to(dev))
    torch.cuda.synchronize()
    return res


def reference_fp8(wl):
    if wl.q_len > 1:
        return oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                             wl.page_size, k_scale=wl.k_scale, v_scale=wl.v_scale)
    return oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table, wl.page_size,
                                   k_scale=wl.k_scale, v_scale=wl.v_scale)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_fp8_config_parity(fd, cfg):
    wl = make_config(cfg, kv_fp8=True)
    res = run_fp8(fd, wl)
    ref_out, ref_lse = reference_fp8(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"fp8 config {cfg} plan={res.plan.as_dict()}")


FP8_SHAPES = [
    # (d, q dtype, Hq, Hkv, lens, page)
    (64, torch.float16, 8, 8, [1024], 0),                          # 4 lanes per row
    (64, torch.bfloat16, 16, 16, [3000, 17], 0),                   # 16 heads per head-rows load
    (64, torch.bfloat16, 8, 2, [1, 17, 300, 2049], 0),             # G = 4 on the vector kernel
    (128, torch.float16, 4, 4, [1, 15, 16, 17, 63, 64, 65, 255], 0),
    (128, torch.bfloat16, 16, 2, [1000, 3001, 77], 0),             # G = 8, matrix cores
    (128, torch.float16, 16, 16, [70000], 0),
    (128, torch.bfloat16, 32, 8, [513, 1, 2500], 16),              # paged, matrix cores
    (128, torch.float16, 16, 8, [100, 4000, 33], 16),              # paged, G = 2
    (128, torch.bfloat16, 32, 32, [40000, 77], 0),                 # 32 heads: head columns apply
]


@pytest.mark.parametrize("shape", range(len(FP8_SHAPES)))
@pytest.mark.parametrize("splits", [0, 1, 3, 64])
def test_fp8_shapes_and_forced_splits(fd, shape, splits):
    d, qdt, hq, hkv, lens, page = FP8_SHAPES[shape]
    wl = quantize_kv_fp8(make_workload(name=f"fp8shape{shape}", batch=len(lens), num_q_heads=hq,
                                       num_kv_heads=hkv, head_dim=d, seq_lens=lens, dtype=qdt, seed=700 + shape,
                                       page_size=page))
    res = run_fp8(fd, wl, num_splits=splits)
    ref_out, ref_lse = reference_fp8(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"fp8 shape {shape} splits {splits}")


@pytest.mark.parametrize("shape", [0, 1, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("kernel", [0, 1, 2, 3, 4])
def test_fp8_every_partial_kernel(fd, monkeypatch, shape, kernel):
    """Each partial kernel that covers a shape (the planner keeps its own
    choice when the forced one does not apply)."""
    d, qdt, hq, hkv, lens, page = FP8_SHAPES[shape]
    monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    wl = quantize_kv_fp8(make_workload(name=f"fp8shape{shape}", batch=len(lens), num_q_heads=hq,
                                       num_kv_heads=hkv, head_dim=d, seq_lens=lens, dtype=qdt, seed=700 + shape,
                                       page_size=page))
    res = run_fp8(fd, wl, num_splits=0)
    ref_out, ref_lse = reference_fp8(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"fp8 shape {shape} kernel {res.plan.partial_kernel}")


def test_fp8_scales_reach_the_right_heads(fd):
    """Distinct powers of two per KV head on top of the quantiser's scales:
    the GPU must apply each head's K and V scale to that head's group only."""
    wl = quantize_kv_fp8(make_workload(name="fp8scales", batch=2, num_q_heads=16, num_kv_heads=4, head_dim=128,
                                       seq_lens=[900, 2100], dtype=torch.bfloat16, seed=731))
    wl.k_scale = wl.k_scale * torch.tensor([1.0, 0.25, 2.0, 0.5])
    wl.v_scale = wl.v_scale * torch.tensor([8.0, 1.0, 0.125, 4.0])
    res = run_fp8(fd, wl)
    ref_out, ref_lse = reference_fp8(wl)
    parity(res.out, res.lse, ref_out, ref_lse, o_tol=2e-3 * 8, what="per-head scales")


def test_fp8_split_statistics_match_oracle(fd):
    wl = quantize_kv_fp8(make_workload(name="fp8stats", batch=2, num_q_heads=8, num_kv_heads=8, head_dim=128,
                                       seq_lens=[1500, 333], dtype=torch.float16, seed=732))
    res = run_fp8(fd, wl, num_splits=5)
    prob = fd.make_problem(batch=2, num_q_heads=8, num_kv_heads=8, head_dim=128, kv_dtype=torch.float8_e4m3fn,
                           q_dtype=torch.float16)
    O_s, m_s, l_s = fd.workspace_views(prob, res.plan, res.workspace)
    Oo, mo, lo = oracle.decode_partials(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, res.plan.chunk_tokens,
                                        k_scale=wl.k_scale, v_scale=wl.v_scale)
    S = res.plan.max_splits
    for b, L in enumerate(wl.lens):
        n = -(-L // res.plan.chunk_tokens)
        assert np.allclose(m_s.double().cpu().numpy()[b, :, :n], mo[b, :, :n], rtol=0, atol=2e-5)
        assert np.allclose(l_s.double().cpu().numpy()[b, :, :n], lo[b, :, :n], rtol=2e-5, atol=0)
        assert np.allclose(O_s.double().cpu().numpy()[b, :, :n], Oo[b, :, :n], rtol=1e-4, atol=1e-4)
    assert S >= 1


@pytest.mark.parametrize("case", [(torch.float16, 8, 8, 4, [4, 17, 1000], 0),
                                  (torch.bfloat16, 32, 8, 4, [600, 4096], 0),
                                  (torch.bfloat16, 64, 8, 2, [100, 3000], 16),
                                  (torch.bfloat16, 64, 8, 8, [8, 3000], 16),     # 64 rows: four column tiles
                                  (torch.float16, 16, 16, 40, [40, 1200], 0)])   # 40 rows: three column tiles
def test_fp8_multi_query(fd, case):
    qdt, hq, hkv, ql, lens, page = case
    wl = quantize_kv_fp8(make_workload(name="fp8mq", batch=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                                       head_dim=128, seq_lens=lens, dtype=qdt, seed=740 + hq, page_size=page,
                                       q_len=ql))
    res = run_fp8(fd, wl, num_splits=0)
    assert res.plan.partial_kernel in (1, 4)
    ref_out, ref_lse = reference_fp8(wl)
    parity(res.out, res.lse, ref_out, ref_lse, what=f"fp8 multi-query {hq}/{hkv} q_len {ql}")


@pytest.mark.parametrize("L,fp8,chunk", [(8192, False, 256), (16384, False, 512), (16384, True, 256),
                                         (32768, True, 512)])
def test_shortened_head_row_splits(fd, L, fp8, chunk):
    """Batch 1, 32 heads: contexts too short for the head-rows kernel's usual
    1024-token (FP8: 2048) splits to give every CU a work-group get halved
    head-row splits from the planner, down to 256 tokens, instead of token
    rows; every head against the oracle."""
    wl = make_workload(name=f"mha{L}", batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128, seq_lens=[L],
                       dtype=torch.float16, seed=1500 + L // 1024)
    if fp8:
        wl = quantize_kv_fp8(wl)
        res = run_fp8(fd, wl)
        ref_out, ref_lse = reference_fp8(wl)
    else:
        from tests.test_parity_gpu import reference, run
        res = run(fd, wl)
        ref_out, ref_lse = reference(wl)
    assert (res.plan.partial_kernel, res.plan.chunk_tokens) == (2, chunk), res.plan.as_dict()
    parity(res.out, res.lse, ref_out, ref_lse, what=f"{L} tokens fp8={fp8} plan={res.plan.as_dict()}")
