"""GPU test of fd_decode_attention_noalloc: the allocation-free entry point.

It runs the same plan, partial and merge kernels as fd_decode_attention with
its partials in the library's fixed per-GPU buffer instead of a caller's
workspace, so on the same inputs and stream its outputs must equal the
workspace call's bit for bit, and both must meet the parity bar against the
oracle. Two calls in a row, the second on a smaller batch, show that what the
first call left in the buffer does not reach the second's result. A plan
that needs more than the buffer holds is refused on the host.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_parity_gpu import announce, parity, to_dev
from workloads import make_config, make_workload, quantize_kv_fp8
from workloads.synth import to_paged

pytestmark = pytest.mark.gpu


def _problem(fd, wl):
    return fd.make_problem(batch=wl.batch, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                           head_dim=wl.head_dim, kv_dtype=wl.kv_dtype, q_dtype=wl.dtype, scale=wl.scale,
                           page_size=wl.page_size, max_pages_per_seq=wl.max_pages_per_seq, q_len=wl.q_len)


def _both_calls(fd, wl):
    """The workspace call, then the allocation-free call, on one stream."""
    q, k, v, bt = to_dev(wl)
    dev = q.device
    ks = wl.k_scale.to(dev) if wl.k_scale is not None else None
    vs = wl.v_scale.to(dev) if wl.v_scale is not None else None
    prob = _problem(fd, wl)
    plan = fd.fd_plan_splits(prob, wl.lens)
    assert plan.workspace_bytes <= fd.NOALLOC_WORKSPACE_BYTES
    announce(f"noalloc {wl.name} B={wl.batch} {wl.kv_dtype} plan={plan.as_dict()}")
    lens_dev = wl.seq_lens.to(dev)
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    shape = tuple(wl.q.shape)
    out_ws = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    lse_ws = torch.full(shape[:-1], float("nan"), dtype=torch.float32, device=dev)
    fd.fd_decode_attention(prob, q, k, v, bt, wl.lens, lens_dev, out_ws, lse_ws, ws, k_scale=ks, v_scale=vs)
    out = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full(shape[:-1], float("nan"), dtype=torch.float32, device=dev)
    fd.fd_decode_attention_noalloc(prob, q, k, v, bt, wl.lens, lens_dev, out, lse, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out, lse


def _check_against_oracle(wl, out, lse, npairs):
    rng = np.random.default_rng(wl.seed)
    pairs = sorted({(int(rng.integers(0, wl.batch)), int(rng.integers(0, wl.num_q_heads))) for _ in range(npairs)}
                   | {(0, 0), (wl.batch - 1, wl.num_q_heads - 1)})
    ref_out, ref_lse = oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                               wl.page_size, pairs=pairs, k_scale=wl.k_scale, v_scale=wl.v_scale)
    parity(out, lse, ref_out, ref_lse, what=f"noalloc {wl.name}")


def test_noalloc_equals_workspace_call_twice_shrinking():
    import split_kv_flash_decoding_amd as fd

    fd.load_library()
    large = make_config(4)  # 16 sequences of 1024-16384 tokens, 32/8 heads, bf16
    small = to_paged(make_workload(name="noalloc-small", batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128,
                                   seq_lens=[700, 33, 2100], dtype=torch.float16, seed=2601), 16)
    for wl in (large, small):
        out_ws, lse_ws, out, lse = _both_calls(fd, wl)
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        assert torch.equal(out, out_ws), (out - out_ws).abs().max().item()
        assert torch.equal(lse, lse_ws), (lse - lse_ws).abs().max().item()
        _check_against_oracle(wl, out, lse, 48)


def test_noalloc_fp8_cache():
    import split_kv_flash_decoding_amd as fd

    fd.load_library()
    wl = quantize_kv_fp8(to_paged(make_workload(name="noalloc-fp8", batch=5, num_q_heads=32, num_kv_heads=8,
                                                head_dim=128, seq_lens=[4000, 17, 900, 1, 2500],
                                                dtype=torch.bfloat16, seed=2602), 16))
    out_ws, lse_ws, out, lse = _both_calls(fd, wl)
    assert torch.equal(out, out_ws) and torch.equal(lse, lse_ws)
    _check_against_oracle(wl, out, lse, 40)


def test_noalloc_refuses_a_plan_larger_than_its_buffer():
    """Eight query tokens of 64 heads for 512 sequences: 262144 query rows,
    130 MiB of partials even at one split each, more than the buffer holds:
    refused on the host, nothing launched."""
    import split_kv_flash_decoding_amd as fd

    fd.load_library()
    B, hq, hkv, ql = 512, 64, 8, 8
    lens = [64] * B
    prob = fd.make_problem(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, kv_dtype=torch.bfloat16,
                           page_size=16, max_pages_per_seq=4, q_len=ql)
    plan = fd.fd_plan_splits(prob, lens)
    assert plan.workspace_bytes > fd.NOALLOC_WORKSPACE_BYTES, plan.as_dict()
    dev = torch.device("cuda", 0)
    q = torch.zeros((B, ql, hq, 128), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((4, 16, hkv, 128), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, 4), dtype=torch.int32, device=dev)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = torch.zeros((B, ql, hq, 128), dtype=torch.float32, device=dev)
    lse = torch.zeros((B, ql, hq), dtype=torch.float32, device=dev)
    with pytest.raises(fd.FdError) as err:
        fd.fd_decode_attention_noalloc(prob, q, kv, kv, bt, lens, lens_dev, out, lse)
    assert err.value.status == fd.FD_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert not out.any()
