"""GPU parity for fd_decode_fused: partials and merge in one launch.

The merge run by each head group's last work-group must give what the
separate combine kernel gives on the same partials, and the oracle's result;
the arrival counters must be back at zero after every call (several calls in
a row on one workspace, and graph replays, stay correct).
"""

import numpy as np
import pytest
import torch

from tests.test_parity_fp8_gpu import reference_fp8
from tests.test_parity_gpu import announce, parity
from workloads import make_config, make_workload
from workloads.synth import quantize_kv_fp8, to_paged

pytestmark = pytest.mark.gpu


def _setup(fd, wl, num_splits=0, out_dtype=torch.float32):
    dev = torch.device("cuda", 0)
    t = dict(q=wl.q.to(dev), k=wl.k.to(dev), v=wl.v.to(dev), bt=wl.block_table.to(dev) if wl.paged else None,
             lens=wl.seq_lens.to(dev),
             ks=wl.k_scale.to(dev) if wl.k_scale is not None else None,
             vs=wl.v_scale.to(dev) if wl.v_scale is not None else None)
    prob = fd.make_problem(batch=wl.batch, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                           head_dim=wl.head_dim, kv_dtype=wl.kv_dtype, q_dtype=wl.dtype, out_dtype=out_dtype,
                           scale=wl.scale, page_size=wl.page_size, max_pages_per_seq=wl.max_pages_per_seq,
                           q_len=wl.q_len)
    plan = fd.fd_plan_splits(prob, wl.lens, 0, num_splits or wl.force_num_splits)
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    fd.fd_workspace_init(prob, plan, ws)
    shape = tuple(wl.q.shape)
    return prob, plan, ws, t, shape


def _fused(fd, prob, plan, ws, t, shape, out_dtype=torch.float32):
    out = torch.full(shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full(shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    fd.fd_decode_fused(prob, plan, t["q"], t["k"], t["v"], t["bt"], t["lens"], ws, out, lse, None, t["ks"], t["vs"])
    return out, lse


def _two_launch(fd, prob, plan, t, shape, out_dtype=torch.float32):
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device="cuda")
    out = torch.empty(shape, dtype=out_dtype, device="cuda")
    lse = torch.empty(shape[:-1], dtype=torch.float32, device="cuda")
    fd.fd_decode_partial(prob, plan, t["q"], t["k"], t["v"], t["bt"], t["lens"], ws, None, t["ks"], t["vs"])
    fd.fd_combine(prob, plan, t["lens"], ws, out, lse)
    return out, lse


CASES = [
    ("config 1", lambda: make_config(1)),
    ("config 2", lambda: make_config(2)),
    ("config 3", lambda: make_config(3)),
    ("config 4", lambda: make_config(4)),
    ("config 5", lambda: make_config(5)),
    ("config 3 fp8", lambda: make_config(3, kv_fp8=True)),
    ("config 5 fp8", lambda: make_config(5, kv_fp8=True)),
    ("config 4 q_len 4", lambda: make_config(4, q_len=4)),
    ("G8 paged q_len 8", lambda: to_paged(make_workload(name="g8q8", batch=4, num_q_heads=64, num_kv_heads=8,
                                                        head_dim=128, seq_lens=[8, 700, 5000, 129],
                                                        dtype=torch.bfloat16, seed=1503, q_len=8), 16)),
    ("MHA q_len 40", lambda: make_workload(name="mq40", batch=2, num_q_heads=8, num_kv_heads=8, head_dim=128,
                                           seq_lens=[40, 2500], dtype=torch.float16, seed=1502, q_len=40)),
    ("d64 GQA paged", lambda: to_paged(make_workload(name="d64", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                                     seq_lens=[1, 300, 4097], dtype=torch.bfloat16, seed=1500), 16)),
    ("d64 fp8 head rows", lambda: quantize_kv_fp8(make_workload(name="d64f8", batch=1, num_q_heads=32,
                                                                num_kv_heads=16, head_dim=64, seq_lens=[200000],
                                                                dtype=torch.float16, seed=1501))),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_matches_two_launches_and_oracle(fd, case):
    name, mk = CASES[case]
    wl = mk()
    prob, plan, ws, t, shape = _setup(fd, wl)
    announce(f"fused {name}: plan={plan.as_dict()}")
    outs = []
    for rep in range(3):  # the counters must come back to zero after every call
        outs.append(_fused(fd, prob, plan, ws, t, shape))
    torch.cuda.synchronize()
    ref2 = _two_launch(fd, prob, plan, t, shape)
    torch.cuda.synchronize()
    for out, lse in outs:
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        assert torch.allclose(out, ref2[0], rtol=1e-6, atol=1e-7) and torch.allclose(lse, ref2[1], rtol=0, atol=1e-6)
    part = wl.batch * wl.q_len * wl.num_q_heads * plan.max_splits * (wl.head_dim + 2) * 4
    off = -(-part // 16) * 16 // 4
    assert int(ws.view(torch.int32)[off: off + wl.batch * wl.num_kv_heads].abs().sum()) == 0
    if wl.kv_dtype == torch.float8_e4m3fn:
        ref_out, ref_lse = reference_fp8(wl)
    elif wl.q_len > 1:
        import oracle
        ref_out, ref_lse = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                                         wl.page_size)
    else:
        import oracle
        ref_out, ref_lse = oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                                   wl.page_size)
    parity(outs[-1][0], outs[-1][1], ref_out, ref_lse, what=f"fused {name}")


@pytest.mark.parametrize("kernel", [0, 1, 2, 3, 4])
def test_fused_each_partial_kernel_and_output_type(fd, monkeypatch, kernel):
    monkeypatch.setenv("FD_PARTIAL_KERNEL", str(kernel))
    # head columns (3) need a multiple of 32 KV heads at d = 128
    hq, hkv = (64, 32) if kernel == 3 else (16, 8)
    wl = make_workload(name="fk", batch=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seq_lens=[5000, 17, 2300],
                       dtype=torch.bfloat16, seed=1510)
    for od in (torch.float32, torch.bfloat16):
        prob, plan, ws, t, shape = _setup(fd, wl, num_splits=0, out_dtype=od)
        assert plan.partial_kernel == kernel
        fused = _fused(fd, prob, plan, ws, t, shape, od)
        two = _two_launch(fd, prob, plan, t, shape, od)
        torch.cuda.synchronize()
        # the fused merge and the combine add the S splits in different orders:
        # fp32 sums of S terms that differ by up to about S rounding steps
        rtol = max(1e-6, plan.max_splits * 2.0 ** -23)
        assert torch.allclose(fused[0].float(), two[0].float(), rtol=rtol, atol=1e-7)
        assert torch.allclose(fused[1], two[1], rtol=0, atol=1e-6)


def test_fused_graph_replay(fd):
    wl = to_paged(make_workload(name="fg", batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128,
                                seq_lens=[700, 3000, 64, 1500], dtype=torch.bfloat16, seed=1520), 16)
    prob, plan, ws, t, shape = _setup(fd, wl)
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(shape[:-1], dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fd.fd_decode_fused(prob, plan, t["q"], t["k"], t["v"], t["bt"], t["lens"], ws, out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fd.fd_decode_fused(prob, plan, t["q"], t["k"], t["v"], t["bt"], t["lens"], ws, out, lse)
    import oracle
    for rep in range(4):
        t["q"].mul_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle.decode_attention(t["q"].cpu(), wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table, 16)
        parity(out, lse, ref_out, ref_lse, what=f"fused graph replay {rep}")
