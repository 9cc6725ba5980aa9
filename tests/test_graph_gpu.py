"""Decode steps replayed from one captured HIP graph.

The plan holds scalars only and the kernels derive every sequence's split
count from the device lengths, so one plan made for upper-bound lengths
serves every later step whose lengths stay within those bounds: a graph
captured once (partial + combine) is replayed as the sequences grow, with
only the contents of the length array and the cache changing. (Recording a
whole decode step and replaying it is the CUDA-graph practice described on
the attention-kernels page, "CUDA Graph" section.) Each replay is checked
against the oracle on that step's lengths, with eager work in between.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_parity_gpu import announce, parity
from workloads import make_workload
from workloads.synth import to_paged

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hq,hkv,dt", [(64, 8, torch.bfloat16), (32, 32, torch.float16)])
def test_graph_replay_across_growing_lengths(fd, hq, hkv, dt):
    B = 4
    final = [700, 3000, 64, 1500]           # the longest lengths any step reaches (plan bound)
    steps = [[650, 2950, 20, 1450], [651, 2951, 21, 1451], [700, 3000, 64, 1500]]
    wl = make_workload(name="graph", batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seq_lens=final,
                       dtype=dt, seed=1300 + hq)
    wl = to_paged(wl, 16, spare_pages=2)
    dev = torch.device("cuda", 0)
    q, k, v, bt = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), wl.block_table.to(dev)
    prob = fd.make_problem(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, kv_dtype=dt, scale=wl.scale,
                           page_size=16, max_pages_per_seq=wl.max_pages_per_seq)
    plan = fd.fd_plan_splits(prob, final)
    lens_dev = torch.tensor(steps[0], dtype=torch.int32, device=dev)
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    out = torch.empty((B, hq, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    announce(f"graph capture: Hq={hq} Hkv={hkv} {dt} plan={plan.as_dict()}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        fd.fd_decode_partial(prob, plan, q, k, v, bt, lens_dev, ws)
        fd.fd_combine(prob, plan, lens_dev, ws, out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fd.fd_decode_partial(prob, plan, q, k, v, bt, lens_dev, ws)
        fd.fd_combine(prob, plan, lens_dev, ws, out, lse)
    torch.cuda.synchronize()

    for rep in range(2):
        for lens in steps:
            lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
            q.mul_(-1.0)  # new queries every step (eager work between replays)
            graph.replay()
            torch.cuda.synchronize()
            qh = q.cpu()
            ref_out, ref_lse = oracle.decode_attention(qh, wl.k, wl.v, lens, wl.scale, wl.block_table, 16)
            parity(out, lse, ref_out, ref_lse, what=f"graph replay {rep} lens {lens}")
            # and the eager one-shot call on the same inputs agrees bit for bit
            res = fd.decode_attention(q, k, v, lens, block_table=bt, page_size=16,
                                      max_pages_per_seq=wl.max_pages_per_seq, scale=wl.scale)
            torch.cuda.synchronize()
            if res.plan.chunk_tokens == plan.chunk_tokens and res.plan.partial_kernel == plan.partial_kernel:
                assert torch.equal(res.out, out) and torch.equal(res.lse, lse)
            else:
                assert np.allclose(res.out.cpu().numpy(), out.cpu().numpy(), rtol=1e-5, atol=1e-6)
