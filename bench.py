#!/usr/bin/env python3
"""Split-KV decode attention benchmark on one MI355X.

One step is one pass of the whole decode path over the resident batch: the
host split planner, the partial kernel (per-split online softmax) and the
combine kernel. The default workload is the 128K-token MHA decode (batch 1,
32 heads, d = 128, fp16, 1% of key rows scaled by 4). Prints one JSON line.

  value     KV-read GB/s over the whole step = algorithmic KV bytes / step time
            (K and V read once: sum_b L_b * Hkv * d * 2 * sizeof(fp16))
  roofline  the partial kernel alone: the same bytes / its mean launch time,
            measured with HIP events around every 8th launch in the timed
            region (an event pair adds ~6 us to its step); runs of fewer than
            64 steps carry no pairs in the timed region and time the partial
            launches of a second pass of the same steps instead; against the
            8 TB/s HBM peak
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
            workload on this host (a reported baseline, not a target); the
            heads it computes are compared with the GPU output
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV-read GB/s and µs/call, decode attention 128K ctx b=1 (fraction of HBM peak)"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak
LAUNCH_BOUND_BYTES = 32 << 20  # decode: K/V bytes below which a call is bound by launch and latency
EVENT_EVERY = 8  # decode: steps per event-timed partial launch in the timed region (runs of 64+ steps)
KERNEL_SOURCES = os.path.join(ROOT, "split_kv_flash_decoding_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


# The sources the decode partial kernels and their launch (planner, entry
# points) are built from: counters taken on the partial kernel go stale when
# any of them changes.
PARTIAL_SOURCES = ("fd_api.hip", "fd_device.h", "fd_host.cpp", "fd_internal.h", "fd_partial_mfma.hip",
                   "fd_partial_valu.hip")


PREFILL_SOURCES = ("fd_api.hip", "fd_device.h", "fd_internal.h", "fd_prefill.hip")
APPEND_SOURCES = ("fd_api.hip", "fd_device.h", "fd_internal.h", "fd_append.hip")
SOURCES = {"partial": PARTIAL_SOURCES, "prefill": PREFILL_SOURCES, "append": APPEND_SOURCES}


def strip_comments(src: str) -> str:
    """C/C++ source without its // and /* */ comments (string and character
    literals kept), trailing blanks and blank lines, so that a comment-only
    edit keeps the hash."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(l.rstrip() for l in "".join(out).splitlines() if l.strip())


def kernel_source_hash(kernel: str = "partial") -> str:
    """Hash of the timed kernel's sources (SOURCES[kernel]), comments stripped:
    counters taken on a kernel stay current until its code changes."""
    h = hashlib.sha256()
    for name in SOURCES[kernel]:
        with open(os.path.join(KERNEL_SOURCES, name), encoding="utf-8") as f:
            h.update(name.encode() + strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def kv_bytes(wl) -> int:
    return wl.total_tokens * wl.num_kv_heads * wl.head_dim * 2 * wl.k.element_size()


def measured_traffic(workload: str, kernel: str = "partial"):
    """Per-launch HBM bytes of the timed kernel from committed rocprofv3 PMC
    runs, if they were taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def blas_threads() -> int:
    """Threads the oracle's NumPy BLAS runs with."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return 1


def cpu_baseline(wl, budget_s: float, out, lse):
    """Time the oracle, unchanged, on whole heads of the workload until the
    budget is spent, and compare the heads it computed with the GPU result."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    if wl.q_len > 1:
        t0 = time.perf_counter()
        ref_o, ref_l = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table,
                                                     wl.page_size, k_scale=wl.k_scale, v_scale=wl.v_scale)
        el = time.perf_counter() - t0
        d = out.double().cpu().numpy() - ref_o
        return {"value": kv_bytes(wl) / el / 1e9, "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
                "sample": f"the whole workload ({wl.q_len} query tokens per sequence), {el:.1f} s wall",
                "parity_of_sampled_heads": {
                    "o_max_abs": float(np.max(np.abs(d))),
                    "o_rel_rms": float(np.linalg.norm(d) / np.linalg.norm(ref_o)),
                    "lse_abs": float(np.max(np.abs(lse.double().cpu().numpy() - ref_l)))}}
    hq = wl.num_q_heads
    done = 0
    ref_o = ref_l = None
    t0 = time.perf_counter()
    # Whole query heads in turn, starting over once every head is done, until
    # the budget is spent (a few passes over a small workload, part of one
    # over a large one).
    while True:
        h = done % hq
        o, l = oracle.decode_attention(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, wl.block_table, wl.page_size,
                                       pairs=[(b, h) for b in range(wl.batch)], k_scale=wl.k_scale,
                                       v_scale=wl.v_scale)
        if done < hq:
            ref_o = o if ref_o is None else np.where(np.isnan(o), ref_o, o)
            ref_l = l if ref_l is None else np.where(np.isnan(l), ref_l, l)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    mask = ~np.isnan(ref_l)
    d = out.double().cpu().numpy()[mask] - ref_o[mask]
    parity = {"o_max_abs": float(np.max(np.abs(d))),
              "o_rel_rms": float(np.linalg.norm(d) / np.linalg.norm(ref_o[mask])),
              "lse_abs": float(np.max(np.abs(lse.double().cpu().numpy()[mask] - ref_l[mask])))}
    # Algorithmic bytes of the heads computed: a KV head serves G query heads.
    sample_bytes = wl.total_tokens * (done / wl.group_size) * wl.head_dim * 2 * wl.k.element_size()
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except Exception:
        model = "unknown"
    return {
        "value": sample_bytes / el / 1e9,
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{done} query heads ({done / hq:.2f} passes over the {hq}) x {wl.total_tokens} tokens "
                  f"(all batch rows), {el:.1f} s wall; fp64 NumPy oracle; host {model}, "
                  f"{len(os.sched_getaffinity(0))} cores in affinity mask",
        "us_per_call_extrapolated": el / done * hq * 1e6,
        "parity_of_sampled_heads": parity,
    }


def time_gbps(fn, nbytes: int, reps: int = 10) -> float:
    """GB/s of `fn` (which reads nbytes) over reps calls, timed by events."""
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return reps * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9


def probe_patterns(fd, k, v, sink, row_bytes: int, chunks=None) -> dict:
    """Read bandwidth of K and V (equal byte sizes) by access pattern: the
    plain streaming read (K, then V), and the row pattern of the decode
    kernels (include/fd_probe.h) over rows of row_bytes: 1 KB column blocks
    with the waves splitting the rows (head rows), at chunks that give about
    1, 2 and 4 work-groups per compute unit, plain and from rotated starts,
    and 8 KB blocks with the waves across them (head columns) where the rows
    hold 8 KB."""
    nbytes = 2 * k.numel() * k.element_size()
    out = {"stream": time_gbps(lambda: (fd.fd_probe_read(k, sink), fd.fd_probe_read(v, sink)), nbytes)}
    if row_bytes % 1024:
        return out
    rows = k.numel() * k.element_size() // row_bytes
    for per_cu in (1, 2, 4):
        chunk = max(16, -(-rows * (row_bytes // 1024) // (256 * per_cu)))
        out[f"rows_1k_{per_cu}wg_per_cu"] = time_gbps(
            lambda: fd.fd_probe_read_rows(k, v, row_bytes, chunk, 0, sink), nbytes)
        out[f"rows_1k_rot_{per_cu}wg_per_cu"] = time_gbps(
            lambda: fd.fd_probe_read_rows(k, v, row_bytes, chunk, 2, sink), nbytes)
    if row_bytes % 8192 == 0:
        for per_cu in (1, 2):
            chunk = max(16, -(-rows * (row_bytes // 8192) // (256 * per_cu)))
            out[f"cols_8k_{per_cu}wg_per_cu"] = time_gbps(
                lambda: fd.fd_probe_read_rows(k, v, row_bytes, chunk, 1, sink), nbytes)
    return out


PROBE_METRIC = "HBM read GB/s of the decode access patterns, 2 GiB K/V pair shaped as the 128K-token cache"


def run_probe(args, fd, dev) -> int:
    """One step = one read of a 1 GiB K and a 1 GiB V buffer shaped as the
    128K-token, 32-head, d = 128 fp16 cache ([131072, 8192 B]) in each
    pattern of probe_patterns; value = the best pattern's GB/s."""
    import torch

    rows, row_bytes = 131072, 8192
    k = torch.empty(rows * row_bytes // 2, dtype=torch.float16, device=dev).fill_(1.0)
    v = torch.empty_like(k).fill_(2.0)
    sink = torch.empty(fd.PROBE_SINK_FLOATS, dtype=torch.float32, device=dev)
    runs = [probe_patterns(fd, k, v, sink, row_bytes) for _ in range(max(1, args.steps // 10))]
    pats = {n: max(r[n] for r in runs) for n in runs[0]}
    for n, g in pats.items():
        log(f"{n}: {g:.0f} GB/s (best of {len(runs)} runs of 10 reads)")
    best, gbps = max(pats.items(), key=lambda kv: kv[1])
    rec = {
        "metric": PROBE_METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": len(runs) * 10,
        "warmup": 3, "ms_per_step": round(2 * rows * row_bytes / (gbps * 1e9) * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic (constant-filled buffers)",
        "config": {"workload": "hbm_read_patterns_2x1GiB_rows8192", "rows": rows, "row_bytes": row_bytes,
                   "best_pattern": best, "patterns_gbps": {n: round(g, 1) for n, g in pats.items()}},
        "roofline": {"bound": "hbm", "kernel": f"probe ({best})", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


PREFILL_METRIC = "TFLOP/s, causal prefill attention (FA-2 forward), 8K tokens, GQA 32/8, d=128"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA peak


def prefill_flops(wl) -> float:
    """Algorithmic flops: 4d per (query row, visible token, query head) (2d for
    the score, 2d for the weighted sum of V)."""
    q_len = wl.q.shape[1]
    visible = sum(sum(L - q_len + i + 1 for i in range(q_len)) for L in wl.lens)
    return 4.0 * wl.head_dim * wl.num_q_heads * visible


def run_prefill(args, fd, dev) -> int:
    """One step = one fd_prefill_attention call over the resident prompt."""
    import numpy as np
    import torch

    from workloads import make_prefill

    t = time.perf_counter()
    wl = make_prefill()
    log(f"generated {wl.name} in {time.perf_counter() - t:.1f} s")
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    lens_dev = wl.seq_lens.to(dev)
    q_len = wl.q.shape[1]
    problem = fd.make_problem(batch=wl.batch, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                              head_dim=wl.head_dim, kv_dtype=wl.dtype, out_dtype=torch.float32, scale=wl.scale,
                              q_len=q_len)
    out = torch.empty(tuple(q.shape), dtype=torch.float32, device=dev)
    lse = torch.empty(tuple(q.shape[:-1]), dtype=torch.float32, device=dev)
    flops = prefill_flops(wl)
    for _ in range(max(1, args.warmup)):
        fd.fd_prefill_attention(problem, q, k, v, None, lens_dev, out, lse)
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for _ in range(K):
        fd.fd_prefill_attention(problem, q, k, v, None, lens_dev, out, lse)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end) / K
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{K} steps: {ms * 1e3:.1f} us/step (events), wall {wall / K * 1e6:.1f} us/step; {tflops:.1f} TFLOP/s")
    # A plain copy of known size calibrates the HBM counters taken on this run.
    src = torch.empty((256 << 20) // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    fd.fd_probe_copy(dst, src)
    torch.cuda.synchronize()
    del src, dst
    traffic = measured_traffic(wl.name, "prefill")
    rec = {
        "metric": PREFILL_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) q/K/V; no dataset involved)",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.num_q_heads,
                   "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "q_len": q_len,
                   "seq_lens_total": wl.total_tokens, "accumulate": "f32", "out_dtype": "f32",
                   "flops_per_call": flops},
        # The kernel is the whole step: one launch, timed by the same events.
        "roofline": {"bound": "mfma", "kernel": "prefill", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        import oracle

        log(f"timing the CPU oracle on sampled query rows for about {args.cpu_budget:.0f} s ...")
        r = np.random.default_rng(0)
        done, fl = 0, 0.0
        t0 = time.perf_counter()
        ref_rows = []
        while time.perf_counter() - t0 < args.cpu_budget:
            rows = [(0, int(r.integers(0, q_len)), int(r.integers(0, wl.num_q_heads))) for _ in range(64)]
            o, l = oracle.decode_attention_multi(wl.q, wl.k, wl.v, wl.seq_lens, wl.scale, rows=rows)
            for (b, i, h) in rows:
                fl += 4.0 * wl.head_dim * (wl.lens[b] - q_len + i + 1)
                ref_rows.append((b, i, h, o[b, i, h], l[b, i, h]))
            done += len(rows)
        el = time.perf_counter() - t0
        got = out.double().cpu().numpy()
        got_l = lse.double().cpu().numpy()
        d_o = np.concatenate([got[b, i, h] - o_ for b, i, h, o_, _ in ref_rows])
        ref_o = np.concatenate([o_ for _, _, _, o_, _ in ref_rows])
        rec["cpu_baseline"] = {
            "value": round(fl / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} random (row, head) pairs of the same prompt, {el:.1f} s wall",
            "parity_of_sampled_rows": {
                "o_max_abs": float(np.max(np.abs(d_o))),
                "o_rel_rms": float(np.linalg.norm(d_o) / np.linalg.norm(ref_o)),
                "lse_abs": float(max(abs(got_l[b, i, h] - l_) for b, i, h, _, l_ in ref_rows))}}
    else:
        rec["cpu_baseline"] = None
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


APPEND_METRIC = "GB/s, KV append with RoPE into the paged cache (q rotated in place), 8K-token prompt, GQA 32/8, d=128"


def append_bytes(n_tokens: int, hq: int, hkv: int, d: int, elem: int, cache_elem: int) -> int:
    """Algorithmic bytes of an append: per new token, k_new and v_new read,
    their cache rows written, q read and written back."""
    return n_tokens * (2 * hkv * d * elem + 2 * hkv * d * cache_elem + 2 * hq * d * elem)


def run_append(args, fd, dev) -> int:
    """One step = one fd_append_kv call: the prompt's keys (rotated) and values
    into the paged cache, and its queries rotated in place."""
    import numpy as np
    import torch

    from workloads import make_append, make_workload
    from workloads.synth import to_paged

    t = time.perf_counter()
    wl, k_new_h, v_new_h = make_append()
    log(f"generated {wl.name} in {time.perf_counter() - t:.1f} s")
    n = wl.q.shape[1]
    kc, vc = wl.k.to(dev), wl.v.to(dev)
    q = wl.q.to(dev).contiguous()
    k_new, v_new = k_new_h.to(dev), v_new_h.to(dev)
    bt, lens_dev = wl.block_table.to(dev), wl.seq_lens.to(dev)
    problem = fd.make_problem(batch=1, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                              head_dim=wl.head_dim, kv_dtype=wl.dtype, page_size=16,
                              max_pages_per_seq=wl.max_pages_per_seq, q_len=n)
    nbytes = append_bytes(n, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 2, 2)

    def call():
        fd.fd_append_kv(problem, k_new, v_new, q, kc, vc, bt, lens_dev, rope_style="half", rope_base=10000.0)

    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for _ in range(K):
        call()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end) / K
    # The spread, from a second run with an event pair around every call.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(min(K, 50) + 1)]
    ev[0].record()
    for i in range(len(ev) - 1):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    gbps = nbytes / (ms * 1e-3) / 1e9
    pq = statistics.quantiles(per, n=10)
    log(f"{K} steps: {ms * 1e3:.1f} us/step (events), wall {wall / K * 1e6:.1f} us/step; {gbps:.0f} GB/s; "
        f"median {statistics.median(per) * 1e3:.1f} us, p10 {pq[0] * 1e3:.1f}, p90 {pq[-1] * 1e3:.1f}")

    # A decode step's append for context (latency-bound): 64 sequences, one
    # new token each, 64 query / 8 KV heads.
    st = to_paged(make_workload(name="append_step", batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128,
                                seq_lens=("uniform", 1, 64), dtype=torch.bfloat16, seed=2200), 16, spare_pages=1)
    sp = fd.make_problem(batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, kv_dtype=torch.bfloat16,
                         page_size=16, max_pages_per_seq=st.max_pages_per_seq, q_len=1)
    s_q = st.q.reshape(64, 1, 64, 128).to(dev).contiguous()
    s_k, s_v, s_bt, s_lens = st.k.to(dev), st.v.to(dev), st.block_table.to(dev), st.seq_lens.to(dev)
    s_new = torch.randn((64, 1, 8, 128), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).to(dev)
    for _ in range(10):
        fd.fd_append_kv(sp, s_new, s_new, s_q, s_k, s_v, s_bt, s_lens, rope_style="half")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(100):
        fd.fd_append_kv(sp, s_new, s_new, s_q, s_k, s_v, s_bt, s_lens, rope_style="half")
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / 100 * 1e3
    log(f"decode-step append (64 sequences x 1 token, 64/8 heads): {step_us:.1f} us")
    # A plain copy of known size calibrates the HBM counters taken on this run.
    src = torch.empty((256 << 20) // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    fd.fd_probe_copy(dst, src)
    torch.cuda.synchronize()
    del src, dst

    rec = {
        "metric": APPEND_METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) q/K/V; no dataset involved)",
        "config": {"workload": wl.name, "batch": 1, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "new_tokens": n, "page_size": 16, "rope": "half, base 10000",
                   "bytes_per_call": nbytes, "decode_step_append_us": round(step_us, 2)},
        # One launch per step, timed by the same events.
        "roofline": {"bound": "hbm", "kernel": "append", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(wl.name, "append"),
                     "us_median": round(statistics.median(per) * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        import oracle.append as oapp

        # The GPU result of one append on the original queries, then the
        # oracle token by token (each sampled token as a one-token sequence
        # ending at its position) until the budget is spent.
        q.copy_(wl.q.reshape(q.shape))
        call()
        torch.cuda.synchronize()
        got_k, got_v, got_q = kc.cpu(), vc.cpu(), q.cpu()
        log(f"timing the CPU oracle on sampled tokens for about {args.cpu_budget:.0f} s ...")
        r = np.random.default_rng(0)
        done, mism, total_el = 0, 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_budget:
            js = [int(j) for j in r.integers(0, n, 8)]
            table = wl.block_table[0:1].repeat(len(js), 1)
            lens = [j + 1 for j in js]
            rk, rv, rq = oapp.append_kv(wl.k, wl.v, table, lens, k_new_h[0, js][:, None], v_new_h[0, js][:, None],
                                        wl.q[0, js][:, None], rope_style="half", rope_base=10000.0)
            for i, j in enumerate(js):
                pg, sl = int(wl.block_table[0, j // 16]), j % 16
                for got, ref in ((got_k[pg, sl], rk[pg, sl]), (got_v[pg, sl], rv[pg, sl]), (got_q[0, j], rq[i, 0])):
                    mism += int((got.view(torch.int16) != ref.view(torch.int16)).sum())
                    total_el += got.numel()
            done += len(js)
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {
            "value": round(append_bytes(done, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 2, 2) / el / 1e9, 6),
            "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} random tokens of the same prompt, each appended alone at its position, "
                      f"{el:.1f} s wall (pure-Python rounding, one thread)",
            "parity_of_sampled_tokens": {"elements": total_el, "differing_bits": mism}}
    else:
        rec["cpu_baseline"] = None
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=("decode", "prefill", "append", "probe"), default="decode",
                    help="decode (default; --config picks the workload), the 8192-token causal prefill, the "
                         "8192-token KV append with RoPE, or the HBM read probes' access patterns")
    ap.add_argument("--config", type=int, default=3, help="decode workload 1..5 (default: 128K MHA)")
    ap.add_argument("--q-len", type=int, default=1, help="query tokens per sequence (speculative verification)")
    ap.add_argument("--kv-fp8", action="store_true", help="FP8 (E4M3) cache with per-KV-head scales")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", default=None)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: this decode path is built and timed on a single "
                         "MI355X; run it with --gpus 1.\n")
        return 2

    import torch

    import split_kv_flash_decoding_amd as fd
    from workloads import make_config

    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a GPU\n")
        return 2
    fd.load_library()
    dev = torch.device("cuda", 0)
    if args.workload == "prefill":
        return run_prefill(args, fd, dev)
    if args.workload == "append":
        return run_append(args, fd, dev)
    if args.workload == "probe":
        return run_probe(args, fd, dev)

    t = time.perf_counter()
    wl = make_config(args.config, q_len=args.q_len, kv_fp8=args.kv_fp8)
    log(f"generated {wl.name} in {time.perf_counter() - t:.1f} s")
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    bt = wl.block_table.to(dev) if wl.paged else None
    lens_host = wl.lens
    lens_dev = wl.seq_lens.to(dev)
    ks = wl.k_scale.to(dev) if wl.k_scale is not None else None
    vs = wl.v_scale.to(dev) if wl.v_scale is not None else None
    problem = fd.make_problem(batch=wl.batch, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                              head_dim=wl.head_dim, kv_dtype=wl.kv_dtype, q_dtype=wl.dtype, out_dtype=torch.float32,
                              scale=wl.scale, page_size=wl.page_size, max_pages_per_seq=wl.max_pages_per_seq,
                              q_len=wl.q_len)
    plan = fd.fd_plan_splits(problem, lens_host, 0, wl.force_num_splits)
    ws = torch.empty(-(-plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    out = torch.empty(tuple(wl.q.shape), dtype=torch.float32, device=dev)
    lse = torch.empty(tuple(wl.q.shape[:-1]), dtype=torch.float32, device=dev)
    nbytes = kv_bytes(wl)
    log(f"plan {plan.as_dict()}; KV bytes {nbytes}")

    def step():
        p = fd.fd_plan_splits(problem, lens_host, 0, wl.force_num_splits)
        fd.fd_decode_partial(problem, p, q, k, v, bt, lens_dev, ws, None, ks, vs)
        fd.fd_combine(problem, p, lens_dev, ws, out, lse)

    step()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # The partial kernel is timed by event pairs. A pair costs its step ~6 us
    # (measured on MI355X, 128K MHA: 323.2 us per step with a pair on every
    # step, 317.2 us without), so the timed region carries one on every
    # EVENT_EVERY-th step only, and runs too short for that (under
    # 8 * EVENT_EVERY steps) carry none: their partial launches are timed in a
    # second pass of K steps right after the timed region, a pair around every
    # partial launch.
    in_loop = K >= 8 * EVENT_EVERY
    timed = [i for i in range(K) if i % EVENT_EVERY == 0] if in_loop else []
    ev_a = {i: torch.cuda.Event(enable_timing=True) for i in timed}
    ev_b = {i: torch.cuda.Event(enable_timing=True) for i in timed}
    # Steps without a pair make the one-shot C call (planner, partial kernel,
    # combine) with its arguments converted once: the same GPU work as the
    # three calls, less host time ahead of the first launch. A workload with a
    # forced split count makes the three C calls (planner with the forced
    # count, partial kernel, combine) with their arguments converted once.
    one_shot = fd.bind_decode_attention(problem, q, k, v, bt, lens_host, lens_dev, out, lse, ws, None, ks, vs,
                                        num_splits=wl.force_num_splits)
    one_shot()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        if i not in ev_a:
            one_shot()
            continue
        p = fd.fd_plan_splits(problem, lens_host, 0, wl.force_num_splits)
        ev_a[i].record()
        fd.fd_decode_partial(problem, p, q, k, v, bt, lens_dev, ws, None, ks, vs)
        ev_b[i].record()
        fd.fd_combine(problem, p, lens_dev, ws, out, lse)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(end) / K
    if not in_loop:
        timed = list(range(K))
        ev_a = {i: torch.cuda.Event(enable_timing=True) for i in timed}
        ev_b = {i: torch.cuda.Event(enable_timing=True) for i in timed}
        for i in timed:
            p = fd.fd_plan_splits(problem, lens_host, 0, wl.force_num_splits)
            ev_a[i].record()
            fd.fd_decode_partial(problem, p, q, k, v, bt, lens_dev, ws, None, ks, vs)
            ev_b[i].record()
            fd.fd_combine(problem, p, lens_dev, ws, out, lse)
        torch.cuda.synchronize()
    partial_ms = [ev_a[i].elapsed_time(ev_b[i]) for i in timed]
    partial_mean = statistics.fmean(partial_ms)
    pq = statistics.quantiles(partial_ms, n=10)  # deciles: pq[0] = p10, pq[-1] = p90
    log(f"{K} steps: {ms_per_step * 1e3:.1f} us/step (events), wall {wall / K * 1e6:.1f} us/step; "
        f"partial kernel mean {partial_mean * 1e3:.1f} us, median {statistics.median(partial_ms) * 1e3:.1f} us, "
        f"p10 {pq[0] * 1e3:.1f}, p90 {pq[-1] * 1e3:.1f}")

    # Cold caches: a 1 GiB write between steps (outside the timed pair) evicts
    # the K/V from the L2s and the 256 MB Infinity Cache before each partial.
    scratch = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev)
    n_cold = min(K, 20)
    ca = [torch.cuda.Event(enable_timing=True) for _ in range(n_cold)]
    cb = [torch.cuda.Event(enable_timing=True) for _ in range(n_cold)]
    for i in range(n_cold):
        scratch.fill_(float(i))
        p = fd.fd_plan_splits(problem, lens_host, 0, wl.force_num_splits)
        ca[i].record()
        fd.fd_decode_partial(problem, p, q, k, v, bt, lens_dev, ws, None, ks, vs)
        cb[i].record()
        fd.fd_combine(problem, p, lens_dev, ws, out, lse)
    torch.cuda.synchronize()
    cold_ms = [a.elapsed_time(b) for a, b in zip(ca, cb)]
    del scratch
    cold_mean = statistics.fmean(cold_ms)
    log(f"cold-cache partial kernel mean {cold_mean * 1e3:.1f} us over {len(cold_ms)} steps")

    # What the memory delivers on the same buffers: the best of a plain
    # streaming read and the decode kernels' row pattern (K and V read
    # together, 1 KB of a token row per wave instruction), for context.
    sink = torch.empty(fd.PROBE_SINK_FLOATS, dtype=torch.float32, device=dev)
    probes = probe_patterns(fd, k, v, sink, wl.num_kv_heads * wl.head_dim * k.element_size())
    probe_name, probe_gbps = max(probes.items(), key=lambda kv: kv[1])
    log("read probes over K and V: " + ", ".join(f"{n} {g:.0f} GB/s" for n, g in probes.items()))
    # A plain copy of known size: its HBM counter readings calibrate the
    # FETCH_SIZE / WRITE_SIZE counters taken on the decode kernels.
    copy_bytes = 256 << 20
    src = torch.empty(copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    fd.fd_probe_copy(dst, src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * copy_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    log(f"calibration copy of {copy_bytes >> 20} MiB: {copy_gbps:.0f} GB/s (read + write)")
    del src, dst

    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (partial_mean * 1e-3) / 1e9
    # Below LAUNCH_BOUND_BYTES of K/V a launch ends before streaming reaches
    # its rate, for the probes too: their ratio then means nothing.
    launch_bound = nbytes < LAUNCH_BOUND_BYTES
    workload = wl.name
    traffic = measured_traffic(workload)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8_e4m3"}[wl.kv_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V; no dataset involved)",
        "config": {
            "workload": workload,
            "batch": wl.batch, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim, "q_len": wl.q_len, "seq_lens_total": wl.total_tokens,
            "page_size": wl.page_size,
            "accumulate": "f32", "out_dtype": "f32",
            "chunk_tokens": plan.chunk_tokens, "splits": plan.max_splits, "total_splits": plan.total_splits,
            "split_mode": plan.split_mode,
            "kv_bytes_per_call": nbytes,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "partial",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "partial_us_mean": round(partial_mean * 1e3, 2),
            "partial_timing": "every 8th step of the timed region" if in_loop else
                              "every partial launch of a second pass of the same steps after the timed region",
            "partial_us_median": round(statistics.median(partial_ms) * 1e3, 2),
            "partial_us_p10": round(pq[0] * 1e3, 2),
            "partial_us_p90": round(pq[-1] * 1e3, 2),
            "cold_partial_us_mean": round(cold_mean * 1e3, 2),
            "cold_achieved": round(nbytes / (cold_mean * 1e-3) / 1e9, 1),
            "hbm_read_probe_gbps": round(probe_gbps, 1),
            "hbm_read_probe_pattern": probe_name,
            "frac_of_probe": None if launch_bound else round(achieved / probe_gbps, 4),
            "launch_bound": launch_bound,
        },
    }
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for about {args.cpu_budget:.0f} s ...")
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget, out, lse)
    else:
        rec["cpu_baseline"] = None
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
