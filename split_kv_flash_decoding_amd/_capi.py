"""ctypes binding of include/fd.h.

Argument marshalling only: every step of decode attention runs in the HIP
library. PyTorch provides device memory and the stream handle. The library
must be built (``python -m split_kv_flash_decoding_amd.build``); if it is
missing, loading raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# FD_LIBRARY names another build of the library to load instead (an
# experiment with different compile-time settings).
LIB_PATH = os.environ.get("FD_LIBRARY") or os.path.join(HERE, "libfd.so")

FD_OK, FD_ERR_INVALID_ARGUMENT, FD_ERR_UNSUPPORTED, FD_ERR_WORKSPACE_TOO_SMALL, FD_ERR_HIP = range(5)
FD_F16, FD_BF16, FD_F32, FD_FP8_E4M3 = range(4)
FD_ROPE_NONE, FD_ROPE_INTERLEAVED, FD_ROPE_HALF = range(3)
ROPE_STYLES = {None: FD_ROPE_NONE, "none": FD_ROPE_NONE, "interleaved": FD_ROPE_INTERLEAVED, "half": FD_ROPE_HALF}

# Every function fd.h declares; the CPU tests check the library exports them.
EXPORTED = (
    "fd_plan_splits",
    "fd_decode_partial",
    "fd_decode_partial_scaled",
    "fd_combine",
    "fd_decode_attention",
    "fd_decode_attention_scaled",
    "fd_decode_attention_noalloc",
    "fd_append_kv",
    "fd_prefill_attention",
    "fd_decode_fused",
    "fd_workspace_init",
    "fd_status_string",
    "fd_last_error_message",
    "fd_probe_read",
    "fd_probe_read_rows",
    "fd_probe_copy",
)
PROBE_SINK_FLOATS = 4096


class FdProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
    ]

    @property
    def rows(self) -> int:
        """Query rows per sequence: q_len * Hq."""
        return max(1, self.q_len) * self.num_q_heads


class FdPlan(ctypes.Structure):
    _fields_ = [
        ("chunk_tokens", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("total_splits", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("partial_kernel", ctypes.c_int32),
        ("split_mode", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_uint64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class FdError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{status_string(status)}: {message}")


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libfd.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m split_kv_flash_decoding_amd.build`")
    lib = ctypes.CDLL(p)
    P, Pl = ctypes.POINTER(FdProblem), ctypes.POINTER(FdPlan)
    vp, i32p, f32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p
    lib.fd_plan_splits.argtypes = [P, i32p, ctypes.c_int32, ctypes.c_int32, Pl]
    lib.fd_decode_partial.argtypes = [P, Pl, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fd_combine.argtypes = [P, Pl, vp, vp, ctypes.c_size_t, vp, f32p, vp]
    lib.fd_decode_attention.argtypes = [P, vp, vp, vp, vp, i32p, vp, vp, f32p, vp, ctypes.c_size_t, vp]
    lib.fd_decode_partial_scaled.argtypes = [P, Pl, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fd_decode_attention_scaled.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, vp, vp, f32p, vp,
                                               ctypes.c_size_t, vp]
    lib.fd_decode_attention_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, vp, vp, f32p, vp]
    lib.fd_append_kv.argtypes = [P, ctypes.c_int32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                 vp, vp, vp]
    lib.fd_prefill_attention.argtypes = [P, vp, vp, vp, vp, vp, vp, f32p, vp]
    lib.fd_decode_fused.argtypes = [P, Pl, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, f32p, vp]
    lib.fd_workspace_init.argtypes = [P, Pl, vp, ctypes.c_size_t, vp]
    for name in ("fd_plan_splits", "fd_decode_partial", "fd_combine", "fd_decode_attention",
                 "fd_decode_partial_scaled", "fd_decode_attention_scaled", "fd_decode_attention_noalloc",
                 "fd_append_kv", "fd_prefill_attention",
                 "fd_decode_fused", "fd_workspace_init"):
        getattr(lib, name).restype = ctypes.c_int
    lib.fd_status_string.argtypes = [ctypes.c_int]
    lib.fd_status_string.restype = ctypes.c_char_p
    lib.fd_last_error_message.argtypes = []
    lib.fd_last_error_message.restype = ctypes.c_char_p
    lib.fd_probe_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.fd_probe_read.restype = ctypes.c_int
    lib.fd_probe_read_rows.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, vp, vp]
    lib.fd_probe_read_rows.restype = ctypes.c_int
    lib.fd_probe_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.fd_probe_copy.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fd_status_string(status).decode()


def _check(status: int) -> None:
    if status != FD_OK:
        raise FdError(status, load_library().fd_last_error_message().decode())


# ------------------------------------------------------------------ problems


def _dtype_code(dt) -> int:
    import torch

    table = {torch.float16: FD_F16, torch.bfloat16: FD_BF16, torch.float32: FD_F32,
             torch.float8_e4m3fn: FD_FP8_E4M3}
    if dt not in table:
        raise ValueError(f"unsupported dtype {dt}")
    return table[dt]


def make_problem(*, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, kv_dtype,
                 out_dtype=None, scale: Optional[float] = None, page_size: int = 0,
                 max_pages_per_seq: int = 0, q_len: int = 1, q_dtype=None, num_pages: int = 0) -> FdProblem:
    """``kv_dtype``: the cache's torch dtype (float16, bfloat16 or
    float8_e4m3fn); ``q_dtype``: q's dtype for an FP8 cache (default
    float16)."""
    import torch

    return FdProblem(
        batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        kv_dtype=_dtype_code(kv_dtype), out_dtype=_dtype_code(out_dtype or torch.float32),
        scale=0.0 if scale is None else float(scale), page_size=page_size,
        max_pages_per_seq=max_pages_per_seq, q_len=q_len,
        q_dtype=_dtype_code(q_dtype or torch.float16) if kv_dtype == torch.float8_e4m3fn else 0,
        num_pages=num_pages)


def _q_shape(problem: FdProblem, d: int):
    B, hq = problem.batch, problem.num_q_heads
    return (B, hq, d) if problem.q_len <= 1 else (B, problem.q_len, hq, d)


def _q_shapes(problem: FdProblem, d: int):
    """Accepted q / out shapes: [B, Hq, d] or [B, 1, Hq, d] for one query token."""
    B, hq = problem.batch, problem.num_q_heads
    return {_q_shape(problem, d), (B, max(1, problem.q_len), hq, d)}


def _lens_array(seq_lens_host: Sequence[int]):
    vals = [int(x) for x in (seq_lens_host.tolist() if hasattr(seq_lens_host, "tolist") else seq_lens_host)]
    return (ctypes.c_int32 * len(vals))(*vals), vals


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_tensors(problem: FdProblem, q, k, v, block_table, seq_lens_dev, total_tokens: Optional[int]):
    import torch

    B, hq, hkv, d = problem.batch, problem.num_q_heads, problem.num_kv_heads, problem.head_dim
    types = {FD_F16: torch.float16, FD_BF16: torch.bfloat16, FD_FP8_E4M3: torch.float8_e4m3fn}
    kvdt = types.get(problem.kv_dtype)
    qdt = types.get(problem.q_dtype if problem.kv_dtype == FD_FP8_E4M3 else problem.kv_dtype)
    for name, t, dt in (("q", q, qdt), ("k", k, kvdt), ("v", v, kvdt)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt:
            raise ValueError(f"{name} must be a contiguous {dt} CUDA tensor")
    if tuple(q.shape) not in _q_shapes(problem, d):
        raise ValueError(f"q has shape {tuple(q.shape)}, expected {_q_shape(problem, d)}")
    if k.shape != v.shape:
        raise ValueError("k and v shapes differ")
    if problem.page_size:
        if k.dim() != 4 or tuple(k.shape[1:]) != (problem.page_size, hkv, d):
            raise ValueError(f"paged k must be [P, {problem.page_size}, {hkv}, {d}]")
        if block_table is None or block_table.dtype != torch.int32 or not block_table.is_cuda \
                or tuple(block_table.shape) != (B, problem.max_pages_per_seq) or not block_table.is_contiguous():
            raise ValueError(f"block_table must be a contiguous int32 CUDA tensor [{B}, {problem.max_pages_per_seq}]")
    else:
        if k.dim() != 3 or tuple(k.shape[1:]) != (hkv, d):
            raise ValueError(f"contiguous k must be [rows, {hkv}, {d}]")
        if total_tokens is not None and k.shape[0] < total_tokens:
            raise ValueError(f"k holds {k.shape[0]} rows, the lengths need {total_tokens}")
    if seq_lens_dev.dtype != torch.int32 or not seq_lens_dev.is_cuda or seq_lens_dev.numel() != B:
        raise ValueError("seq_lens_dev must be an int32 CUDA tensor with one entry per sequence")


# ------------------------------------------------------------------ the calls


def fd_plan_splits(problem: FdProblem, seq_lens_host, num_cus: int = 0, force_num_splits: int = 0) -> FdPlan:
    lib = load_library()
    arr, _ = _lens_array(seq_lens_host)
    plan = FdPlan()
    _check(lib.fd_plan_splits(ctypes.byref(problem), arr, num_cus, force_num_splits, ctypes.byref(plan)))
    return plan


def _with_pool(problem: FdProblem, k) -> FdProblem:
    """The problem with the pool size of a paged cache filled in from k, so
    the kernels check every page index against it."""
    if problem.page_size and problem.num_pages == 0:
        p = FdProblem.from_buffer_copy(problem)
        p.num_pages = int(k.shape[0])
        return p
    return problem


def _check_scales(problem: FdProblem, k_scale, v_scale) -> None:
    import torch

    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t is not None and (not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous()
                              or t.numel() != problem.num_kv_heads):
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor with one entry per KV head")


def fd_decode_partial(problem: FdProblem, plan: FdPlan, q, k, v, block_table, seq_lens_dev, workspace,
                      stream=None, k_scale=None, v_scale=None) -> None:
    """fd_decode_partial, or fd_decode_partial_scaled when the cache is FP8 or
    scales are given."""
    _check_tensors(problem, q, k, v, block_table, seq_lens_dev, plan.total_tokens)
    problem = _with_pool(problem, k)
    lib = load_library()
    if problem.kv_dtype == FD_FP8_E4M3 or k_scale is not None or v_scale is not None:
        _check_scales(problem, k_scale, v_scale)
        _check(lib.fd_decode_partial_scaled(
            ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
            _ptr(block_table), _ptr(seq_lens_dev), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream)))
        return
    _check(lib.fd_decode_partial(
        ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v), _ptr(block_table),
        _ptr(seq_lens_dev), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def fd_workspace_init(problem: FdProblem, plan: FdPlan, workspace, stream=None) -> None:
    """Zero the fused merge's arrival counters (once per workspace)."""
    _check(load_library().fd_workspace_init(ctypes.byref(problem), ctypes.byref(plan), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(stream)))


def fd_decode_fused(problem: FdProblem, plan: FdPlan, q, k, v, block_table, seq_lens_dev, workspace, out, lse=None,
                    stream=None, k_scale=None, v_scale=None) -> None:
    """Partials and merge in one launch (include/fd.h); the workspace's
    counters must have been zeroed once with fd_workspace_init."""
    _check_tensors(problem, q, k, v, block_table, seq_lens_dev, plan.total_tokens)
    _check_out(problem, out, lse)
    _check_scales(problem, k_scale, v_scale)
    problem = _with_pool(problem, k)
    _check(load_library().fd_decode_fused(
        ctypes.byref(problem), ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), _ptr(seq_lens_dev), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(out), _ptr(lse), _stream(stream)))


def _check_out(problem: FdProblem, out, lse) -> None:
    oshape = tuple(out.shape) if tuple(out.shape) in _q_shapes(problem, problem.head_dim) else \
        _q_shape(problem, problem.head_dim)
    if tuple(out.shape) != oshape or not out.is_contiguous() or _dtype_code(out.dtype) != problem.out_dtype \
            or not out.is_cuda:
        raise ValueError(f"out must be a contiguous CUDA tensor {list(oshape)} of the problem's out_dtype")
    if lse is not None and (tuple(lse.shape) != oshape[:-1] or not lse.is_contiguous()
                            or _dtype_code(lse.dtype) != FD_F32 or not lse.is_cuda):
        raise ValueError(f"lse must be a contiguous float32 CUDA tensor {list(oshape[:-1])}")


def fd_combine(problem: FdProblem, plan: FdPlan, seq_lens_dev, workspace, out, lse=None, stream=None) -> None:
    _check_out(problem, out, lse)
    _check(load_library().fd_combine(
        ctypes.byref(problem), ctypes.byref(plan), _ptr(seq_lens_dev), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


def fd_decode_attention(problem: FdProblem, q, k, v, block_table, seq_lens_host, seq_lens_dev, out, lse,
                        workspace, stream=None, k_scale=None, v_scale=None) -> None:
    """fd_decode_attention, or fd_decode_attention_scaled when the cache is
    FP8 or scales are given."""
    arr, vals = _lens_array(seq_lens_host)
    _check_tensors(problem, q, k, v, block_table, seq_lens_dev, sum(vals))
    _check_out(problem, out, lse)
    problem = _with_pool(problem, k)
    lib = load_library()
    if problem.kv_dtype == FD_FP8_E4M3 or k_scale is not None or v_scale is not None:
        _check_scales(problem, k_scale, v_scale)
        _check(lib.fd_decode_attention_scaled(
            ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
            arr, _ptr(seq_lens_dev), _ptr(out), _ptr(lse), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)))
        return
    _check(lib.fd_decode_attention(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), arr, _ptr(seq_lens_dev),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def bind_decode_attention(problem: FdProblem, q, k, v, block_table, seq_lens_host, seq_lens_dev, out, lse,
                          workspace, stream=None, k_scale=None, v_scale=None, num_splits: int = 0):
    """fd_decode_attention (or its _scaled form) with every argument checked
    and converted once: returns a callable that makes the one C call (plan,
    partial kernel, combine) on the same buffers each time it is called,
    for loops that repeat a step on resident data. The lengths are copied
    now; the tensors must stay alive and unchanged in shape. With
    num_splits > 0 (a forced split count, which the one-shot call does not
    take) the callable makes the three C calls fd_plan_splits,
    fd_decode_partial[_scaled] and fd_combine instead, with the same
    once-converted arguments."""
    arr, vals = _lens_array(seq_lens_host)
    _check_tensors(problem, q, k, v, block_table, seq_lens_dev, sum(vals))
    _check_out(problem, out, lse)
    problem = FdProblem.from_buffer_copy(_with_pool(problem, k))
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _stream(stream)
    pp = ctypes.byref(problem)
    scaled = problem.kv_dtype == FD_FP8_E4M3 or k_scale is not None or v_scale is not None
    if scaled:
        _check_scales(problem, k_scale, v_scale)
    if num_splits > 0:
        plan = FdPlan()
        pl = ctypes.byref(plan)
        plan_args = (pp, arr, 0, int(num_splits), pl)
        if scaled:
            part_fn = lib.fd_decode_partial_scaled
            part_args = (pp, pl, _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                         _ptr(seq_lens_dev), _ptr(workspace), ws_bytes, st)
        else:
            part_fn = lib.fd_decode_partial
            part_args = (pp, pl, _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), _ptr(seq_lens_dev), _ptr(workspace),
                         ws_bytes, st)
        comb_args = (pp, pl, _ptr(seq_lens_dev), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), st)

        def run_split() -> None:
            for fn, args in ((lib.fd_plan_splits, plan_args), (part_fn, part_args), (lib.fd_combine, comb_args)):
                status = fn(*args)
                if status:
                    _check(status)

        run_split.keep = (problem, plan, arr, q, k, v, block_table, seq_lens_dev, out, lse, workspace, k_scale,
                          v_scale)
        return run_split
    if scaled:
        fn = lib.fd_decode_attention_scaled
        args = (pp, _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), arr,
                _ptr(seq_lens_dev), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, st)
    else:
        fn = lib.fd_decode_attention
        args = (pp, _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), arr, _ptr(seq_lens_dev), _ptr(out), _ptr(lse),
                _ptr(workspace), ws_bytes, st)

    def run() -> None:
        status = fn(*args)
        if status:
            _check(status)

    run.keep = (problem, arr, q, k, v, block_table, seq_lens_dev, out, lse, workspace, k_scale, v_scale)
    return run


NOALLOC_WORKSPACE_BYTES = 64 << 20  # FD_NOALLOC_WORKSPACE_BYTES


def fd_decode_attention_noalloc(problem: FdProblem, q, k, v, block_table, seq_lens_host, seq_lens_dev, out, lse,
                                stream=None, k_scale=None, v_scale=None) -> None:
    """fd_decode_attention_noalloc: plan, partials and merge with the partials
    in the library's fixed per-GPU buffer (no workspace argument, nothing
    allocated). Calls that overlap on one GPU race on that buffer."""
    arr, vals = _lens_array(seq_lens_host)
    _check_tensors(problem, q, k, v, block_table, seq_lens_dev, sum(vals))
    _check_out(problem, out, lse)
    _check_scales(problem, k_scale, v_scale)
    problem = _with_pool(problem, k)
    _check(load_library().fd_decode_attention_noalloc(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), arr,
        _ptr(seq_lens_dev), _ptr(out), _ptr(lse), _stream(stream)))


def fd_prefill_attention(problem: FdProblem, q, k, v, block_table, seq_lens_dev, out, lse=None,
                         stream=None) -> None:
    """Causal attention of every sequence's q_len query tokens over its cache
    in one pass (include/fd.h). q and out are [B, q_len, Hq, d]."""
    _check_tensors(problem, q, k, v, block_table, seq_lens_dev, None)
    _check_out(problem, out, lse)
    problem = _with_pool(problem, k)
    _check(load_library().fd_prefill_attention(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(block_table), _ptr(seq_lens_dev), _ptr(out),
        _ptr(lse), _stream(stream)))


def prefill_attention(q, k, v, seq_lens, *, block_table=None, page_size: int = 0, max_pages_per_seq: int = 0,
                      scale: Optional[float] = None, out_dtype=None, stream=None):
    """fd_prefill_attention with out and lse allocated by torch on q's device;
    q is [B, q_len, Hq, d]. Returns (out, lse)."""
    import torch

    B, q_len, hq, d = q.shape
    problem = make_problem(batch=B, num_q_heads=hq, num_kv_heads=k.shape[-2], head_dim=d, kv_dtype=k.dtype,
                           out_dtype=out_dtype or torch.float32, scale=scale, page_size=page_size,
                           max_pages_per_seq=max_pages_per_seq or (block_table.shape[1] if block_table is not None else 0),
                           q_len=q_len)
    lens_dev = seq_lens if (hasattr(seq_lens, "is_cuda") and seq_lens.is_cuda) else \
        torch.tensor(list(seq_lens.tolist() if hasattr(seq_lens, "tolist") else seq_lens), dtype=torch.int32,
                     device=q.device)
    out = torch.empty(tuple(q.shape), dtype=out_dtype or torch.float32, device=q.device)
    lse = torch.empty(tuple(q.shape[:-1]), dtype=torch.float32, device=q.device)
    fd_prefill_attention(problem, q, k, v, block_table, lens_dev, out, lse, stream)
    return out, lse


def fd_append_kv(problem: FdProblem, k_new, v_new, q, k_cache, v_cache, block_table, seq_lens_dev, *,
                 rope_style=None, rope_base: float = 10000.0, k_scale=None, v_scale=None, stream=None) -> None:
    """Write each sequence's q_len new tokens into the paged cache, keys and
    (optionally) q rotated in place by RoPE at their positions (include/fd.h).
    seq_lens_dev holds the lengths after the append."""
    import torch

    types = {FD_F16: torch.float16, FD_BF16: torch.bfloat16, FD_FP8_E4M3: torch.float8_e4m3fn}
    B, hq, hkv, d = problem.batch, problem.num_q_heads, problem.num_kv_heads, problem.head_dim
    n = max(1, problem.q_len)
    qdt = types.get(problem.q_dtype if problem.kv_dtype == FD_FP8_E4M3 else problem.kv_dtype)
    kvdt = types.get(problem.kv_dtype)
    for name, t, shape, dt in (("k_new", k_new, (B, n, hkv, d), qdt), ("v_new", v_new, (B, n, hkv, d), qdt),
                               ("q", q, (B, n, hq, d), qdt)):
        if t is None and name == "q":
            continue
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt or t.numel() != math.prod(shape):
            raise ValueError(f"{name} must be a contiguous {dt} CUDA tensor of {list(shape)} elements")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != kvdt or t.dim() != 4 \
                or tuple(t.shape[1:]) != (problem.page_size, hkv, d):
            raise ValueError(f"{name} must be a contiguous {kvdt} CUDA pool [P, {problem.page_size}, {hkv}, {d}]")
    if block_table is None or block_table.dtype != torch.int32 or not block_table.is_cuda \
            or tuple(block_table.shape) != (B, problem.max_pages_per_seq) or not block_table.is_contiguous():
        raise ValueError(f"block_table must be a contiguous int32 CUDA tensor [{B}, {problem.max_pages_per_seq}]")
    if seq_lens_dev.dtype != torch.int32 or not seq_lens_dev.is_cuda or seq_lens_dev.numel() != B:
        raise ValueError("seq_lens_dev must be an int32 CUDA tensor with one entry per sequence")
    _check_scales(problem, k_scale, v_scale)
    _check(load_library().fd_append_kv(
        ctypes.byref(problem), ROPE_STYLES[rope_style], float(rope_base), _ptr(k_new), _ptr(v_new), _ptr(q),
        _ptr(k_scale), _ptr(v_scale), _ptr(k_cache), _ptr(v_cache), int(k_cache.shape[0]), _ptr(block_table),
        _ptr(seq_lens_dev), _stream(stream)))


# --------------------------------------------------------------- convenience


@dataclass
class DecodeResult:
    out: object
    lse: object
    plan: FdPlan
    workspace: object


def workspace_views(problem: FdProblem, plan: FdPlan, workspace):
    """(O [B,R,S,d], m [B,R,S], l [B,R,S]) float32 views of a workspace, R =
    q_len * Hq query rows (row i * Hq + h for query token i, head h)."""
    B, hq, d, S = problem.batch, problem.rows, problem.head_dim, plan.max_splits
    n_o = B * hq * S * d
    flat = workspace.view(-1)[: n_o + B * hq * S * 2]
    O = flat[:n_o].view(B, hq, S, d)
    ml = flat[n_o:].view(B, hq, S, 2)
    return O, ml[..., 0], ml[..., 1]


def decode_attention(q, k, v, seq_lens, *, block_table=None, page_size: int = 0, max_pages_per_seq: int = 0,
                     scale: Optional[float] = None, out_dtype=None, num_splits: int = 0, num_cus: int = 0,
                     stream=None, k_scale=None, v_scale=None) -> DecodeResult:
    """Plan, partials and merge for one batch; allocates out, lse and the
    workspace with torch on q's device. ``seq_lens`` may be a CPU tensor or
    list. q is [B, Hq, d], or [B, q_len, Hq, d] for several query tokens per
    sequence (the last q_len tokens of each cache, causal among themselves).
    k and v may be float8_e4m3fn codes with per-KV-head ``k_scale`` /
    ``v_scale`` (float32 CUDA tensors [Hkv])."""
    import torch

    if q.dim() == 4:
        B, q_len, hq, d = q.shape
    else:
        (B, hq, d), q_len = q.shape, 1
    hkv = k.shape[-2]
    problem = make_problem(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, kv_dtype=k.dtype, q_dtype=q.dtype,
                           out_dtype=out_dtype or torch.float32, scale=scale, page_size=page_size,
                           max_pages_per_seq=max_pages_per_seq or (block_table.shape[1] if block_table is not None else 0),
                           q_len=q_len)
    lens_host = seq_lens.tolist() if hasattr(seq_lens, "tolist") else list(seq_lens)
    plan = fd_plan_splits(problem, lens_host, num_cus=num_cus, force_num_splits=num_splits)
    if block_table is not None:
        # The kernels trust page indices; check the ones they will read (this synchronises).
        num_pages = k.shape[0]
        for b, n in enumerate(lens_host):
            used = block_table[b, : -(-int(n) // page_size)]
            lo, hi = int(used.min()), int(used.max())
            if lo < 0 or hi >= num_pages:
                raise ValueError(f"block_table row {b} names page {lo if lo < 0 else hi} outside [0, {num_pages})")
    dev = q.device
    lens_dev = torch.tensor(lens_host, dtype=torch.int32, device=dev)
    ws = torch.empty(int(math.ceil(plan.workspace_bytes / 4)), dtype=torch.float32, device=dev)
    oshape = _q_shape(problem, d)
    out = torch.empty(oshape, dtype=out_dtype or torch.float32, device=dev)
    lse = torch.empty(oshape[:-1], dtype=torch.float32, device=dev)
    fd_decode_partial(problem, plan, q, k, v, block_table, lens_dev, ws, stream, k_scale, v_scale)
    fd_combine(problem, plan, lens_dev, ws, out, lse, stream)
    return DecodeResult(out=out, lse=lse, plan=plan, workspace=ws)


# ------------------------------------------------------------------- probes


def fd_probe_read(src, sink, stream=None) -> None:
    """Stream every byte of the CUDA tensor ``src`` once (include/fd_probe.h)."""
    if not src.is_cuda or not sink.is_cuda or sink.numel() * sink.element_size() < PROBE_SINK_FLOATS * 4:
        raise ValueError("src and sink must be CUDA tensors; sink holds PROBE_SINK_FLOATS floats")
    _check(load_library().fd_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))


def fd_probe_read_rows(a, b, row_bytes: int, chunk_rows: int, waves_across, sink, stream=None) -> None:
    """Read the CUDA tensors ``a`` and ``b`` (the same byte size, a whole
    number of ``row_bytes`` rows) in the decode kernels' row pattern
    (include/fd_probe.h): 1 KB column blocks with the eight waves splitting
    the rows (``waves_across`` 0 or False; 2: each chunk from a rotated start,
    as the head-rows kernel walks a 16-bit cache), or 8 KB blocks with wave w
    reading column w (1 or True)."""
    nbytes = a.numel() * a.element_size()
    if not a.is_cuda or not b.is_cuda or b.numel() * b.element_size() != nbytes or nbytes % row_bytes:
        raise ValueError("a and b must be CUDA tensors of one size, a whole number of rows")
    if not sink.is_cuda or sink.numel() * sink.element_size() < PROBE_SINK_FLOATS * 4:
        raise ValueError("sink must be a CUDA tensor of PROBE_SINK_FLOATS floats")
    _check(load_library().fd_probe_read_rows(_ptr(a), _ptr(b), nbytes // row_bytes, row_bytes,
                                             8192 if int(waves_across) == 1 else 1024, chunk_rows, int(waves_across),
                                             _ptr(sink), _stream(stream)))


def fd_probe_copy(dst, src, stream=None) -> None:
    """Copy the CUDA tensor ``src`` into ``dst`` (same byte size)."""
    nbytes = src.numel() * src.element_size()
    if not src.is_cuda or not dst.is_cuda or dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src must be CUDA tensors of equal byte size")
    _check(load_library().fd_probe_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))
