"""Split-KV flash decoding on AMD Instinct MI355X (gfx950).

The computation runs in ``libfd.so`` (HIP kernels behind the C ABI in
``include/fd.h``); this package is its ctypes binding. Functions carry the C
names: ``fd_plan_splits``, ``fd_decode_partial``, ``fd_combine`` and
``fd_decode_attention``; ``decode_attention`` is a convenience wrapper that
allocates the outputs and the workspace with torch.
"""

from ._capi import (  # noqa: F401
    EXPORTED,
    FD_BF16,
    FD_ERR_HIP,
    FD_ERR_INVALID_ARGUMENT,
    FD_ERR_UNSUPPORTED,
    FD_ERR_WORKSPACE_TOO_SMALL,
    FD_F16,
    FD_F32,
    FD_FP8_E4M3,
    FD_OK,
    LIB_PATH,
    NOALLOC_WORKSPACE_BYTES,
    PROBE_SINK_FLOATS,
    DecodeResult,
    FdError,
    FdPlan,
    FdProblem,
    bind_decode_attention,
    decode_attention,
    FD_ROPE_HALF,
    FD_ROPE_INTERLEAVED,
    FD_ROPE_NONE,
    fd_append_kv,
    fd_combine,
    fd_decode_attention,
    fd_decode_attention_noalloc,
    fd_decode_fused,
    fd_decode_partial,
    fd_plan_splits,
    fd_prefill_attention,
    prefill_attention,
    fd_probe_copy,
    fd_probe_read,
    fd_probe_read_rows,
    fd_workspace_init,
    load_library,
    make_problem,
    status_string,
    workspace_views,
)
