// The C-ABI entry points that launch work (fd_decode_partial[_scaled],
// fd_combine, fd_decode_attention[_scaled]) and the compute-unit query the
// planner uses. Argument checks run on the host before anything is enqueued.

#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>

#include "fd_device.h"

namespace fd {

fd_status query_num_cus(int32_t* out) {
    // One slot per device, read and written atomically: host threads that
    // plan at the same time may both query the device on first use, and both
    // store the same count.
    static std::atomic<int32_t> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    const bool cached = dev >= 0 && dev < 64;
    if (cached) {
        const int32_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return FD_OK;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0)
        return fail(FD_ERR_HIP, "compute-unit query failed: %s", hipGetErrorString(e));
    if (cached) cache[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return FD_OK;
}

namespace {

// Partials, and with `out` non-NULL the fused merge as well.
fd_status decode_partial(const fd_problem* p, const fd_plan* plan, const void* q, const void* k, const void* v,
                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                         const int32_t* seq_lens_dev, void* workspace, size_t workspace_bytes_avail, void* stream,
                         void* out = nullptr, float* lse = nullptr) {
    float scale = 0.f;
    fd_status st = check_problem(p, &scale);
    if (st != FD_OK) return st;
    st = check_plan(p, plan);
    if (st != FD_OK) return st;
    if (!q || !k || !v || !seq_lens_dev || !workspace)
        return fail(FD_ERR_INVALID_ARGUMENT, "q, k, v, seq_lens_dev and workspace must be non-NULL");
    if (p->page_size && !block_table)
        return fail(FD_ERR_INVALID_ARGUMENT, "paged cache needs a block table");
    if (workspace_bytes_avail < workspace_bytes(p, plan->max_splits))
        return fail(FD_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, the plan needs %llu",
                    workspace_bytes_avail, (unsigned long long)workspace_bytes(p, plan->max_splits));
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
        return fail(FD_ERR_INVALID_ARGUMENT, "q, k and v must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(workspace) & 15)
        return fail(FD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3)
        return fail(FD_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be 4-byte aligned");

    fdk::PartialArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = k;
    a.v = v;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.kv_dt = p->kv_dtype;
    a.q_dt = q_dtype_of(p);
    a.table = block_table;
    a.lens = seq_lens_dev;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + workspace_o_bytes(p, plan->max_splits));
    a.batch = p->batch;
    a.hq = p->num_q_heads;
    a.hkv = p->num_kv_heads;
    a.chunk = plan->chunk_tokens;
    a.s_max = plan->max_splits;
    a.split_mode = plan->split_mode;
    a.max_pages = p->page_size ? p->max_pages_per_seq : 0;
    a.q_len = problem_q_len(p);
    a.qk_scale_log2 = scale * fdk::kLog2e;
    a.num_pages = p->page_size ? p->num_pages : 0;
    a.counters = out ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                                   workspace_counters_offset(p, plan->max_splits))
                     : nullptr;
    a.out = out;
    a.lse = lse;
    a.out_dt = p->out_dtype;

    // One work-group per (split, KV head group) of the work list (see
    // locate_unit), times the matrix-core kernel's column tiles (the grid is
    // then padded to whole groups of 8 entries; the padding exits at once).
    const int32_t groups = p->num_kv_heads / heads_per_workgroup(p, plan->partial_kernel);
    const int32_t tiles = plan->partial_kernel == kPartialMfma ? mfma_column_tiles(p) : 1;
    int64_t units = (int64_t)plan->total_splits * groups;
    if (tiles > 1) units = (units + 7) / 8 * 8 * tiles;
    if (plan->total_splits < 1 || units > INT32_MAX)
        return fail(FD_ERR_INVALID_ARGUMENT, "plan has %d splits (x %d head groups)", plan->total_splits, groups);
    dim3 grid((uint32_t)units);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int G = p->num_q_heads / p->num_kv_heads;
    const bool paged = p->page_size != 0;
    hipError_t e;
    switch (plan->partial_kernel) {
        case kPartialMfma: e = fdk::launch_partial_mfma(G, paged, a, grid, hs); break;
        case kPartialMfmaHeads: e = fdk::launch_partial_mfma_heads(G, paged, a, grid, hs); break;
        case kPartialHeadRows: e = fdk::launch_partial_valu_heads(p->head_dim, G, paged, a, grid, hs); break;
        case kPartialHeadCols: e = fdk::launch_partial_valu_head_cols(p->head_dim, G, paged, a, grid, hs); break;
        default: e = fdk::launch_partial_valu(p->head_dim, G, paged, a, grid, hs); break;
    }
    if (e != hipSuccess) return fail(FD_ERR_HIP, "partial kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

__global__ void zero_u32(uint32_t* p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// The partials of fd_decode_attention_noalloc: one copy per GPU, set aside
// when the library's code is loaded on that device and held until the
// process ends. Host code never uses this name as an address (on the host it
// stands for the variable, not its device memory); scratch_address looks the
// device address up.
static __device__ __align__(256) uint8_t scratch[FD_NOALLOC_WORKSPACE_BYTES];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

fd_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(FD_ERR_UNSUPPORTED, "device %d: the allocation-free call serves devices 0-63", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(FD_ERR_HIP, "address of the allocation-free workspace on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FD_OK;
}

fd_status reject_fp8(const fd_problem* p, const char* call) {
    if (p && p->kv_dtype == FD_FP8_E4M3)
        return fail(FD_ERR_INVALID_ARGUMENT, "an fp8 cache needs its scales: call %s_scaled", call);
    return FD_OK;
}

}  // namespace

}  // namespace fd

using namespace fd;

extern "C" {

fd_status fd_decode_partial(const fd_problem* p, const fd_plan* plan, const void* q, const void* k,
                            const void* v, const int32_t* block_table, const int32_t* seq_lens_dev,
                            void* workspace, size_t workspace_bytes_avail, void* stream) {
    clear_error();
    fd_status st = reject_fp8(p, "fd_decode_partial");
    if (st != FD_OK) return st;
    return decode_partial(p, plan, q, k, v, nullptr, nullptr, block_table, seq_lens_dev, workspace,
                          workspace_bytes_avail, stream);
}

fd_status fd_decode_partial_scaled(const fd_problem* p, const fd_plan* plan, const void* q, const void* k,
                                   const void* v, const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, const int32_t* seq_lens_dev, void* workspace,
                                   size_t workspace_bytes_avail, void* stream) {
    clear_error();
    return decode_partial(p, plan, q, k, v, k_scale, v_scale, block_table, seq_lens_dev, workspace,
                          workspace_bytes_avail, stream);
}

fd_status fd_workspace_init(const fd_problem* p, const fd_plan* plan, void* workspace, size_t workspace_bytes_avail,
                            void* stream) {
    clear_error();
    fd_status st = check_problem(p, nullptr);
    if (st != FD_OK) return st;
    st = check_plan(p, plan);
    if (st != FD_OK) return st;
    if (!workspace) return fail(FD_ERR_INVALID_ARGUMENT, "workspace must be non-NULL");
    if (workspace_bytes_avail < workspace_bytes(p, plan->max_splits))
        return fail(FD_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, the plan needs %llu",
                    workspace_bytes_avail, (unsigned long long)workspace_bytes(p, plan->max_splits));
    if (reinterpret_cast<uintptr_t>(workspace) & 15)
        return fail(FD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    // A kernel, not a memset: the call may be recorded in a graph.
    const int64_t n = (int64_t)p->batch * p->num_kv_heads;
    uint32_t* c = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + workspace_counters_offset(p, plan->max_splits));
    const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_u32, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), c, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FD_ERR_HIP, "workspace init launch: %s", hipGetErrorString(e));
    return FD_OK;
}

fd_status fd_decode_fused(const fd_problem* p, const fd_plan* plan, const void* q, const void* k, const void* v,
                          const float* k_scale, const float* v_scale, const int32_t* block_table,
                          const int32_t* seq_lens_dev, void* workspace, size_t workspace_bytes_avail, void* out,
                          float* lse, void* stream) {
    clear_error();
    if (!out) return fail(FD_ERR_INVALID_ARGUMENT, "out must be non-NULL");
    return decode_partial(p, plan, q, k, v, k_scale, v_scale, block_table, seq_lens_dev, workspace,
                          workspace_bytes_avail, stream, out, lse);
}

fd_status fd_combine(const fd_problem* p, const fd_plan* plan, const int32_t* seq_lens_dev,
                     const void* workspace, size_t workspace_bytes_avail, void* out, float* lse,
                     void* stream) {
    clear_error();
    fd_status st = check_problem(p, nullptr);
    if (st != FD_OK) return st;
    st = check_plan(p, plan);
    if (st != FD_OK) return st;
    if (!seq_lens_dev || !workspace || !out)
        return fail(FD_ERR_INVALID_ARGUMENT, "seq_lens_dev, workspace and out must be non-NULL");
    if (workspace_bytes_avail < workspace_bytes(p, plan->max_splits))
        return fail(FD_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, the plan needs %llu",
                    workspace_bytes_avail, (unsigned long long)workspace_bytes(p, plan->max_splits));
    const float* ws_o = static_cast<const float*>(workspace);
    const float* ws_ml =
        reinterpret_cast<const float*>(static_cast<const char*>(workspace) + workspace_o_bytes(p, plan->max_splits));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // The combine treats the q_len * Hq query rows of a sequence alike.
    hipError_t e = fdk::launch_combine(p->head_dim, p->out_dtype, ws_o, ws_ml, seq_lens_dev, out, lse, p->batch,
                                       problem_q_len(p) * p->num_q_heads, plan->chunk_tokens, plan->max_splits,
                                       plan->split_mode, p->page_size ? p->max_pages_per_seq * kPageSize : INT32_MAX,
                                       combine_form(p, plan->max_splits), hs);
    if (e != hipSuccess) return fail(FD_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

fd_status fd_decode_attention_scaled(const fd_problem* p, const void* q, const void* k, const void* v,
                                     const float* k_scale, const float* v_scale, const int32_t* block_table,
                                     const int32_t* seq_lens_host, const int32_t* seq_lens_dev, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes_avail, void* stream) {
    fd_plan plan;
    fd_status st = fd_plan_splits(p, seq_lens_host, 0, 0, &plan);
    if (st != FD_OK) return st;
    if (!out) return fail(FD_ERR_INVALID_ARGUMENT, "out must be non-NULL");
    if (workspace_bytes_avail < plan.workspace_bytes)
        return fail(FD_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, the plan needs %llu",
                    workspace_bytes_avail, (unsigned long long)plan.workspace_bytes);
    st = fd_decode_partial_scaled(p, &plan, q, k, v, k_scale, v_scale, block_table, seq_lens_dev, workspace,
                                  workspace_bytes_avail, stream);
    if (st != FD_OK) return st;
    return fd_combine(p, &plan, seq_lens_dev, workspace, workspace_bytes_avail, out, lse, stream);
}

fd_status fd_decode_attention(const fd_problem* p, const void* q, const void* k, const void* v,
                              const int32_t* block_table, const int32_t* seq_lens_host,
                              const int32_t* seq_lens_dev, void* out, float* lse, void* workspace,
                              size_t workspace_bytes_avail, void* stream) {
    clear_error();
    fd_status st = reject_fp8(p, "fd_decode_attention");
    if (st != FD_OK) return st;
    return fd_decode_attention_scaled(p, q, k, v, nullptr, nullptr, block_table, seq_lens_host, seq_lens_dev, out,
                                      lse, workspace, workspace_bytes_avail, stream);
}

fd_status fd_decode_attention_noalloc(const fd_problem* p, const void* q, const void* k, const void* v,
                                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                                      const int32_t* seq_lens_host, const int32_t* seq_lens_dev, void* out,
                                      float* lse, void* stream) {
    fd_plan plan;
    fd_status st = fd_plan_splits(p, seq_lens_host, 0, 0, &plan);
    if (st != FD_OK) return st;
    if (!out) return fail(FD_ERR_INVALID_ARGUMENT, "out must be non-NULL");
    if (plan.workspace_bytes > FD_NOALLOC_WORKSPACE_BYTES)
        return fail(FD_ERR_WORKSPACE_TOO_SMALL, "the plan needs %llu bytes of partials; the allocation-free call "
                    "holds %zu per GPU (use fd_decode_attention_scaled with a workspace)",
                    (unsigned long long)plan.workspace_bytes, FD_NOALLOC_WORKSPACE_BYTES);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != FD_OK) return st;
    st = fd_decode_partial_scaled(p, &plan, q, k, v, k_scale, v_scale, block_table, seq_lens_dev, ws,
                                  FD_NOALLOC_WORKSPACE_BYTES, stream);
    if (st != FD_OK) return st;
    return fd_combine(p, &plan, seq_lens_dev, ws, FD_NOALLOC_WORKSPACE_BYTES, out, lse, stream);
}

fd_status fd_prefill_attention(const fd_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* block_table, const int32_t* seq_lens_dev, void* out, float* lse,
                               void* stream) {
    clear_error();
    if (!p) return fail(FD_ERR_INVALID_ARGUMENT, "problem is NULL");
    // Any number of query tokens: the decode kernels' q_len limits do not apply.
    fd_problem one = *p;
    one.q_len = 1;
    float scale = 0.f;
    fd_status st = check_problem(&one, &scale);
    if (st != FD_OK) return st;
    if (p->q_len < 0) return fail(FD_ERR_INVALID_ARGUMENT, "q_len %d < 0", p->q_len);
    if (p->head_dim != 128) return fail(FD_ERR_UNSUPPORTED, "prefill is built for head_dim 128");
    if (p->kv_dtype == FD_FP8_E4M3) return fail(FD_ERR_UNSUPPORTED, "prefill reads fp16 or bf16 caches");
    if (!q || !k || !v || !seq_lens_dev || !out)
        return fail(FD_ERR_INVALID_ARGUMENT, "q, k, v, seq_lens_dev and out must be non-NULL");
    if (p->page_size && !block_table) return fail(FD_ERR_INVALID_ARGUMENT, "paged cache needs a block table");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
        return fail(FD_ERR_INVALID_ARGUMENT, "q, k and v must be 16-byte aligned");
    const int64_t blocks = (int64_t)p->batch * p->num_q_heads * ((problem_q_len(p) + 127) / 128);
    if (blocks > INT32_MAX) return fail(FD_ERR_INVALID_ARGUMENT, "too many query blocks");
    fdk::PrefillArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.table = block_table;
    a.lens = seq_lens_dev;
    a.out = out;
    a.lse = lse;
    a.batch = p->batch;
    a.hq = p->num_q_heads;
    a.hkv = p->num_kv_heads;
    a.q_len = problem_q_len(p);
    a.max_pages = p->page_size ? p->max_pages_per_seq : 0;
    a.qk_scale_log2 = scale * fdk::kLog2e;
    a.num_pages = p->page_size ? p->num_pages : 0;
    hipError_t e = fdk::launch_prefill(a, p->kv_dtype, p->out_dtype, p->page_size != 0,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FD_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

fd_status fd_append_kv(const fd_problem* p, int32_t rope_style, float rope_base, const void* k_new,
                       const void* v_new, void* q, const float* k_scale, const float* v_scale, void* k_cache,
                       void* v_cache, int32_t num_pages, const int32_t* block_table, const int32_t* seq_lens_dev,
                       void* stream) {
    clear_error();
    if (!p) return fail(FD_ERR_INVALID_ARGUMENT, "problem is NULL");
    // Any number of new tokens may be appended; the decode kernels' limits on
    // q_len do not apply here.
    fd_problem one = *p;
    one.q_len = 1;
    fd_status st = check_problem(&one, nullptr);
    if (st != FD_OK) return st;
    if (p->q_len < 0) return fail(FD_ERR_INVALID_ARGUMENT, "q_len %d < 0", p->q_len);
    if (p->page_size != kPageSize)
        return fail(FD_ERR_UNSUPPORTED, "fd_append_kv writes a paged cache (page_size 16)");
    if (rope_style < FD_ROPE_NONE || rope_style > FD_ROPE_HALF)
        return fail(FD_ERR_INVALID_ARGUMENT, "rope_style %d unknown", rope_style);
    if (rope_style != FD_ROPE_NONE && !(rope_base > 0.f && rope_base < __builtin_inff()))
        return fail(FD_ERR_INVALID_ARGUMENT, "rope_base must be positive and finite");
    if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !seq_lens_dev)
        return fail(FD_ERR_INVALID_ARGUMENT, "k_new, v_new, k_cache, v_cache, block_table and seq_lens_dev "
                    "must be non-NULL");
    if (num_pages < 1) return fail(FD_ERR_INVALID_ARGUMENT, "num_pages %d < 1", num_pages);
    const uintptr_t a16 = reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                          reinterpret_cast<uintptr_t>(q);
    const uintptr_t acache = reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache);
    if ((a16 & 15) || (acache & (kv_elem_bytes(p) == 1 ? 7 : 15)))
        return fail(FD_ERR_INVALID_ARGUMENT, "k_new, v_new, q and 16-bit caches must be 16-byte aligned, "
                    "FP8 caches 8-byte aligned");
    if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3)
        return fail(FD_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be 4-byte aligned");
    const int64_t blocks = (int64_t)p->batch * problem_q_len(p);
    if (blocks > INT32_MAX) return fail(FD_ERR_INVALID_ARGUMENT, "too many new tokens");

    fdk::AppendArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.q = q;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.table = block_table;
    a.lens = seq_lens_dev;
    a.n = problem_q_len(p);
    a.hkv = p->num_kv_heads;
    a.hq = p->num_q_heads;
    a.d = p->head_dim;
    a.max_pages = p->max_pages_per_seq;
    a.num_pages = num_pages;
    a.style = rope_style;
    a.rope_base = rope_base;
    // base^(-2i/d) as 2^(log2(base) * (-2i/d)) in double: within a few ulps
    // of the rounded power (a relative angle error near 1e-15, far below what
    // moves a stored 16-bit result); once per call instead of once per token.
    for (int i = 0; i < 64; ++i)
        a.inv_freq[i] = i < p->head_dim / 2 ? std::exp2(std::log2((double)rope_base) * (-2.0 * i / p->head_dim)) : 0.0;
    hipError_t e = fdk::launch_append(a, q_dtype_of(p), p->kv_dtype, (int)blocks, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FD_ERR_HIP, "append kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

}  // extern "C"
