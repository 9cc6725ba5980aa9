// Host-side validation, split planning and error reporting for fd.h.
// Pure C++: the only HIP call reachable from here is the compute-unit query,
// which lives in fd_api.hip and runs only when the caller passes
// num_cus = 0.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "fd_internal.h"

namespace fd {

namespace {
thread_local char g_msg[512] = "";

int32_t env_int(const char* name, int32_t dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    char* end = nullptr;
    long v = strtol(s, &end, 10);
    if (end == s || v < 0 || v > (1L << 30)) return dflt;
    return static_cast<int32_t>(v);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

fd_status fail(fd_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_msg[0] = '\0'; }

fd_status check_problem(const fd_problem* p, float* scale_out) {
    if (!p) return fail(FD_ERR_INVALID_ARGUMENT, "problem is NULL");
    if (p->batch < 1 || p->batch > kMaxGridYZ)
        return fail(FD_ERR_INVALID_ARGUMENT, "batch %d outside [1, %d]", p->batch, kMaxGridYZ);
    if (p->num_q_heads < 1 || p->num_kv_heads < 1)
        return fail(FD_ERR_INVALID_ARGUMENT, "head counts must be positive (Hq=%d, Hkv=%d)",
                    p->num_q_heads, p->num_kv_heads);
    if (p->num_q_heads % p->num_kv_heads)
        return fail(FD_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", p->num_q_heads,
                    p->num_kv_heads);
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(FD_ERR_UNSUPPORTED, "group size Hq/Hkv=%d not built (1, 2, 4, 8)", G);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(FD_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", p->head_dim);
    if (p->kv_dtype != FD_F16 && p->kv_dtype != FD_BF16)
        return fail(p->kv_dtype == FD_F32 ? FD_ERR_UNSUPPORTED : FD_ERR_INVALID_ARGUMENT,
                    "kv_dtype %d: fp16 or bf16 only", p->kv_dtype);
    if (p->out_dtype != FD_F16 && p->out_dtype != FD_BF16 && p->out_dtype != FD_F32)
        return fail(FD_ERR_INVALID_ARGUMENT, "out_dtype %d unknown", p->out_dtype);
    if (p->page_size != 0 && p->page_size != kPageSize)
        return fail(p->page_size < 0 ? FD_ERR_INVALID_ARGUMENT : FD_ERR_UNSUPPORTED,
                    "page_size %d: 0 (contiguous) or 16 only", p->page_size);
    if (p->page_size && p->max_pages_per_seq < 1)
        return fail(FD_ERR_INVALID_ARGUMENT, "paged cache needs max_pages_per_seq >= 1");
    if (!(p->scale == p->scale) || isinf(p->scale))
        return fail(FD_ERR_INVALID_ARGUMENT, "scale is not finite");
    if (scale_out) *scale_out = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
    return FD_OK;
}

uint64_t workspace_o_bytes(const fd_problem* p, int32_t max_splits) {
    return (uint64_t)p->batch * p->num_q_heads * max_splits * p->head_dim * sizeof(float);
}

uint64_t workspace_bytes(const fd_problem* p, int32_t max_splits) {
    return workspace_o_bytes(p, max_splits) +
           (uint64_t)p->batch * p->num_q_heads * max_splits * 2 * sizeof(float);
}

bool mfma_applicable(const fd_problem* p) {
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    return p->head_dim == 128 && (G == 2 || G == 4 || G == 8);
}

fd_status check_plan(const fd_problem* p, const fd_plan* plan) {
    if (!plan) return fail(FD_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (plan->chunk_tokens < 1 || plan->max_splits < 1 || plan->max_splits > kMaxGridYZ)
        return fail(FD_ERR_INVALID_ARGUMENT, "plan has chunk_tokens=%d max_splits=%d",
                    plan->chunk_tokens, plan->max_splits);
    if (plan->workspace_bytes < workspace_bytes(p, plan->max_splits))
        return fail(FD_ERR_INVALID_ARGUMENT, "plan does not belong to this problem (workspace_bytes)");
    if (plan->partial_kernel != 0 && plan->partial_kernel != 1)
        return fail(FD_ERR_INVALID_ARGUMENT, "plan names unknown partial kernel %d", plan->partial_kernel);
    return FD_OK;
}

}  // namespace fd

using namespace fd;

extern "C" {

const char* fd_status_string(fd_status s) {
    switch (s) {
        case FD_OK: return "FD_OK";
        case FD_ERR_INVALID_ARGUMENT: return "FD_ERR_INVALID_ARGUMENT";
        case FD_ERR_UNSUPPORTED: return "FD_ERR_UNSUPPORTED";
        case FD_ERR_WORKSPACE_TOO_SMALL: return "FD_ERR_WORKSPACE_TOO_SMALL";
        case FD_ERR_HIP: return "FD_ERR_HIP";
    }
    return "FD_ERR_UNKNOWN";
}

const char* fd_last_error_message(void) { return g_msg; }

fd_status fd_plan_splits(const fd_problem* p, const int32_t* lens, int32_t num_cus,
                         int32_t force_num_splits, fd_plan* out) {
    clear_error();
    fd_status st = check_problem(p, nullptr);
    if (st != FD_OK) return st;
    if (!lens) return fail(FD_ERR_INVALID_ARGUMENT, "seq_lens_host is NULL");
    if (!out) return fail(FD_ERR_INVALID_ARGUMENT, "plan output is NULL");
    if (num_cus < 0) return fail(FD_ERR_INVALID_ARGUMENT, "num_cus %d < 0", num_cus);
    if (force_num_splits < 0)
        return fail(FD_ERR_INVALID_ARGUMENT, "force_num_splits %d < 0", force_num_splits);

    int64_t total = 0;
    int32_t lmax = 0;
    const int64_t cap = p->page_size ? (int64_t)p->max_pages_per_seq * p->page_size : INT32_MAX;
    for (int32_t b = 0; b < p->batch; ++b) {
        if (lens[b] < 1)
            return fail(FD_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %d: every sequence needs a token", b,
                        lens[b]);
        if (lens[b] > cap)
            return fail(FD_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %d exceeds the block table (%lld tokens)",
                        b, lens[b], (long long)cap);
        total += lens[b];
        lmax = std::max(lmax, lens[b]);
    }

    if (num_cus == 0) {
        st = query_num_cus(&num_cus);
        if (st != FD_OK) return st;
    }

    if (force_num_splits == 0) force_num_splits = env_int("FD_NUM_SPLITS", 0);
    int64_t chunk;
    if (force_num_splits > 0) {
        chunk = ceil_div(lmax, force_num_splits);
    } else {
        const int64_t min_chunk = std::max<int32_t>(1, env_int("FD_MIN_CHUNK", kDefaultMinChunk));
        const int64_t wg_per_cu = std::max<int32_t>(1, env_int("FD_WG_PER_CU", kDefaultWgPerCu));
        const int64_t target = (int64_t)num_cus * wg_per_cu;
        // Work-groups are (sequence, KV head, split); pick the chunk that makes
        // about `target` of them, never below the minimum chunk.
        chunk = ceil_div(total * p->num_kv_heads, std::max<int64_t>(1, target));
        chunk = std::max(chunk, min_chunk);
        chunk = ceil_div(chunk, kChunkGranule) * kChunkGranule;
    }
    chunk = std::min<int64_t>(std::max<int64_t>(chunk, 1), std::max<int32_t>(lmax, 1));
    int64_t smax = ceil_div(lmax, chunk);
    if (smax > kMaxGridYZ)
        return fail(FD_ERR_UNSUPPORTED, "%lld splits exceed the grid limit %d", (long long)smax,
                    kMaxGridYZ);
    int64_t nsplit = 0;
    for (int32_t b = 0; b < p->batch; ++b) nsplit += ceil_div(lens[b], chunk);

    fd_plan plan;
    memset(&plan, 0, sizeof(plan));
    plan.chunk_tokens = (int32_t)chunk;
    plan.max_splits = (int32_t)smax;
    plan.total_splits = (int32_t)std::min<int64_t>(nsplit, INT32_MAX);
    plan.num_cus = num_cus;
    // Query heads per KV head decide the partial kernel: one query per K/V row
    // leaves nothing for a matrix instruction to share; a group of four or
    // more forms a contraction worth an MFMA. FD_PARTIAL_KERNEL=0/1 overrides.
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    int32_t kernel = (mfma_applicable(p) && G >= 4) ? 1 : 0;
    const int32_t forced = env_int("FD_PARTIAL_KERNEL", -1);
    if (forced == 0) kernel = 0;
    if (forced == 1 && mfma_applicable(p)) kernel = 1;
    plan.partial_kernel = kernel;
    plan.total_tokens = total;
    plan.workspace_bytes = workspace_bytes(p, plan.max_splits);
    *out = plan;
    if (getenv("FD_LOG"))
        fprintf(stderr, "[fd] plan: B=%d Hq=%d Hkv=%d d=%d tokens=%lld chunk=%d S_max=%d splits=%d cus=%d kernel=%d ws=%llu\n",
                p->batch, p->num_q_heads, p->num_kv_heads, p->head_dim, (long long)total, plan.chunk_tokens,
                plan.max_splits, plan.total_splits, plan.num_cus, plan.partial_kernel,
                (unsigned long long)plan.workspace_bytes);
    return FD_OK;
}

}  // extern "C"
