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
    if (p->kv_dtype != FD_F16 && p->kv_dtype != FD_BF16 && p->kv_dtype != FD_FP8_E4M3)
        return fail(p->kv_dtype == FD_F32 ? FD_ERR_UNSUPPORTED : FD_ERR_INVALID_ARGUMENT,
                    "kv_dtype %d: fp16, bf16 or fp8 e4m3 only", p->kv_dtype);
    if (p->kv_dtype == FD_FP8_E4M3 && p->q_dtype != FD_F16 && p->q_dtype != FD_BF16)
        return fail(FD_ERR_INVALID_ARGUMENT, "q_dtype %d: an fp8 cache takes fp16 or bf16 queries", p->q_dtype);
    if (p->out_dtype != FD_F16 && p->out_dtype != FD_BF16 && p->out_dtype != FD_F32)
        return fail(FD_ERR_INVALID_ARGUMENT, "out_dtype %d unknown", p->out_dtype);
    if (p->page_size != 0 && p->page_size != kPageSize)
        return fail(p->page_size < 0 ? FD_ERR_INVALID_ARGUMENT : FD_ERR_UNSUPPORTED,
                    "page_size %d: 0 (contiguous) or 16 only", p->page_size);
    if (p->page_size && p->max_pages_per_seq < 1)
        return fail(FD_ERR_INVALID_ARGUMENT, "paged cache needs max_pages_per_seq >= 1");
    if (p->num_pages < 0) return fail(FD_ERR_INVALID_ARGUMENT, "num_pages %d < 0", p->num_pages);
    if (!(p->scale == p->scale) || isinf(p->scale))
        return fail(FD_ERR_INVALID_ARGUMENT, "scale is not finite");
    if (p->q_len < 0) return fail(FD_ERR_INVALID_ARGUMENT, "q_len %d < 0", p->q_len);
    if (problem_q_len(p) > 1 && (p->head_dim != 128 || problem_q_len(p) * G > kMaxQueryRows))
        return fail(FD_ERR_UNSUPPORTED, "q_len %d with %d query heads per KV head and d=%d not built "
                    "(several query tokens need d = 128 and q_len * Hq/Hkv <= %d)",
                    p->q_len, G, p->head_dim, kMaxQueryRows);
    if (scale_out) *scale_out = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
    return FD_OK;
}

uint64_t workspace_o_bytes(const fd_problem* p, int32_t max_splits) {
    return (uint64_t)p->batch * problem_q_len(p) * p->num_q_heads * max_splits * p->head_dim * sizeof(float);
}

uint64_t workspace_counters_offset(const fd_problem* p, int32_t max_splits) {
    const uint64_t end = workspace_o_bytes(p, max_splits) +
                         (uint64_t)p->batch * problem_q_len(p) * p->num_q_heads * max_splits * 2 * sizeof(float);
    return (end + 15) / 16 * 16;
}

uint64_t workspace_bytes(const fd_problem* p, int32_t max_splits) {
    const uint64_t counters = (uint64_t)p->batch * p->num_kv_heads * sizeof(uint32_t);
    return workspace_counters_offset(p, max_splits) + (counters + 15) / 16 * 16;
}

bool mfma_applicable(const fd_problem* p) {
    const int32_t rows = problem_q_len(p) * (p->num_q_heads / p->num_kv_heads);
    return p->head_dim == 128 && rows >= 2 && rows <= kMaxQueryRows;
}

bool mfma_heads_applicable(const fd_problem* p) {
    const int32_t nt = mfma_column_tiles(p);
    return mfma_applicable(p) && (nt == 1 || nt == 2 || nt == 4) && p->num_kv_heads % (kMfmaWaves / nt) == 0;
}

bool head_rows_applicable(const fd_problem* p) {
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    return problem_q_len(p) == 1 && G <= 2 && p->num_kv_heads % rows_per_load(p) == 0;
}

bool head_cols_applicable(const fd_problem* p) {
    return head_rows_applicable(p) && p->num_kv_heads % (rows_per_load(p) * head_cols_waves(p)) == 0;
}

int32_t heads_per_workgroup(const fd_problem* p, int32_t kernel) {
    if (kernel == kPartialHeadCols) return rows_per_load(p) * head_cols_waves(p);
    if (kernel == kPartialMfmaHeads) return kMfmaWaves / mfma_column_tiles(p);
    return kernel == kPartialHeadRows ? rows_per_load(p) : 1;
}

int32_t workgroups_per_split(const fd_problem* p, int32_t kernel) {
    const int32_t groups = p->num_kv_heads / heads_per_workgroup(p, kernel);
    return kernel == kPartialMfma ? groups * mfma_column_tiles(p) : groups;
}

int32_t combine_form(const fd_problem* p, int32_t max_splits) {
    const int64_t per_seq = (int64_t)problem_q_len(p) * p->num_q_heads;
    const int64_t rows = (int64_t)p->batch * per_seq;
    const int32_t forced = env_int("FD_COMBINE_FORM", -1);
    if (forced == 0 || forced == 1 || forced == 3 || (forced == 2 && per_seq % 2 == 0)) return forced;
    if (rows >= kCombineTwoRowRows && per_seq % 2 == 0) return 2;
    if (rows >= kCombinePerWaveRows) return 1;
    return max_splits >= kCombineWideSplits ? 3 : 0;
}

fd_status check_plan(const fd_problem* p, const fd_plan* plan) {
    if (!plan) return fail(FD_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (plan->chunk_tokens < 1 || plan->max_splits < 1 || plan->max_splits > kMaxGridYZ)
        return fail(FD_ERR_INVALID_ARGUMENT, "plan has chunk_tokens=%d max_splits=%d",
                    plan->chunk_tokens, plan->max_splits);
    if (plan->workspace_bytes < workspace_bytes(p, plan->max_splits))
        return fail(FD_ERR_INVALID_ARGUMENT, "plan does not belong to this problem (workspace_bytes)");
    if (plan->split_mode != 0 &&
        (plan->split_mode != 1 || !is_mfma_kernel(plan->partial_kernel) || plan->chunk_tokens % kTileTokens))
        return fail(FD_ERR_INVALID_ARGUMENT, "plan split_mode %d with kernel %d and chunk %d: the balanced mode "
                    "needs the matrix-core kernel and a chunk that is a multiple of %d",
                    plan->split_mode, plan->partial_kernel, plan->chunk_tokens, kTileTokens);
    if ((!is_mfma_kernel(plan->partial_kernel) && problem_q_len(p) > 1) ||
        (plan->partial_kernel == kPartialMfma && !mfma_applicable(p)) ||
        (plan->partial_kernel == kPartialMfmaHeads && !mfma_heads_applicable(p)) ||
        (plan->partial_kernel == kPartialHeadRows && !head_rows_applicable(p)) ||
        (plan->partial_kernel == kPartialHeadCols && !head_cols_applicable(p)) ||
        plan->partial_kernel < kPartialTokenRows || plan->partial_kernel > kPartialMfmaHeads)
        return fail(FD_ERR_INVALID_ARGUMENT, "plan names partial kernel %d, which does not cover this problem",
                    plan->partial_kernel);
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
        if (lens[b] < problem_q_len(p))
            return fail(FD_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %d is shorter than its %d query tokens", b,
                        lens[b], problem_q_len(p));
        total += lens[b];
        lmax = std::max(lmax, lens[b]);
    }

    if (num_cus == 0) {
        st = query_num_cus(&num_cus);
        if (st != FD_OK) return st;
    }

    // Query heads per KV head decide the partial kernel: a group of four or
    // more forms a contraction worth an MFMA; one or two queries per K/V row
    // leave a matrix instruction mostly idle, and the vector kernel reads
    // whole multi-head rows when Hkv allows. FD_PARTIAL_KERNEL=0/1/2 overrides
    // (when the forced kernel covers the problem).
    const int32_t G = p->num_q_heads / p->num_kv_heads;
    // Of the two matrix-core forms, the one whose waves each own a (KV head,
    // column tile) wherever the heads fill its work-groups (measured on
    // MI355X, same GPU, twice: GQA varlen 114.5 -> 109.3 us, paged GQA
    // 335.4 -> 324.8 us, paged GQA with 8 query tokens 704 -> 604 us).
    int32_t kernel = kPartialTokenRows;
    if (mfma_applicable(p) && (G >= 4 || problem_q_len(p) > 1))
        kernel = mfma_heads_applicable(p) ? kPartialMfmaHeads : kPartialMfma;
    else if (head_rows_applicable(p))
        kernel = kPartialHeadRows;
    const int32_t forced = env_int("FD_PARTIAL_KERNEL", -1);
    if (forced == kPartialTokenRows && problem_q_len(p) == 1) kernel = kPartialTokenRows;
    if (forced == kPartialMfma && mfma_applicable(p)) kernel = kPartialMfma;
    if (forced == kPartialHeadRows && head_rows_applicable(p)) kernel = kPartialHeadRows;
    if (forced == kPartialHeadCols && head_cols_applicable(p)) kernel = kPartialHeadCols;
    if (forced == kPartialMfmaHeads && mfma_heads_applicable(p)) kernel = kPartialMfmaHeads;
    if (force_num_splits == 0) force_num_splits = env_int("FD_NUM_SPLITS", 0);

    auto choose_chunk = [&](int32_t kern) -> int64_t {
        const int64_t wg_heads = workgroups_per_split(p, kern);
        int64_t c;
        if (force_num_splits > 0) {
            c = ceil_div(lmax, force_num_splits);
        } else {
            // Head-rows work-groups cover several heads and run best from
            // ~1024 tokens (2 KB per head of a 16-bit cache) per split when
            // the chip is full (measured on a 32K-token cache: 512-token
            // chunks 86.8 us against 85.3-85.9 at 1024 with the rotated
            // traversal, 102.2 without it); an FP8 split needs twice the
            // tokens for the same bytes (128K-token FP8 cache: 2048-token
            // splits 3% faster than 1024). Shorter contexts get shorter
            // head-row splits below (down to kHeadRowsFloorChunk).
            const int32_t head_rows_min = kHeadRowsMinChunk * 2 / kv_elem_bytes(p);
            // Head columns: the same bytes per work-group as head rows.
            const int32_t head_cols_min =
                std::max<int32_t>(kChunkGranule, head_rows_min / head_cols_waves(p));
            const int64_t min_chunk = std::max<int32_t>(
                1, env_int("FD_MIN_CHUNK", kern == kPartialHeadRows   ? head_rows_min
                                           : kern == kPartialHeadCols ? head_cols_min
                                                                      : kDefaultMinChunk));
            // Work-groups are (sequence, KV head group, split). A chunk that
            // makes about num_cus * k of them, never below the minimum chunk, a
            // multiple of 64.
            auto chunk_for = [&](int64_t k) {
                int64_t cc = ceil_div(total * wg_heads, std::max<int64_t>(1, (int64_t)num_cus * k));
                cc = std::max(cc, min_chunk);
                return ceil_div(cc, kChunkGranule) * kChunkGranule;
            };
            int32_t wg_per_cu = env_int("FD_WG_PER_CU", 0);
            if (wg_per_cu == 0 && kern == kPartialMfmaHeads && mfma_column_tiles(p) == 4)
                wg_per_cu = kWideMultiQueryWgPerCu;
            // One column tile on a 16-bit cache: one per CU, as on the balanced
            // list (measured per step, same GPU: 128K-token MHA with 4 query
            // tokens 325.5/326.1 -> 316.1/316.4 us, three per CU 332.8; equal
            // lengths, 32/8 heads: 16 x 8K tokens 86.1 -> 82.4 us, 16 x 4K
            // 48.2 -> 46.3, 4 x 32K 85.8 -> 82.4, 1 x 128K 89.1 -> 84.1; 64/8
            // heads, 64 x 2K 88.3 -> 84.1).
            if (wg_per_cu == 0 && kern == kPartialMfmaHeads && mfma_column_tiles(p) == 1 && kv_elem_bytes(p) == 2)
                wg_per_cu = kBalancedWgPerCuSingle16;
            if (wg_per_cu > 0) {
                c = chunk_for(wg_per_cu);
            } else {
                // The largest chunk (fewest, longest work-groups) such that the
                // full-size splits alone give every compute unit two
                // work-groups (three when shorter last splits exist) and at most
                // an eighth of the tokens sit in shorter last splits. Measured on
                // MI355X: uniform long contexts run best with ~2 work-groups per
                // CU; mixed lengths need smaller chunks so the longest-first work
                // list can even out the tail.
                static const int32_t kSteps[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
                c = chunk_for(kSteps[9]);
                for (int32_t k : kSteps) {
                    const int64_t cc = std::min<int64_t>(chunk_for(k), lmax);
                    int64_t full = 0, rest = 0;
                    for (int32_t b = 0; b < p->batch; ++b) {
                        full += lens[b] / cc;
                        rest += lens[b] % cc;
                    }
                    // An FP8 split holds half the bytes of a 16-bit one: the
                    // token-rows kernel wants twice the work-groups (measured:
                    // 32K-token FP8 MHA, 2048-token splits 53.3 us, 1024 50.5 us).
                    const int64_t per_cu = (rest == 0 ? 2 : 3) *
                                           (kern == kPartialTokenRows ? 2 / kv_elem_bytes(p) : 1);
                    const int64_t need = per_cu * (int64_t)num_cus;
                    if (full * wg_heads >= need && rest * 8 <= total) {
                        c = cc;
                        break;
                    }
                }
            }
        }
        return std::min<int64_t>(std::max<int64_t>(c, 1), std::max<int32_t>(lmax, 1));
    };
    int64_t chunk = choose_chunk(kernel);
    if (kernel == kPartialHeadRows && forced != kPartialHeadRows) {
        // Too few multi-head work-groups to occupy the chip: shorter head-row
        // splits first, halving the chunk down to kHeadRowsFloorChunk tokens
        // (or FD_MIN_CHUNK), until every CU has one; failing that (short or
        // forced few splits), one KV head per work-group (token rows) gives
        // Hkv/4 to Hkv/8 times more. Measured on MI355X (same GPU, one-shot
        // step, batch 1, 32 heads, d = 128): 16-bit 16K tokens 48.2 us as
        // token rows -> 45.8 us as 512-token head rows, 8K 26.2 -> 25.7 us
        // (256); FP8 32K 51.8 -> 49.5 us (512), FP8 64K 101.5 -> 89.2 us
        // (1024); FP8 16K unchanged (28.8 / 28.6 us) and FP8 8K stays on token
        // rows (20.2 us; 256-token head rows 22.6 us).
        const int64_t groups = p->num_kv_heads / heads_per_workgroup(p, kernel);
        auto workgroups = [&](int64_t c) {
            int64_t n = 0;
            for (int32_t b = 0; b < p->batch; ++b) n += ceil_div(lens[b], c);
            return n * groups;
        };
        if (force_num_splits == 0) {
            const int64_t floor_chunk = std::max<int32_t>(kHeadRowsFloorChunk, env_int("FD_MIN_CHUNK", 0));
            while (workgroups(chunk) < num_cus && chunk > floor_chunk)
                chunk = std::max<int64_t>(floor_chunk, ceil_div(chunk / 2, kChunkGranule) * kChunkGranule);
        }
        if (workgroups(chunk) < num_cus) {
            kernel = kPartialTokenRows;
            chunk = choose_chunk(kernel);
        }
    }
    // A ragged batch on the matrix-core kernel: per-sequence chunks leave
    // short last splits and a last round of work-groups that occupies part of
    // the chip, so the tiles of all sequences are dealt out in equal work
    // items instead (split_mode 1): one round of a few work-groups per
    // compute unit (kBalancedWgPerCu16 and the constants beside it).
    // FD_SPLIT_MODE=0/1 overrides; FD_WG_PER_CU sets the work-groups per CU.
    bool ragged = false;
    for (int32_t b = 1; b < p->batch; ++b) ragged |= lens[b] != lens[0];
    const bool balanced_ok = is_mfma_kernel(kernel);
    int32_t split_mode = (balanced_ok && force_num_splits == 0 && ragged && p->batch <= kBalancedMaxBatch) ? 1 : 0;
    const int32_t forced_mode = env_int("FD_SPLIT_MODE", -1);
    if (forced_mode == 0 || (forced_mode == 1 && balanced_ok)) split_mode = forced_mode;

    int64_t smax, nsplit = 0;
    if (split_mode == 1) {
        // List positions: per sequence kShareCost, then one per tile.
        int64_t positions = 0, nmax = 0;
        for (int32_t b = 0; b < p->batch; ++b) {
            const int64_t n = ceil_div(lens[b], kTileTokens);
            positions += n + kShareCost;
            nmax = std::max(nmax, n);
        }
        const int32_t per_cu = env_int("FD_WG_PER_CU", 0) > 0 ? env_int("FD_WG_PER_CU", 0)
                               : (kernel == kPartialMfmaHeads && mfma_column_tiles(p) == 4) ? kWideMultiQueryWgPerCu
                               : (kernel == kPartialMfmaHeads && mfma_column_tiles(p) == 1 && kv_elem_bytes(p) == 2)
                                   ? kBalancedWgPerCuSingle16
                               : (kernel == kPartialMfma && kv_elem_bytes(p) == 1) ? kBalancedWgPerCuFp8
                                                                                   : kBalancedWgPerCu16;
        const int64_t target = std::max<int64_t>(1, (int64_t)num_cus * per_cu);
        const int64_t P = std::max<int64_t>(ceil_div(positions * workgroups_per_split(p, kernel), target),
                                            kBalancedMinTiles);
        if (P * kTileTokens > INT32_MAX)
            return fail(FD_ERR_UNSUPPORTED, "work items of %lld tiles exceed the chunk range", (long long)P);
        chunk = P * kTileTokens;
        smax = ceil_div(nmax, P) + 1;
        nsplit = ceil_div(positions, P);
    } else {
        smax = ceil_div(lmax, chunk);
        for (int32_t b = 0; b < p->batch; ++b) nsplit += ceil_div(lens[b], chunk);
    }
    if (smax > kMaxGridYZ)
        return fail(FD_ERR_UNSUPPORTED, "%lld splits exceed the grid limit %d", (long long)smax,
                    kMaxGridYZ);

    fd_plan plan;
    memset(&plan, 0, sizeof(plan));
    plan.chunk_tokens = (int32_t)chunk;
    plan.max_splits = (int32_t)smax;
    plan.total_splits = (int32_t)std::min<int64_t>(nsplit, INT32_MAX);
    plan.num_cus = num_cus;
    plan.partial_kernel = kernel;
    plan.split_mode = split_mode;
    plan.total_tokens = total;
    plan.workspace_bytes = workspace_bytes(p, plan.max_splits);
    *out = plan;
    if (getenv("FD_LOG"))
        fprintf(stderr, "[fd] plan: B=%d Hq=%d Hkv=%d d=%d tokens=%lld chunk=%d S_max=%d splits=%d cus=%d kernel=%d mode=%d ws=%llu\n",
                p->batch, p->num_q_heads, p->num_kv_heads, p->head_dim, (long long)total, plan.chunk_tokens,
                plan.max_splits, plan.total_splits, plan.num_cus, plan.partial_kernel, plan.split_mode,
                (unsigned long long)plan.workspace_bytes);
    return FD_OK;
}

}  // extern "C"
