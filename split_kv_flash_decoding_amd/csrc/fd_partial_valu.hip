// Partial kernel, vector-ALU form: per-split online softmax for any group
// size G (query heads per KV head), d in {64, 128}, fp16/bf16 or FP8 (E4M3)
// K/V with per-head scales, contiguous or paged cache.
//
// The method: a single query token per sequence attends over a long KV cache
// that is cut along the token axis into splits; every split computes its local
// softmax statistics (running max m, running sum l) and an unnormalised partial
// output ("FlashAttention 全景演进与大模型 Token 生成全链路性能优化实战",
// §2.3 FlashDecoding; the tile recurrence is §2.2 of the lpnh.cn memory-wall
// article; rows and waves merge by the two-block identity of the capstone's
// §1.2 formal proof).
//
// One work-group of kWaves wave64s per (sequence, KV head, split), taken from
// the longest-first work list (locate_unit):
//   * a token row of one KV head is d fp16/bf16 values = d/8 lanes x 16 bytes
//     (d/16 lanes for FP8), so one wave-wide 16-byte load covers 64/(d/8)
//     consecutive tokens (4 at d = 128, 8 at d = 64; twice that for FP8,
//     whose codes widen exactly to the query's 16-bit type before the dot
//     product and to fp32 before the P.V update); each wave streams U such loads of K and U
//     of V per stage and issues the next stage's loads before it computes on
//     the current one (double buffering in registers: the data is used once,
//     so it never needs a trip through LDS); the loads carry the non-temporal
//     hint, since every K/V byte is read exactly once (measured +10% on
//     MI355X against plain loads);
//   * q.k is a packed fp16/bf16 dot product accumulating in fp32
//     (v_dot2_f32_f16 / v_dot2_f32_bf16) followed by a DPP butterfly across
//     the d/8 lanes of the row;
//   * each row of lanes keeps its own running max, sum and fp32 output slice
//     in registers (log2 domain: scores are pre-multiplied by scale*log2(e)
//     so every exponential is a hardware exp2);
//   * at the end the rows of a wave merge through lane shuffles, the waves
//     merge through LDS, and the split's (O, m, l) go to the workspace.
// The query heads of one GQA group share every K/V load (G scores per row).
// This is the kernel for MHA (G = 1), where one KV row serves one query head
// and a matrix instruction would idle 15/16 of its lanes.

#include "fd_device.h"

namespace fdk {

template <int D, int G, int KT, int QT, bool PAGED>
__global__ __launch_bounds__(kThreads) void partial_valu(const PartialArgs a) {
    using KV = KvLoad<KT, QT>;
    constexpr int EPL = KV::kElems;  // elements per 16-byte load
    constexpr int EB = 16 / EPL;     // bytes per element
    constexpr int LPR = D / EPL;     // lanes per token row
    constexpr int RPW = 64 / LPR;    // token rows per wave-wide load
    constexpr int U = kUnroll;       // loads of K (and of V) per stage
    constexpr int TPW = U * RPW;     // tokens per wave stage
    constexpr int QW = KV::kQWords;
    const uint16_t* __restrict__ q = a.q;
    const uint8_t* __restrict__ k = static_cast<const uint8_t*>(a.k);
    const uint8_t* __restrict__ v = static_cast<const uint8_t*>(a.v);
    const int32_t* __restrict__ block_table = a.table;
    const int32_t* __restrict__ seq_lens = a.lens;
    float* __restrict__ ws_o = a.ws_o;
    float* __restrict__ ws_ml = a.ws_ml;
    const int batch = a.batch, hq = a.hq, hkv = a.hkv, chunk = a.chunk, s_max = a.s_max, max_pages = a.max_pages;

    WorkUnit wu;
    if (!locate_unit(blockIdx.x, seq_lens, batch, hkv, chunk, PAGED ? max_pages * 16 : INT32_MAX, wu)) return;
    if (wu.s >= s_max) return;
    const int g = wu.g, s = wu.s, b = wu.b, t0 = wu.t0, t1 = wu.t1;
    const int64_t row0 = wu.row0;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane / LPR;
    const int c = lane % LPR;

    const int32_t* table = PAGED ? block_table + (int64_t)b * max_pages : nullptr;
    const int64_t head_off = (int64_t)g * D * EB + c * 16;  // bytes
    const float qk_scale_log2 = a.qk_scale_log2 * head_scale(a.k_scale, g);

    auto row_offset = [&](int t) -> int64_t {
        int64_t row;
        if constexpr (PAGED) {
            row = (int64_t)checked_page(table[t >> 4], a.num_pages) * 16 + (t & 15);
        } else {
            row = row0 + t;
        }
        return row * hkv * D * EB + head_off;
    };

    // This lane's slice of the G query heads of KV head g.
    u32x4 qv[G][QW];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int w = 0; w < QW; ++w)
            qv[j][w] = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * hq + g * G + j) * D + c * EPL + 8 * w);

    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = neg_inf();
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
    }

    const int ntok = t1 - t0;
    const int ntiles = (ntok + TPW - 1) / TPW;

    auto load = [&](int tile, u32x4* kb, u32x4* vb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int t = t0 + tile * TPW + u * RPW + r;
            t = min(t, t1 - 1);  // rows past the split re-read its last row; masked below
            const int64_t off = row_offset(t);
            kb[u] = load16(k + off);
            vb[u] = load16(v + off);
        }
    };

    auto compute = [&](int tile, const u32x4* kb, const u32x4* vb) {
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = (t0 + tile * TPW + u * RPW + r) < t1;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float dot = row_sum<LPR>(KV::dot(qv[j], kb[u]));
                sc[u][j] = valid ? dot * qk_scale_log2 : neg_inf();
            }
        }
        // Running statistics first, then O = alpha O + sum_u p_u v_u with each
        // V load widened to fp32 just before its products (one load's worth
        // of fp32 values live at a time, not U).
        float p[G][U];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = sc[0][j];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
            const float mn = fmaxf(m[j], mx);
            const float mu = (mn == neg_inf()) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m[j] - mu);
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[j][u] = __builtin_amdgcn_exp2f(sc[u][j] - mu);
                ps += p[j][u];
            }
            l[j] = l[j] * alpha + ps;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[j][e] *= alpha;
            m[j] = mn;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            KV::to_f32(vb[u], vf);
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[j][e] = fmaf(p[j][u], vf[e], o[j][e]);
        }
    };

    u32x4 ka[U], va[U], kb2[U], vb2[U];
    int tile = wave;
    if (tile < ntiles) load(tile, ka, va);
    while (tile < ntiles) {
        int nxt = tile + kWaves;
        if (nxt < ntiles) load(nxt, kb2, vb2);
        compute(tile, ka, va);
        tile = nxt;
        if (tile >= ntiles) break;
        nxt = tile + kWaves;
        if (nxt < ntiles) load(nxt, ka, va);
        compute(tile, kb2, vb2);
        tile = nxt;
    }

    // Merge the rows of lanes of this wave (they hold disjoint token subsets).
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float o2[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) o2[e] = __shfl_xor(o[j][e], off);
            const float m2 = __shfl_xor(m[j], off);
            const float l2 = __shfl_xor(l[j], off);
            merge_stats<EPL>(m[j], l[j], o[j], m2, l2, o2);
        }
    }

    // Merge the waves through LDS and write the split's statistics.
    __shared__ float sm_o[kWaves][G][D];
    __shared__ float sm_m[kWaves][G];
    __shared__ float sm_l[kWaves][G];
    if (r == 0) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_o[wave][j][c * EPL + e] = o[j][e];
            if (c == 0) {
                sm_m[wave][j] = m[j];
                sm_l[wave][j] = l[j];
            }
        }
    }
    __syncthreads();
    const float v_sc = head_scale(a.v_scale, g);
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int j = idx / D;
        const int col = idx % D;
        float M = sm_m[0][j];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
        const float mu = (M == neg_inf()) ? 0.f : M;
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float a = __builtin_amdgcn_exp2f(sm_m[w][j] - mu);
            acc += a * sm_o[w][j][col];
            lsum += a * sm_l[w][j];
        }
        const int h = g * G + j;
        const int64_t slot = ((int64_t)b * hq + h) * s_max + s;
        ws_o[slot * D + col] = acc * v_sc;
        if (col == 0) {
            ws_ml[slot * 2] = M * kLn2;
            ws_ml[slot * 2 + 1] = lsum;
        }
    }
    if (a.counters) fused_merge<D, G, kWaves>(a, b, (wu.L + chunk - 1) / chunk, g, 1, G, 1, &sm_o[0][0][0]);
}

// ------------------------------------------------- partial kernel, head rows

// The same online softmax with the roles of the lane rows swapped: row r of a
// wave holds KV head g0 + r (RPW consecutive heads per work-group), so one
// 16-byte load instruction covers one token of RPW heads, RPW * 2d bytes in a
// row of the token-major cache (1 KB at d = 128). Whole contiguous kilobytes
// per instruction stream from HBM faster than RPW separate 2d-byte rows
// (a read-only probe of the two patterns measured ~7.0 against ~6.5 TB/s on
// MI355X). Rows never mix heads, so only the waves merge at the end.
// Requires Hkv % RPW == 0. PAGE_MODE: 0 contiguous, 1 paged (a table lookup
// per token), 2 paged with page-aligned splits and U dividing 16 (page
// indices fetched 64 at a time and read with readlane).
// Waves per work-group: eight, except head columns (WH) on an FP8 cache,
// four (a work-group then covers 32 heads, a whole 4 KB token row of a
// 32-head cache with d = 128; eight would need 64 heads). Eight against four head-rows waves, measured on MI355X
// (same GPU, 200 steps, twice, per partial launch): 16-bit 32K-token MHA
// 87.9/88.2 -> 86.2/86.0 us, 128K-token MHA 320.4/321.1 -> 319.1/318.6 us;
// FP8 32K 48.3/47.7 -> 47.7/47.2 us, 128K 168.2 -> 166.0 us.
constexpr int head_rows_waves(int kt, bool wh) { return (wh && kt == FD_FP8_E4M3) ? 4 : 8; }

// WH (head columns): the waves of a work-group take different heads of the
// same tokens instead of different tokens of the same heads. Wave w owns KV
// heads (blk * NW + w) * RPW .. +RPW for every token of the split, so the
// work-group reads NW * RPW * 2d bytes of each token row together (8 KB at
// 32 heads, d = 128: whole rows of the token-major cache), and no two waves
// share a head: each writes its own partial, with no merge through LDS and
// no barrier. Requires Hkv % (NW * RPW) == 0.
template <int D, int G, int KT, int QT, int PAGE_MODE, bool WH = false>
__global__ __launch_bounds__(64 * head_rows_waves(KT, WH)) void partial_valu_heads(const PartialArgs a) {
    using KV = KvLoad<KT, QT>;
    constexpr int NW = head_rows_waves(KT, WH);  // waves per work-group
    constexpr int EPL = KV::kElems;  // elements per 16-byte load
    constexpr int EB = 16 / EPL;     // bytes per element
    constexpr int LPR = D / EPL;     // lanes per head row
    constexpr int RPW = 64 / LPR;    // heads per wave
    constexpr int HPW = WH ? NW * RPW : RPW;  // heads per work-group
    constexpr int SSTEP = WH ? 1 : NW;         // a wave's stride through the split's stages
    constexpr int U = kUnroll;       // tokens per wave stage
    constexpr int QW = KV::kQWords;
    constexpr bool PAGED = PAGE_MODE != 0;
    const uint16_t* __restrict__ q = a.q;
    const int32_t* __restrict__ block_table = a.table;
    const int32_t* __restrict__ seq_lens = a.lens;
    float* __restrict__ ws_o = a.ws_o;
    float* __restrict__ ws_ml = a.ws_ml;
    const int batch = a.batch, hq = a.hq, hkv = a.hkv, chunk = a.chunk, s_max = a.s_max, max_pages = a.max_pages;

    WorkUnit wu;
    if (!locate_unit(blockIdx.x, seq_lens, batch, hkv / HPW, chunk, PAGED ? max_pages * 16 : INT32_MAX, wu)) return;
    if (wu.s >= s_max) return;
    const int s = wu.s, b = wu.b, t0 = wu.t0, t1 = wu.t1;
    const int64_t row0 = wu.row0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane / LPR;
    const int c = lane % LPR;
    const int g0 = WH ? (wu.g * NW + wave) * RPW : wu.g * RPW;  // this wave's first KV head
    const int g = g0 + r;                                      // this row's KV head

    const int32_t* table = PAGED ? block_table + (int64_t)b * max_pages : nullptr;
    const int64_t row_stride = (int64_t)hkv * D * EB;  // bytes
    const uint8_t* kl = static_cast<const uint8_t*>(a.k) + (int64_t)g * D * EB + c * 16;
    const uint8_t* vl = static_cast<const uint8_t*>(a.v) + (int64_t)g * D * EB + c * 16;
    const float qk_scale_log2 = a.qk_scale_log2 * head_scale(a.k_scale, g);

    u32x4 qv[G][QW];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int w = 0; w < QW; ++w)
            qv[j][w] = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * hq + g * G + j) * D + c * EPL + 8 * w);

    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = neg_inf();
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
    }

    const int nstages = (t1 - t0 + U - 1) / U;

    // Page-aligned splits: lane i holds the page of this wave's stage 64 blk + i.
    const int first_stage = WH ? 0 : wave;
    int pg = 0, pg_blk = -1;
    auto stage_page_row = [&](int stage) -> int64_t {
        const int kk = (stage - first_stage) / SSTEP;
        const int blk = kk >> 6;
        if (blk != pg_blk) {
            const int st = first_stage + SSTEP * (64 * blk + lane);
            pg = st < nstages ? checked_page(table[(t0 + st * U) >> 4], a.num_pages) : 0;
            pg_blk = blk;
        }
        return (int64_t)__builtin_amdgcn_readlane(pg, kk & 63) * 16;
    };

    // Rotated traversal. Full splits of a contiguous 16-bit cache start at
    // different stages (split s at (7 s mod n) NW of its n NW stages, then
    // wrapping round) instead of all at their first rows, which lie a
    // power-of-two chunk apart and would otherwise be walked in step with
    // each other. Measured on MI355X (same GPU, twice):
    // 32K-token MHA 86.3/86.9 -> 85.3/85.9 us per partial launch, 128K-token
    // MHA 318.7/320.4 -> 317.3/317.7 us; with 512-token splits (two
    // work-groups per CU) the 32K cache went from 102.2 to 86.8 us. The FP8
    // head-rows cache ran slower rotated (165.5 -> 174.3 us at 128K) and
    // keeps the plain order.
    // The order of a split's tokens is free: the online softmax merges them in
    // any order.
    int rot = 0;
    if constexpr (PAGE_MODE == 0 && !WH && KT != FD_FP8_E4M3) {
        const int per = nstages / SSTEP;
        if (nstages % SSTEP == 0 && per > 0) rot = ((s * 7) % per) * SSTEP;
    }
    auto load = [&](int stage_, u32x4* kb, u32x4* vb) {
        const int stage = stage_ + rot < nstages ? stage_ + rot : stage_ + rot - nstages;
        const int ts = t0 + stage * U;
        int64_t prow = 0;
        if constexpr (PAGE_MODE == 2) prow = stage_page_row(stage);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = min(ts + u, t1 - 1);  // tokens past the split re-read its last one; masked below
            int64_t row;
            if constexpr (PAGE_MODE == 2) {
                row = prow + (t & 15);
            } else if constexpr (PAGE_MODE == 1) {
                row = (int64_t)checked_page(table[t >> 4], a.num_pages) * 16 + (t & 15);
            } else {
                row = row0 + t;
            }
            kb[u] = load16(kl + row * row_stride);
            vb[u] = load16(vl + row * row_stride);
        }
    };

    auto compute = [&](int stage_, const u32x4* kb, const u32x4* vb) {
        const int stage = stage_ + rot < nstages ? stage_ + rot : stage_ + rot - nstages;
        const int ts = t0 + stage * U;
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = ts + u < t1;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float dot = row_sum<LPR>(KV::dot(qv[j], kb[u]));
                sc[u][j] = valid ? dot * qk_scale_log2 : neg_inf();
            }
        }
        // Running statistics first, then O = alpha O + sum_u p_u v_u with each
        // V load widened to fp32 just before its products (one load's worth
        // of fp32 values live at a time, not U).
        float p[G][U];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = sc[0][j];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
            const float mn = fmaxf(m[j], mx);
            const float mu = (mn == neg_inf()) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m[j] - mu);
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[j][u] = __builtin_amdgcn_exp2f(sc[u][j] - mu);
                ps += p[j][u];
            }
            l[j] = l[j] * alpha + ps;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[j][e] *= alpha;
            m[j] = mn;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            KV::to_f32(vb[u], vf);
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[j][e] = fmaf(p[j][u], vf[e], o[j][e]);
        }
    };

    u32x4 ka[U], va[U], kb2[U], vb2[U];
    int stage = first_stage;
    if (stage < nstages) load(stage, ka, va);
    while (stage < nstages) {
        int nxt = stage + SSTEP;
        if (nxt < nstages) load(nxt, kb2, vb2);
        compute(stage, ka, va);
        stage = nxt;
        if (stage >= nstages) break;
        nxt = stage + SSTEP;
        if (nxt < nstages) load(nxt, ka, va);
        compute(stage, kb2, vb2);
        stage = nxt;
    }

    if constexpr (WH) {
        // Each wave holds whole heads: lane (r, c) writes its slice of head
        // g's outputs; every lane of a row holds the same m and l.
        const float v_sc = head_scale(a.v_scale, g);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int64_t slot = ((int64_t)b * hq + g * G + j) * s_max + s;
#pragma unroll
            for (int e = 0; e < EPL; e += 4)
                *reinterpret_cast<float4*>(ws_o + slot * D + c * EPL + e) =
                    make_float4(o[j][e] * v_sc, o[j][e + 1] * v_sc, o[j][e + 2] * v_sc, o[j][e + 3] * v_sc);
            if (c == 0) {
                ws_ml[slot * 2] = m[j] * kLn2;
                ws_ml[slot * 2 + 1] = l[j];
            }
        }
        if (a.counters) {
            __shared__ float sm_red[NW * 4 * D];
            fused_merge<D, 4, NW>(a, b, (wu.L + chunk - 1) / chunk, wu.g * HPW, HPW, HPW * G, 1, sm_red);
        }
        return;
    }

    // Merge the waves through LDS (every lane of a row holds the same m, l).
    __shared__ float sm_o[NW][RPW][G][D];
    __shared__ float sm_m[NW][RPW][G];
    __shared__ float sm_l[NW][RPW][G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sm_o[wave][r][j][c * EPL + e] = o[j][e];
        if (c == 0) {
            sm_m[wave][r][j] = m[j];
            sm_l[wave][r][j] = l[j];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < RPW * G * D; idx += (64 * NW)) {
        const int rr = idx / (G * D);
        const int j = (idx / D) % G;
        const int col = idx % D;
        float M = sm_m[0][rr][j];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][rr][j]);
        const float mu = (M == neg_inf()) ? 0.f : M;
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float a = __builtin_amdgcn_exp2f(sm_m[w][rr][j] - mu);
            acc += a * sm_o[w][rr][j][col];
            lsum += a * sm_l[w][rr][j];
        }
        const int h = (wu.g * RPW + rr) * G + j;
        const int64_t slot = ((int64_t)b * hq + h) * s_max + s;
        ws_o[slot * D + col] = acc * head_scale(a.v_scale, wu.g * RPW + rr);
        if (col == 0) {
            ws_ml[slot * 2] = M * kLn2;
            ws_ml[slot * 2 + 1] = lsum;
        }
    }
    if (a.counters) fused_merge<D, RPW * G, NW>(a, b, (wu.L + chunk - 1) / chunk, wu.g * RPW, RPW, RPW * G, 1, &sm_o[0][0][0][0]);
}

// ------------------------------------------------------------------ dispatch

// Calls f.template operator()<KT, QT>() for the problem's cache and query types.
template <typename F>
hipError_t with_types(const PartialArgs& a, F&& f) {
    if (a.kv_dt == FD_FP8_E4M3)
        return a.q_dt == FD_F16 ? f.template operator()<FD_FP8_E4M3, FD_F16>()
                                : f.template operator()<FD_FP8_E4M3, FD_BF16>();
    return a.kv_dt == FD_F16 ? f.template operator()<FD_F16, FD_F16>() : f.template operator()<FD_BF16, FD_BF16>();
}

template <int D, int G>
hipError_t launch_tokens_g(bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    return with_types(a, [&]<int KT, int QT>() {
        if (paged)
            hipLaunchKernelGGL((partial_valu<D, G, KT, QT, true>), grid, dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((partial_valu<D, G, KT, QT, false>), grid, dim3(kThreads), 0, st, a);
        return hipGetLastError();
    });
}

template <int D>
hipError_t launch_tokens_d(int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: return launch_tokens_g<D, 1>(paged, a, grid, st);
        case 2: return launch_tokens_g<D, 2>(paged, a, grid, st);
        case 4: return launch_tokens_g<D, 4>(paged, a, grid, st);
        default: return launch_tokens_g<D, 8>(paged, a, grid, st);
    }
}

hipError_t launch_partial_valu(int D, int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    return D == 64 ? launch_tokens_d<64>(G, paged, a, grid, st) : launch_tokens_d<128>(G, paged, a, grid, st);
}

template <int D, int G, bool WH>
hipError_t launch_heads_g(bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    // Paged splits that start on page boundaries read their page indices 64 at a time.
    const int mode = !paged ? 0 : ((a.chunk % 16 == 0) && (16 % kUnroll == 0)) ? 2 : 1;
    return with_types(a, [&]<int KT, int QT>() {
        if (mode == 0)
            hipLaunchKernelGGL((partial_valu_heads<D, G, KT, QT, 0, WH>), grid, dim3(64 * head_rows_waves(KT, WH)), 0, st,
                               a);
        else if (mode == 1)
            hipLaunchKernelGGL((partial_valu_heads<D, G, KT, QT, 1, WH>), grid, dim3(64 * head_rows_waves(KT, WH)), 0, st,
                               a);
        else
            hipLaunchKernelGGL((partial_valu_heads<D, G, KT, QT, 2, WH>), grid, dim3(64 * head_rows_waves(KT, WH)), 0, st,
                               a);
        return hipGetLastError();
    });
}

template <bool WH>
hipError_t launch_heads(int D, int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    if (D == 64)
        return G == 1 ? launch_heads_g<64, 1, WH>(paged, a, grid, st) : launch_heads_g<64, 2, WH>(paged, a, grid, st);
    return G == 1 ? launch_heads_g<128, 1, WH>(paged, a, grid, st) : launch_heads_g<128, 2, WH>(paged, a, grid, st);
}

hipError_t launch_partial_valu_heads(int D, int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    return launch_heads<false>(D, G, paged, a, grid, st);
}

hipError_t launch_partial_valu_head_cols(int D, int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    return launch_heads<true>(D, G, paged, a, grid, st);
}

}  // namespace fdk
