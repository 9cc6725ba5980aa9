// Combine kernel: merges the per-split statistics of every (sequence, query
// head) into the output and its log-sum-exp. M = max_s m_s over all splits,
// then w_s = exp(m_s - M) weighs l_s and O_s;
// out = sum_s w_s O_s / sum_s w_s l_s, lse = M + ln(sum_s w_s l_s). This is
// the cross-chunk reduce of FlashDecoding ("FlashAttention 全景演进与大模型
// Token 生成全链路性能优化实战", §2.3), with every split rescaled by the
// two-block identity of the same page's §1.2. Four forms: four waves per
// row (each sums every fourth split, eight splits' loads in flight, the waves
// add up in LDS) for batches with few rows, sixteen waves per row when those
// rows have many splits; one wave per row,
// four rows per work-group, for batches with many rows, where four waves per
// row would take several rounds of the chip's wave slots for rows that have
// few splits; two rows per wave (32 lanes each) for the largest batches with
// an even number of rows per sequence. Under the balanced split mode a
// sequence's split count comes from the position of its first tile in the
// list of all sequences, a prefix sum each wave computes over seq_lens.

#include "fd_device.h"

namespace fdk {


constexpr int kCombineWaves = 4;

// Splits of sequence b under the plan's split mode (a whole wave calls this).
__device__ inline int combine_split_count(const int32_t* __restrict__ seq_lens, int b, int chunk, int s_max,
                                          int split_mode, int len_cap) {
    if (split_mode == 0) {
        const int L = seq_lens[b];
        return L > 0 ? min((L + chunk - 1) / chunk, s_max) : 0;
    }
    const int lane = threadIdx.x & 63;
    int64_t U = 0;  // list positions of sequences 0..b-1
    for (int base = 0; base < b; base += 64) {
        const int i = base + lane;
        int64_t u = i < b ? seq_positions(seq_tiles(max(0, min(seq_lens[i], len_cap)))) : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) u += __shfl_xor(u, off);
        U += u;
    }
    return min(balanced_splits(U + fd::kShareCost, seq_tiles(max(0, min(seq_lens[b], len_cap))), chunk >> 4),
               s_max);
}

// One wave per (sequence, query row) r = b * hq + h, four rows per work-group.
template <int D, int OUT>
__global__ __launch_bounds__(64 * kCombineWaves) void combine_rows(const float* __restrict__ ws_o,
                                                                   const float* __restrict__ ws_ml,
                                                                   const int32_t* __restrict__ seq_lens,
                                                                   void* __restrict__ out, float* __restrict__ lse,
                                                                   int rows, int hq, int chunk, int s_max,
                                                                   int split_mode, int len_cap) {
    constexpr int PER = D / 64;  // output columns per lane
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
    if (r >= rows) return;  // a whole wave: no barrier follows
    const int b = r / hq;
    const int64_t base = (int64_t)r * s_max;
    const int64_t orow = (int64_t)r * D;
    // The first 64 slots' m_s are read while the split count is worked out
    // (slots past it exist and are masked).
    const float m_first = lane < s_max ? ws_ml[(base + lane) * 2] : neg_inf();
    const int S = combine_split_count(seq_lens, b, chunk, s_max, split_mode, len_cap);
    if (S == 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e) store_out<OUT>(out, orow + lane * PER + e, 0.f);
        if (lse && lane == 0) lse[r] = neg_inf();
        return;
    }
    float M = lane < S ? m_first : neg_inf();
    for (int i = lane + 64; i < S; i += 64) M = fmaxf(M, ws_ml[(base + i) * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float l = 0.f;
#pragma unroll 8
    for (int i = 0; i < S; ++i) {
        const float w = __builtin_amdgcn_exp2f((ws_ml[(base + i) * 2] - M) * kLog2e);
        l = fmaf(w, ws_ml[(base + i) * 2 + 1], l);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, ws_o[(base + i) * D + lane * PER + e], acc[e]);
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < PER; ++e) store_out<OUT>(out, orow + lane * PER + e, acc[e] * inv);
    if (lse && lane == 0) lse[r] = M + __builtin_amdgcn_logf(l) * kLn2;
}

// Two rows per wave (lanes 0-31 row r0, lanes 32-63 row r0 + 1, each lane D/32
// columns), four waves per work-group: for the largest batches, half the waves
// of one row per wave. The rows of a sequence must be even in number, so both
// rows of a wave belong to the same sequence.
template <int D, int OUT>
__global__ __launch_bounds__(64 * kCombineWaves) void combine_rows2(const float* __restrict__ ws_o,
                                                                    const float* __restrict__ ws_ml,
                                                                    const int32_t* __restrict__ seq_lens,
                                                                    void* __restrict__ out, float* __restrict__ lse,
                                                                    int rows, int hq, int chunk, int s_max,
                                                                    int split_mode, int len_cap) {
    constexpr int PER = D / 32;  // output columns per lane
    const int lane = threadIdx.x & 63;
    const int hl = lane & 31;
    const int r0 = 2 * (blockIdx.x * kCombineWaves + (threadIdx.x >> 6));
    if (r0 >= rows) return;  // a whole wave (rows is even): no barrier follows
    const int r = r0 + (lane >> 5);
    const int b = r0 / hq;
    const int64_t base = (int64_t)r * s_max;
    const int64_t orow = (int64_t)r * D;
    const float m_first = hl < s_max ? ws_ml[(base + hl) * 2] : neg_inf();
    const int S = combine_split_count(seq_lens, b, chunk, s_max, split_mode, len_cap);
    if (S == 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e) store_out<OUT>(out, orow + hl * PER + e, 0.f);
        if (lse && hl == 0) lse[r] = neg_inf();
        return;
    }
    float M = hl < S ? m_first : neg_inf();
    for (int i = hl + 32; i < S; i += 32) M = fmaxf(M, ws_ml[(base + i) * 2]);
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float l = 0.f;
#pragma unroll 8
    for (int i = 0; i < S; ++i) {
        const float w = __builtin_amdgcn_exp2f((ws_ml[(base + i) * 2] - M) * kLog2e);
        l = fmaf(w, ws_ml[(base + i) * 2 + 1], l);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, ws_o[(base + i) * D + hl * PER + e], acc[e]);
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < PER; ++e) store_out<OUT>(out, orow + hl * PER + e, acc[e] * inv);
    if (lse && hl == 0) lse[r] = M + __builtin_amdgcn_logf(l) * kLn2;
}

// NW waves per (sequence, query row): grid (hq, B). Four for most batches
// under kCombinePerWaveRows rows; sixteen when such a batch has many splits
// per row (a 128K-token cache cut into hundreds of splits), whose sums would
// otherwise be a long chain of loads for each of four waves.
template <int D, int OUT, int NW = kCombineWaves>
__global__ __launch_bounds__(64 * NW) void combine(const float* __restrict__ ws_o,
                                                              const float* __restrict__ ws_ml,
                                                              const int32_t* __restrict__ seq_lens,
                                                              void* __restrict__ out, float* __restrict__ lse, int hq,
                                                              int chunk, int s_max, int split_mode, int len_cap) {
    constexpr int PER = D / 64;  // output columns per lane
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t base = ((int64_t)b * hq + h) * s_max;
    const int64_t orow = ((int64_t)b * hq + h) * D;
    // Every wave takes M = max_s m_s over all splits by itself (no barrier);
    // the first 64 slots' m_s are read while the split count is worked out
    // (slots past it exist and are masked).
    const float m_first = lane < s_max ? ws_ml[(base + lane) * 2] : neg_inf();
    const int S = combine_split_count(seq_lens, b, chunk, s_max, split_mode, len_cap);
    if (S == 0) {
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < PER; ++e) store_out<OUT>(out, orow + lane * PER + e, 0.f);
            if (lse && lane == 0) lse[(int64_t)b * hq + h] = neg_inf();
        }
        return;
    }
    __shared__ float red_l[NW];
    __shared__ float red_o[NW][D];

    float M = lane < S ? m_first : neg_inf();
    for (int i = lane + 64; i < S; i += 64) M = fmaxf(M, ws_ml[(base + i) * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

    // Wave w takes splits w, w + NW, ...; loads of eight splits in flight.
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float lsum = 0.f;
#pragma unroll 8
    for (int i = wave; i < S; i += NW) {
        const float ms = ws_ml[(base + i) * 2];
        const float ls = ws_ml[(base + i) * 2 + 1];
        const float w = __builtin_amdgcn_exp2f((ms - M) * kLog2e);
        lsum = fmaf(w, ls, lsum);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, ws_o[(base + i) * D + lane * PER + e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) red_o[wave][lane * PER + e] = acc[e];
    if (lane == 0) red_l[wave] = lsum;
    __syncthreads();
    if (wave == 0) {
        float l = red_l[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) l += red_l[w];
        const float inv = 1.0f / l;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            float o = red_o[0][lane * PER + e];
#pragma unroll
            for (int w = 1; w < NW; ++w) o += red_o[w][lane * PER + e];
            store_out<OUT>(out, orow + lane * PER + e, o * inv);
        }
        if (lse && lane == 0) lse[(int64_t)b * hq + h] = M + __builtin_amdgcn_logf(l) * kLn2;
    }
}

template <int D, int OUT>
void launch_combine_out(int form, const float* ws_o, const float* ws_ml, const int32_t* lens, void* out,
                        float* lse, int B, int hq, int chunk, int s_max, int split_mode, int len_cap,
                        hipStream_t st) {
    if (form == 2) {
        const int rows = B * hq;
        const int waves = rows / 2;
        hipLaunchKernelGGL((combine_rows2<D, OUT>), dim3((waves + kCombineWaves - 1) / kCombineWaves),
                           dim3(64 * kCombineWaves), 0, st, ws_o, ws_ml, lens, out, lse, rows, hq, chunk, s_max,
                           split_mode, len_cap);
    } else if (form == 1) {
        const int rows = B * hq;
        hipLaunchKernelGGL((combine_rows<D, OUT>), dim3((rows + kCombineWaves - 1) / kCombineWaves),
                           dim3(64 * kCombineWaves), 0, st, ws_o, ws_ml, lens, out, lse, rows, hq, chunk, s_max,
                           split_mode, len_cap);
    } else if (form == 3) {
        hipLaunchKernelGGL((combine<D, OUT, 16>), dim3(hq, B), dim3(64 * 16), 0, st, ws_o, ws_ml, lens, out, lse, hq,
                           chunk, s_max, split_mode, len_cap);
    } else {
        hipLaunchKernelGGL((combine<D, OUT>), dim3(hq, B), dim3(64 * kCombineWaves), 0, st, ws_o, ws_ml, lens, out,
                           lse, hq, chunk, s_max, split_mode, len_cap);
    }
}

template <int D>
hipError_t launch_combine_d(int form, int out_dt, const float* ws_o, const float* ws_ml, const int32_t* lens,
                            void* out, float* lse, int B, int hq, int chunk, int s_max, int split_mode, int len_cap,
                            hipStream_t st) {
    switch (out_dt) {
        case FD_F32:
            launch_combine_out<D, FD_F32>(form, ws_o, ws_ml, lens, out, lse, B, hq, chunk, s_max, split_mode,
                                          len_cap, st);
            break;
        case FD_F16:
            launch_combine_out<D, FD_F16>(form, ws_o, ws_ml, lens, out, lse, B, hq, chunk, s_max, split_mode,
                                          len_cap, st);
            break;
        default:
            launch_combine_out<D, FD_BF16>(form, ws_o, ws_ml, lens, out, lse, B, hq, chunk, s_max, split_mode,
                                           len_cap, st);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_combine(int D, int out_dt, const float* ws_o, const float* ws_ml, const int32_t* lens,
                          void* out, float* lse, int B, int hq, int chunk, int s_max, int split_mode,
                          int len_cap, int form, hipStream_t st) {
    return D == 64 ? launch_combine_d<64>(form, out_dt, ws_o, ws_ml, lens, out, lse, B, hq, chunk, s_max,
                                          split_mode, len_cap, st)
                   : launch_combine_d<128>(form, out_dt, ws_o, ws_ml, lens, out, lse, B, hq, chunk, s_max,
                                           split_mode, len_cap, st);
}

}  // namespace fdk
