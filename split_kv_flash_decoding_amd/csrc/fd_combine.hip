// Combine kernel: merges the per-split statistics of every (sequence, query
// head) into the output and its log-sum-exp. One wave per (b, h): the wave
// finds M = max_s m_s, then accumulates w_s = exp(m_s - M) times l_s and O_s;
// out = sum_s w_s O_s / sum_s w_s l_s, lse = M + ln(sum_s w_s l_s). This is
// the cross-chunk reduce of FlashDecoding ("FlashAttention 全景演进与大模型
// Token 生成全链路性能优化实战", §2.3), with every split rescaled by the
// two-block identity of the same page's §1.2.

#include "fd_device.h"

namespace fdk {

template <int OUT> __device__ __forceinline__ void store_out(void* out, int64_t i, float x);
template <> __device__ __forceinline__ void store_out<FD_F32>(void* out, int64_t i, float x) {
    reinterpret_cast<float*>(out)[i] = x;
}
template <> __device__ __forceinline__ void store_out<FD_F16>(void* out, int64_t i, float x) {
    reinterpret_cast<_Float16*>(out)[i] = (_Float16)x;
}
template <> __device__ __forceinline__ void store_out<FD_BF16>(void* out, int64_t i, float x) {
    reinterpret_cast<__bf16*>(out)[i] = (__bf16)x;
}

template <int D, int OUT>
__global__ __launch_bounds__(64) void combine(const float* __restrict__ ws_o,
                                              const float* __restrict__ ws_ml,
                                              const int32_t* __restrict__ seq_lens, void* __restrict__ out,
                                              float* __restrict__ lse, int hq, int chunk, int s_max) {
    constexpr int PER = D / 64;  // output columns per lane
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int L = seq_lens[b];
    const int S = L > 0 ? min((L + chunk - 1) / chunk, s_max) : 0;
    const int64_t base = ((int64_t)b * hq + h) * s_max;
    const int64_t orow = ((int64_t)b * hq + h) * D;
    if (S == 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e) store_out<OUT>(out, orow + lane * PER + e, 0.f);
        if (lse && lane == 0) lse[(int64_t)b * hq + h] = neg_inf();
        return;
    }
    float M = neg_inf();
    for (int i = lane; i < S; i += 64) M = fmaxf(M, ws_ml[(base + i) * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float lsum = 0.f;
#pragma unroll 4
    for (int i = 0; i < S; ++i) {
        const float ms = ws_ml[(base + i) * 2];
        const float ls = ws_ml[(base + i) * 2 + 1];
        const float w = __builtin_amdgcn_exp2f((ms - M) * kLog2e);
        lsum = fmaf(w, ls, lsum);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, ws_o[(base + i) * D + lane * PER + e], acc[e]);
    }
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < PER; ++e) store_out<OUT>(out, orow + lane * PER + e, acc[e] * inv);
    if (lse && lane == 0) lse[(int64_t)b * hq + h] = M + __builtin_amdgcn_logf(lsum) * kLn2;
}

template <int D>
hipError_t launch_combine_d(int out_dt, const float* ws_o, const float* ws_ml, const int32_t* lens, void* out,
                          float* lse, int B, int hq, int chunk, int s_max, hipStream_t st) {
    dim3 grid(hq, B);
    switch (out_dt) {
        case FD_F32:
            hipLaunchKernelGGL((combine<D, FD_F32>), grid, dim3(64), 0, st, ws_o, ws_ml, lens, out, lse, hq, chunk, s_max);
            break;
        case FD_F16:
            hipLaunchKernelGGL((combine<D, FD_F16>), grid, dim3(64), 0, st, ws_o, ws_ml, lens, out, lse, hq, chunk, s_max);
            break;
        default:
            hipLaunchKernelGGL((combine<D, FD_BF16>), grid, dim3(64), 0, st, ws_o, ws_ml, lens, out, lse, hq, chunk, s_max);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_combine(int D, int out_dt, const float* ws_o, const float* ws_ml, const int32_t* lens,
                          void* out, float* lse, int B, int hq, int chunk, int s_max, hipStream_t st) {
    return D == 64 ? launch_combine_d<64>(out_dt, ws_o, ws_ml, lens, out, lse, B, hq, chunk, s_max, st)
                   : launch_combine_d<128>(out_dt, ws_o, ws_ml, lens, out, lse, B, hq, chunk, s_max, st);
}

}  // namespace fdk
