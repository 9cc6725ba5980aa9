// KV append: a decode step's new tokens go into the paged cache, with rotary
// position embedding applied to the new keys and to the queries first.
//
// The CUTLASS Split KV article (§5.3) has RoPE applied to the current step's
// K and q by a separate kernel before split-KV decode reads the cache (the
// decode kernels read a cache that does not change while they run), and the
// FlashAttention capstone (§4.1) keeps the cache in 16-token physical blocks
// found through a per-request block table. New token j of sequence b (of n
// new tokens, lengths L_b counted after the append) sits at position
// L_b - n + j: block-table entry pos / 16, slot pos % 16.
//
// RoPE (RoFormer's rotary embedding; the pages name it without its formula):
// pair i of a head vector turns by pos * base^(-2i/d), pairs being dims
// (2i, 2i+1) (interleaved) or (i, i + d/2) (half). The angle, sine and cosine
// and the rotation are computed in fp64 (an fp32 angle at position 1e5 would
// be off by ~0.01 rad), then each result is rounded once to the storage
// format, ties to even, by exact power-of-two scaling and rint; an FP8 cache
// stores the E4M3 code of value / scale[g], saturated at 448.
//
// One work-group per (sequence, new token); its threads take (head, pair)
// items. The kernel moves a few hundred kilobytes per decode step and is
// latency-bound; it writes nothing for a position outside the block table or
// a page index outside [0, num_pages).

#include "fd_device.h"

namespace fdk {

namespace {

// The nearest value of a binary format with `mbits` stored mantissa bits and
// smallest normal exponent `emin` (ties to even; subnormals included). Past
// `fmax`: +-inf, or +-fmax when `saturate`.
__device__ double round_to_format(double v, int mbits, int emin, double fmax, bool saturate) {
    if (!(v == v) || v == 0.0 || __builtin_isinf(v)) return v;
    int E = 0;
    frexp(v, &E);
    const int e = max(E - 1, emin);
    const double quantum = ldexp(1.0, e - mbits);
    const double r = rint(v / quantum);  // exact quotient; rint rounds ties to even
    double out = copysign(r * quantum, v);
    if (fabs(out) > fmax) out = copysign(saturate ? fmax : __builtin_inf(), v);
    return out;
}

// The E4M3 code of a value E4M3 represents exactly (|x| <= 448).
__device__ uint8_t e4m3_encode(double x) {
    const uint32_t sign = signbit(x) ? 0x80u : 0u;
    const double a = fabs(x);
    if (a < 0x1p-6) return (uint8_t)(sign | (uint32_t)(a * 512.0));  // subnormals: a / 2^-9
    int E = 0;
    frexp(a, &E);
    const int e = E - 1;
    const uint32_t mant = (uint32_t)((ldexp(a, -e) - 1.0) * 8.0);
    return (uint8_t)(sign | ((uint32_t)(e + 7) << 3) | mant);
}

template <int DT> struct Store;
template <> struct Store<FD_F16> {
    static __device__ void put(void* base, int64_t i, double v) {
        static_cast<_Float16*>(base)[i] = (_Float16)(float)round_to_format(v, 10, -14, 65504.0, false);
    }
    static __device__ double get(const void* base, int64_t i) { return (double)static_cast<const _Float16*>(base)[i]; }
};
template <> struct Store<FD_BF16> {
    static __device__ void put(void* base, int64_t i, double v) {
        static_cast<__bf16*>(base)[i] = (__bf16)(float)round_to_format(v, 7, -126, 0x1.fep127, false);
    }
    static __device__ double get(const void* base, int64_t i) { return (double)(float)static_cast<const __bf16*>(base)[i]; }
};
template <> struct Store<FD_FP8_E4M3> {
    static __device__ void put(void* base, int64_t i, double v) {
        static_cast<uint8_t*>(base)[i] = e4m3_encode(round_to_format(v, 3, -6, 448.0, true));
    }
};

// (x_a, x_b) turned by `angle` (fp64, no fused multiply-adds, as written).
__device__ void rotate(double& xa, double& xb, double angle) {
#pragma clang fp contract(off)
    double s, c;
    sincos(angle, &s, &c);
    const double a = xa * c - xb * s;
    const double b = xa * s + xb * c;
    xa = a;
    xb = b;
}

}  // namespace

// QT: type of k_new, v_new and q (16-bit); KT: cache element type.
template <int QT, int KT>
__global__ __launch_bounds__(256) void append_kv(const AppendArgs a) {
    const int b = blockIdx.x / a.n;
    const int j = blockIdx.x % a.n;
    const int pos = a.lens[b] - a.n + j;
    if (pos < 0 || pos >= a.max_pages * 16) return;
    const int page = a.table[(int64_t)b * a.max_pages + pos / 16];
    const int d = a.d, half = d / 2;
    const double base = (double)a.rope_base;

    auto pair_dims = [&](int i, int& ia, int& ib) {
        if (a.style == FD_ROPE_INTERLEAVED) {
            ia = 2 * i;
            ib = 2 * i + 1;
        } else {
            ia = i;
            ib = i + half;
        }
    };
    auto angle = [&](int i) { return (double)pos * pow(base, -2.0 * i / d); };

    if (page >= 0 && page < a.num_pages) {
        const int64_t src_row = ((int64_t)b * a.n + j) * a.hkv;             // k_new / v_new row of head 0
        const int64_t dst_row = ((int64_t)page * 16 + pos % 16) * a.hkv;    // cache row of head 0
        for (int idx = threadIdx.x; idx < a.hkv * half; idx += blockDim.x) {
            const int g = idx / half, i = idx % half;
            int ia, ib;
            pair_dims(i, ia, ib);
            double xa = Store<QT>::get(a.k_new, (src_row + g) * d + ia);
            double xb = Store<QT>::get(a.k_new, (src_row + g) * d + ib);
            if (a.style != FD_ROPE_NONE) rotate(xa, xb, angle(i));
            const double inv = a.k_scale ? (double)a.k_scale[g] : 1.0;
            Store<KT>::put(a.k_cache, (dst_row + g) * d + ia, xa / inv);
            Store<KT>::put(a.k_cache, (dst_row + g) * d + ib, xb / inv);
        }
        for (int idx = threadIdx.x; idx < a.hkv * d; idx += blockDim.x) {
            const int g = idx / d;
            const double sc = a.v_scale ? (double)a.v_scale[g] : 1.0;
            Store<KT>::put(a.v_cache, dst_row * d + idx, Store<QT>::get(a.v_new, src_row * d + idx) / sc);
        }
    }
    if (a.q && a.style != FD_ROPE_NONE) {
        const int64_t q_row = ((int64_t)b * a.n + j) * a.hq;
        for (int idx = threadIdx.x; idx < a.hq * half; idx += blockDim.x) {
            const int h = idx / half, i = idx % half;
            int ia, ib;
            pair_dims(i, ia, ib);
            double xa = Store<QT>::get(a.q, (q_row + h) * d + ia);
            double xb = Store<QT>::get(a.q, (q_row + h) * d + ib);
            rotate(xa, xb, angle(i));
            Store<QT>::put(a.q, (q_row + h) * d + ia, xa);
            Store<QT>::put(a.q, (q_row + h) * d + ib, xb);
        }
    }
}

hipError_t launch_append(const AppendArgs& a, int q_dt, int kv_dt, int blocks, hipStream_t st) {
    const dim3 grid(blocks), block(256);
    if (q_dt == FD_F16) {
        if (kv_dt == FD_FP8_E4M3)
            hipLaunchKernelGGL((append_kv<FD_F16, FD_FP8_E4M3>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((append_kv<FD_F16, FD_F16>), grid, block, 0, st, a);
    } else {
        if (kv_dt == FD_FP8_E4M3)
            hipLaunchKernelGGL((append_kv<FD_BF16, FD_FP8_E4M3>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((append_kv<FD_BF16, FD_BF16>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace fdk
