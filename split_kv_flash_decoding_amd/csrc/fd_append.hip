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
// format, ties to even; an FP8 cache stores the E4M3 code of value / scale[g],
// saturated at 448.
//
// One work-group per (sequence, new token); its threads take items: 16-byte
// pieces of the head rows (8 elements; in the half pairing a piece of the
// first half together with its partner piece of the second half), so each K,
// V and q row is read and written with whole, coalesced 16-byte accesses.
// The loads of a thread's first items go out before anything else, since
// they depend on nothing but the token; while they are in flight the
// position is read, the page looked up and the token's d/2 sines and cosines
// computed once into LDS. It writes nothing for a position outside the block
// table or a page index outside [0, num_pages).

#include "fd_device.h"

namespace fdk {

namespace {

// N (4 or 8) 16-bit values of a piece (8 or 16 bytes), widened exactly to fp64.
template <int DT, int N>
__device__ __forceinline__ void widen(u32x4 w, double* x) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const uint16_t h = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
        if constexpr (DT == FD_F16)
            x[e] = (double)__builtin_bit_cast(_Float16, h);
        else
            x[e] = (double)__builtin_bit_cast(float, (uint32_t)h << 16);
    }
}

// The nearest value of a binary format with `mbits` stored mantissa bits and
// smallest normal exponent `emin` (ties to even; subnormals included): v is
// scaled by a power of two so that the format's unit in the last place is 1,
// rounded to an integer by rint (ties to even) and scaled back; both scalings
// are exact. Past `fmax`: +-inf, or +-fmax when `saturate`.
__device__ __forceinline__ double round_to_format(double v, int mbits, int emin, double fmax, bool saturate) {
    if (!(v == v) || v == 0.0 || __builtin_isinf(v)) return v;
    const int e = max(__builtin_amdgcn_frexp_exp(v) - 1, emin);  // v's binade (subnormals share emin)
    double out = ldexp(rint(ldexp(v, mbits - e)), e - mbits);     // rint keeps the sign of a tiny v
    if (fabs(out) > fmax) out = copysign(saturate ? fmax : __builtin_inf(), v);
    return out;
}

// The E4M3 code of a value E4M3 represents exactly (|x| <= 448).
__device__ __forceinline__ uint32_t e4m3_encode(double x) {
    const uint32_t sign = signbit(x) ? 0x80u : 0u;
    const double a = fabs(x);
    if (a < 0x1p-6) return sign | (uint32_t)(a * 512.0);  // subnormals: a / 2^-9
    const int e = __builtin_amdgcn_frexp_exp(a) - 1;
    const uint32_t mant = (uint32_t)((ldexp(a, -e) - 1.0) * 8.0);
    return sign | ((uint32_t)(e + 7) << 3) | mant;
}

// v rounded to fp32 with round-to-odd: the truncation toward zero, its last
// bit set when v was not exact. fp32 keeps at least two more bits than fp16
// and bf16, so rounding this to nearest-even in either gives what one
// rounding of v itself gives (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", 2008).
// No special cases are needed: an exact v (infinities included) comes back
// unchanged; a v past fp32's range rounds to infinity, steps back to the
// largest finite fp32 with its last bit already set, and that rounds to
// infinity again in either 16-bit format, as v itself does; a NaN stays a
// NaN.
__device__ __forceinline__ float round_to_odd_f32(double v) {
    const float f = (float)v;  // nearest, ties to even
    const double back = (double)f;
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u -= (fabs(back) > fabs(v)) ? 1u : 0u;  // rounded away from zero: one step back
    u |= (back != v) ? 1u : 0u;             // inexact: the sticky bit
    return __builtin_bit_cast(float, u);
}

// N (4 or 8) fp64 values rounded once to the storage format DT and stored as
// one piece (2N bytes; N bytes of E4M3 codes).
template <int DT, int N>
__device__ __forceinline__ void store(void* base, int64_t elem, const double* x) {
    if constexpr (DT == FD_FP8_E4M3) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < N; ++e) w[e / 4] |= e4m3_encode(round_to_format(x[e], 3, -6, 448.0, true)) << (8 * (e % 4));
        uint8_t* dst = static_cast<uint8_t*>(base) + elem;
        if constexpr (N == 8)
            *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
        else
            *reinterpret_cast<uint32_t*>(dst) = w[0];
    } else {
        // Two values per conversion instruction (nearest even, element 2i in
        // the low half).
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < N; e += 2) {
            const f32x2_t f = {round_to_odd_f32(x[e]), round_to_odd_f32(x[e + 1])};
            if constexpr (DT == FD_F16)
                w[e / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, half2_t));
            else
                w[e / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
        }
        uint16_t* dst = static_cast<uint16_t*>(base) + elem;
        if constexpr (N == 8)
            *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
        else
            *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    }
}

// sin and cos of x in fp64 for |x| up to ~2^40: x = k pi/2 + r with |r| <=
// pi/4 by Cody and Waite's additive reduction (pi/2 held as a sum of three
// doubles, each step one fused multiply-add, the first exact), then the
// Taylor series of sin and cos at r through r^21 and r^22 (the next terms are
// below 2^-60 for |r| <= pi/4), and the quadrant k mod 4. Within about an
// ulp of the correctly rounded values; written out here instead of calling
// the math library's sincos, whose large-argument path holds enough
// registers to halve this kernel's occupancy.
__device__ __forceinline__ void sincos_f64(double x, double& s, double& c) {
    const double k = rint(x * 0x1.45f306dc9c883p-1);  // x * 2/pi
    double r = fma(-k, 0x1.921fb54442d18p+0, x);      // pi/2, first part
    r = fma(-k, 0x1.1a62633145c07p-54, r);            // second part
    r = fma(-k, -0x1.f1976b7ed8fbcp-110, r);          // third part
    const double r2 = r * r;
    // 1/n! for n = 2 .. 22, alternating signs folded in below.
    constexpr double f2 = 1.0 / 2, f3 = f2 / 3, f4 = f3 / 4, f5 = f4 / 5, f6 = f5 / 6, f7 = f6 / 7, f8 = f7 / 8,
                     f9 = f8 / 9, f10 = f9 / 10, f11 = f10 / 11, f12 = f11 / 12, f13 = f12 / 13, f14 = f13 / 14,
                     f15 = f14 / 15, f16 = f15 / 16, f17 = f16 / 17, f18 = f17 / 18, f19 = f18 / 19,
                     f20 = f19 / 20, f21 = f20 / 21, f22 = f21 / 22;
    double ps = -f21;
    ps = fma(ps, r2, f19);
    ps = fma(ps, r2, -f17);
    ps = fma(ps, r2, f15);
    ps = fma(ps, r2, -f13);
    ps = fma(ps, r2, f11);
    ps = fma(ps, r2, -f9);
    ps = fma(ps, r2, f7);
    ps = fma(ps, r2, -f5);
    ps = fma(ps, r2, f3);
    const double sn = fma(-ps * r2, r, r);  // r - r^3/3! + ...
    double pc = f22;
    pc = fma(pc, r2, -f20);
    pc = fma(pc, r2, f18);
    pc = fma(pc, r2, -f16);
    pc = fma(pc, r2, f14);
    pc = fma(pc, r2, -f12);
    pc = fma(pc, r2, f10);
    pc = fma(pc, r2, -f8);
    pc = fma(pc, r2, f6);
    pc = fma(pc, r2, -f4);
    pc = fma(pc, r2, f2);
    const double cs = fma(-pc, r2, 1.0);  // 1 - r^2/2! + ...
    switch ((int)((int64_t)k & 3)) {
        case 0: s = sn, c = cs; break;
        case 1: s = cs, c = -sn; break;
        case 2: s = -sn, c = -cs; break;
        default: s = -cs, c = sn; break;
    }
}

// (x_a, x_b) turned by the angle with cosine c and sine s, in fp64 with each
// product and sum rounded on its own (no fused multiply-adds).
__device__ __forceinline__ void rotate(double& xa, double& xb, double c, double s) {
#pragma clang fp contract(off)
    const double a = xa * c - xb * s;
    const double b = xa * s + xb * c;
    xa = a;
    xb = b;
}

}  // namespace

// QT: type of k_new, v_new and q (16-bit); KT: cache element type; STYLE: the
// RoPE pairing (fd_rope_style).
template <int QT, int KT, int STYLE>
__global__ __launch_bounds__(256) void append_kv(const AppendArgs a) {
    // Items a thread holds in registers at once (measured on MI355X: 2 to 4,
    // with the loads of all of them issued first, ran no faster than 1).
    constexpr int kNI = 1;
    __shared__ double s_cos[64], s_sin[64];  // the token's d/2 <= 64 angles
    const int b = blockIdx.x / a.n;
    const int j = blockIdx.x % a.n;
    const int64_t tok = (int64_t)b * a.n + j;
    const int d = a.d, half = d / 2;
    // Items: the q rows' (rotated in place), then the K rows' (rotated into
    // the cache), then the V rows' (into the cache); d/8 per row. A rotated
    // item is four pairs: elements 8p .. 8p+7 in the interleaved pairing (one
    // 16-byte piece), 4p .. 4p+3 and their partners 4p + d/2 .. +3 in the half
    // pairing (two 8-byte pieces); a V item is 8 elements.
    const int per_row = d / 8;
    const int row_shift = d == 128 ? 4 : 3;  // log2(per_row); d is 64 or 128
    const int nq = (STYLE != FD_ROPE_NONE && a.q) ? a.hq * per_row : 0;
    const int nk = a.hkv * per_row;
    const int total = nq + nk + a.hkv * per_row;
    const bool plain_v = KT == QT && !a.v_scale;  // V stored as given

    const int pos = a.lens[b] - a.n + j;
    int page = -1;
    for (int base = 0; base < total; base += kNI * 256) {
        u32x4 r0[kNI], r1[kNI];
        auto locate = [&](int idx, int& kind, int& h, int& p) {
            kind = idx < nq ? 0 : idx < nq + nk ? 1 : 2;
            const int k = idx - (kind == 0 ? 0 : kind == 1 ? nq : nq + nk);
            h = k >> row_shift, p = k & (per_row - 1);  // per_row is 8 or 16
        };
        auto src_of = [&](int kind, int h) -> const uint16_t* {
            const void* base_ptr = kind == 0 ? a.q : kind == 1 ? a.k_new : a.v_new;
            const int64_t row = kind == 0 ? tok * a.hq + h : tok * a.hkv + h;
            return static_cast<const uint16_t*>(base_ptr) + row * d;
        };
#pragma unroll
        for (int t = 0; t < kNI; ++t) {
            const int idx = base + t * 256 + (int)threadIdx.x;
            if (idx < total) {
                int kind, h, p;
                locate(idx, kind, h, p);
                const uint16_t* src = src_of(kind, h);
                if (STYLE == FD_ROPE_HALF && kind != 2) {
                    const uint2 lo = *reinterpret_cast<const uint2*>(src + 4 * p);
                    const uint2 hi = *reinterpret_cast<const uint2*>(src + 4 * p + half);
                    r0[t] = u32x4{lo.x, lo.y, 0u, 0u};
                    r1[t] = u32x4{hi.x, hi.y, 0u, 0u};
                } else {
                    r0[t] = *reinterpret_cast<const u32x4*>(src + 8 * p);
                }
            }
        }
        if (base == 0) {
            if (pos < 0 || pos >= a.max_pages * 16) return;  // the whole work-group
            page = a.table[(int64_t)b * a.max_pages + pos / 16];
            if (page >= a.num_pages) page = -1;
            if constexpr (STYLE != FD_ROPE_NONE) {
                for (int i = threadIdx.x; i < half; i += blockDim.x) {
                    // inv_freq[i] = base^(-2i/d), computed once per call on the host.
                    const double angle = (double)pos * a.inv_freq[i];
                    sincos_f64(angle, s_sin[i], s_cos[i]);
                }
                __syncthreads();
            }
        }
        const int64_t dst_row = ((int64_t)page * 16 + pos % 16) * a.hkv;  // cache row of head 0
#pragma unroll
        for (int t = 0; t < kNI; ++t) {
            const int idx = base + t * 256 + (int)threadIdx.x;
            if (idx >= total) continue;
            int kind, h, p;
            locate(idx, kind, h, p);
            if (kind != 0 && page < 0) continue;
            void* dst = kind == 0 ? a.q : kind == 1 ? a.k_cache : a.v_cache;
            const int64_t row = kind == 0 ? (tok * a.hq + h) * d : (dst_row + h) * d;
            if (kind == 2 && plain_v) {
                *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + row + 8 * p) = r0[t];
                continue;
            }
            const float* scales = kind == 1 ? a.k_scale : kind == 2 ? a.v_scale : nullptr;
            const double inv = scales ? (double)scales[h] : 1.0;
            if (STYLE == FD_ROPE_HALF && kind != 2) {
                double x[4], y[4];
                widen<QT, 4>(r0[t], x);
                widen<QT, 4>(r1[t], y);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rotate(x[e], y[e], s_cos[4 * p + e], s_sin[4 * p + e]);
                    if (inv != 1.0) x[e] = x[e] / inv, y[e] = y[e] / inv;
                }
                if (kind == 0) {
                    store<QT, 4>(dst, row + 4 * p, x);
                    store<QT, 4>(dst, row + 4 * p + half, y);
                } else {
                    store<KT, 4>(dst, row + 4 * p, x);
                    store<KT, 4>(dst, row + 4 * p + half, y);
                }
            } else {
                double x[8];
                widen<QT, 8>(r0[t], x);
                if (STYLE == FD_ROPE_INTERLEAVED && kind != 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rotate(x[2 * e], x[2 * e + 1], s_cos[4 * p + e], s_sin[4 * p + e]);
                }
                if (inv != 1.0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = x[e] / inv;
                }
                if (kind == 0)
                    store<QT, 8>(dst, row + 8 * p, x);
                else
                    store<KT, 8>(dst, row + 8 * p, x);
            }
        }
    }
}

template <int QT, int KT>
hipError_t launch_style(const AppendArgs& a, dim3 grid, hipStream_t st) {
    const dim3 block(256);
    if (a.style == FD_ROPE_INTERLEAVED)
        hipLaunchKernelGGL((append_kv<QT, KT, FD_ROPE_INTERLEAVED>), grid, block, 0, st, a);
    else if (a.style == FD_ROPE_HALF)
        hipLaunchKernelGGL((append_kv<QT, KT, FD_ROPE_HALF>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((append_kv<QT, KT, FD_ROPE_NONE>), grid, block, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int q_dt, int kv_dt, int blocks, hipStream_t st) {
    const dim3 grid(blocks);
    if (q_dt == FD_F16)
        return kv_dt == FD_FP8_E4M3 ? launch_style<FD_F16, FD_FP8_E4M3>(a, grid, st)
                                    : launch_style<FD_F16, FD_F16>(a, grid, st);
    return kv_dt == FD_FP8_E4M3 ? launch_style<FD_BF16, FD_FP8_E4M3>(a, grid, st)
                                : launch_style<FD_BF16, FD_BF16>(a, grid, st);
}

}  // namespace fdk
