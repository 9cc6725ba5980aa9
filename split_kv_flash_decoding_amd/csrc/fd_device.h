// Device-side helpers shared by the decode kernels (gfx950 / CDNA4), and the
// launcher interface between the kernel files and the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fdk {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Compile-time tuning knobs of the partial kernel (defaults are the measured
// best on MI355X): 16-byte loads of K (and of V) per wave stage, waves per
// work-group, and whether K/V loads carry the non-temporal hint.
#ifndef FD_PARTIAL_UNROLL
#define FD_PARTIAL_UNROLL 4
#endif
#ifndef FD_PARTIAL_WAVES
#define FD_PARTIAL_WAVES 4
#endif
#ifndef FD_PARTIAL_NT
#define FD_PARTIAL_NT 1
#endif

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kWaves = FD_PARTIAL_WAVES;  // waves per partial work-group
constexpr int kThreads = 64 * kWaves;
constexpr int kUnroll = FD_PARTIAL_UNROLL;

__device__ __forceinline__ u32x4 load16(const void* p) {
#if FD_PARTIAL_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
    return *reinterpret_cast<const u32x4*>(p);
#endif
}

// Cache policy of streaming buffer loads: the non-temporal bit (every K/V byte
// is read once).
constexpr int kBufferLoadPolicy = FD_PARTIAL_NT ? 2 : 0;
// Third descriptor word of a raw (unformatted, stride 0) buffer on CDNA.
constexpr int kBufferRsrcWord3 = 0x00020000;

// A raw buffer over [base, base + bytes): 16-byte loads at offsets at or past
// `bytes` return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferRsrcWord3);
}

template <int POLICY = kBufferLoadPolicy>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_offset) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, POLICY));
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// A page index read from a block table, checked against the pool when its
// size is known (num_pages > 0): an index outside [0, num_pages) reads page 0
// instead, so a bad table gives wrong numbers but never an access outside the
// pool.
__device__ __forceinline__ int checked_page(int page, int num_pages) {
    return (num_pages > 0 && (unsigned)page >= (unsigned)num_pages) ? 0 : page;
}

// Reinterpret one 32-bit word as two 16-bit floats. The word is taken by value:
// bit-casting an element of an ext_vector_type in place reads element 0 for
// every index with this compiler.
__device__ __forceinline__ half2_t as_half2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ bf162_t as_bf162(uint32_t w) { return __builtin_bit_cast(bf162_t, w); }

// ---------------------------------------------------------------- element ops

template <int DT> struct Elt;

template <> struct Elt<FD_F16> {
    // sum_i a[i] * b[i] over 8 fp16 pairs, accumulated in fp32
    static __device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2(as_half2(a[i]), as_half2(b[i]), acc, false);
        return acc;
    }
    static __device__ __forceinline__ void to_f32(u32x4 x, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half2_t h = as_half2(x[i]);
            f[2 * i] = (float)h.x;
            f[2 * i + 1] = (float)h.y;
        }
    }
};

template <> struct Elt<FD_BF16> {
    static __device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(a[i]), as_bf162(b[i]), acc, false);
        return acc;
    }
    static __device__ __forceinline__ void to_f32(u32x4 x, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(x[i] << 16);
            f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
        }
    }
};

// One 16-byte load of the cache, by cache element type KT and query type QT:
// how many elements it holds, their dot product with this lane's query slice
// (kQWords 16-byte words of QT) accumulated in fp32, and their fp32 values.
template <int KT, int QT> struct KvLoad;

template <int DT> struct KvLoad<DT, DT> {
    static constexpr int kElems = 8;
    static constexpr int kQWords = 1;
    static __device__ __forceinline__ float dot(const u32x4* q, u32x4 k) { return Elt<DT>::dot8(q[0], k); }
    static __device__ __forceinline__ void to_f32(u32x4 x, float* f) { Elt<DT>::to_f32(x, f); }
};

// OCP E4M3 codes (16 per load). Two codes at a time widen exactly to a
// 16-bit pair (v_cvt_scalef32_pk_{f16,bf16}_fp8 with a unit scale) for the
// packed dot product, or to two floats (v_cvt_pk_f32_fp8); on gfx950 both
// decode every E4M3 code exactly (checked over all 256 codes on MI355X).
// Word i of a load holds codes 4i .. 4i+3, lowest byte first.
template <int QT> struct KvLoad<FD_FP8_E4M3, QT> {
    static constexpr int kElems = 16;
    static constexpr int kQWords = 2;
    static __device__ __forceinline__ float dot(const u32x4* q, u32x4 k) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = k[i];
            const uint32_t q0 = q[i >> 1][2 * (i & 1)];
            const uint32_t q1 = q[i >> 1][2 * (i & 1) + 1];
            if constexpr (QT == FD_F16) {
                acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, false), as_half2(q0),
                                             acc, false);
                acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, true), as_half2(q1),
                                             acc, false);
            } else {
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false),
                                                      as_bf162(q0), acc, false);
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true),
                                                      as_bf162(q1), acc, false);
            }
        }
        return acc;
    }
    static __device__ __forceinline__ void to_f32(u32x4 x, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = x[i];
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
            f[4 * i] = lo[0];
            f[4 * i + 1] = lo[1];
            f[4 * i + 2] = hi[0];
            f[4 * i + 3] = hi[1];
        }
    }
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of LPR lanes (LPR in {4, 8, 16}); every lane of
// the group receives the sum.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "row width");
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (LPR == 4) return x;
    x += dpp_mov<0x141>(x);  // row_half_mirror: the other quad of the 8
    if constexpr (LPR == 16) x += dpp_mov<0x140>(x);  // row_mirror: the other 8 of the 16
    return x;
}

// Max and sum over the four lane groups l, l ^ 16, l ^ 32 and l ^ 48 (every
// lane receives the result), with gfx950's row swaps (v_permlane16_swap,
// v_permlane32_swap: the odd 16- or 32-lane rows of one operand trade places
// with the even rows of the other; given one value twice, each lane ends up
// with its own value and its partner's) instead of two LDS shuffles.
__device__ __forceinline__ float max_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Merge running statistics (m, l, o) with another set, all in log2 units.
template <int N>
__device__ __forceinline__ void merge_stats(float& m, float& l, float* o, float m2, float l2,
                                            const float* o2) {
    const float mn = fmaxf(m, m2);
    const float mu = (mn == neg_inf()) ? 0.f : mn;
    const float a = __builtin_amdgcn_exp2f(m - mu);
    const float b = __builtin_amdgcn_exp2f(m2 - mu);
    l = l * a + l2 * b;
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = o[e] * a + o2[e] * b;
    m = mn;
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active).
__device__ __forceinline__ int64_t wave_incl_scan(int64_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

// A wave-uniform value moved to scalar registers (values that come out of
// wave shuffles are otherwise kept per lane).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(x & 0xffffffff)));
}

// One work-group's share of a partial kernel: KV head g of split s of
// sequence b, tokens [t0, t1); row0 is the sequence's first row in a packed
// contiguous cache.
struct WorkUnit {
    int b, g, s, t0, t1, L;
    int64_t row0;
};

// The partial kernels' work list, one work-group per entry: entry u is KV
// head u % hkv of work item u / hkv. Items 0..F-1 are the splits that hold a
// full chunk of tokens, in (sequence, split) order; items F.. are the shorter
// last splits, one per sequence whose length is not a multiple of the chunk,
// in sequence order. The hardware dispatches work-groups in index order, so
// every full-size unit starts before any short one (longest-first list
// scheduling), and the grid holds no empty work-groups. Each wave computes
// the lookup by itself from the device lengths (two wave-wide passes over
// seq_lens). Returns false for an entry past the end of the list.
__device__ inline bool locate_unit(int u, const int32_t* __restrict__ seq_lens, int B, int hkv, int chunk,
                                   int len_cap, WorkUnit& out) {
    const int lane = threadIdx.x & 63;
    const int g = u % hkv;
    const int64_t w = u / hkv;
    int64_t F = 0;
    for (int base = 0; base < B; base += 64) {
        const int i = base + lane;
        const int L = i < B ? max(0, min(seq_lens[i], len_cap)) : 0;
        int64_t f = L / chunk;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) f += __shfl_xor(f, off);
        F += f;
    }
    const bool full = w < F;
    const int64_t target = full ? w : w - F;
    int64_t acc = 0, racc = 0;
    for (int base = 0; base < B; base += 64) {
        const int i = base + lane;
        const int L = i < B ? max(0, min(seq_lens[i], len_cap)) : 0;
        const int cnt = full ? L / chunk : (L % chunk != 0 ? 1 : 0);
        const int64_t incl = wave_incl_scan(cnt);
        const int64_t lincl = wave_incl_scan(L);
        const int64_t total = __shfl(incl, 63);
        if (target < acc + total) {
            const unsigned long long mask = __ballot(acc + incl > target);
            const int j = __builtin_ctzll(mask);
            const int64_t incl_j = __shfl(incl, j);
            const int cnt_j = __shfl(cnt, j);
            const int L_j = __shfl(L, j);
            out.b = uniform(base + j);
            out.g = uniform(g);
            out.s = uniform(full ? (int)(target - (acc + incl_j - cnt_j)) : L_j / chunk);
            out.t0 = out.s * chunk;
            out.L = uniform(L_j);
            out.t1 = min(out.t0 + chunk, out.L);
            out.row0 = uniform(racc + __shfl(lincl, j) - L_j);
            return true;
        }
        acc += total;
        racc += __shfl(lincl, 63);
    }
    return false;
}

// Every field through a scalar register (the lookups below end in branches
// that the compiler cannot prove wave-uniform).
__device__ __forceinline__ void uniform_unit(WorkUnit& u) {
    u.b = uniform(u.b);
    u.g = uniform(u.g);
    u.s = uniform(u.s);
    u.t0 = uniform(u.t0);
    u.t1 = uniform(u.t1);
    u.L = uniform(u.L);
    u.row0 = uniform(u.row0);
}

// Tiles of a sequence of L tokens: 16-token tiles (a paged cache's pages).
__device__ __forceinline__ int seq_tiles(int L) { return (L + 15) >> 4; }

// Positions a sequence of n tiles takes in the balanced list: its tiles after
// kShareCost positions that stand for the cost of starting a share; none when
// empty.
__device__ __forceinline__ int64_t seq_positions(int n) { return n > 0 ? n + fd::kShareCost : 0; }

// Split count of a sequence whose n tiles start at position T of the
// balanced list (below), with P positions per work item: the items that hold
// any of its tiles. 0 for an empty sequence.
__device__ __forceinline__ int balanced_splits(int64_t T, int n, int P) {
    return n > 0 ? (int)((T + n - 1) / P - T / P + 1) : 0;
}

// Balanced work list (plan split mode 1): the sequences, in order, take
// consecutive positions of one list, kShareCost positions and then one per
// 16-token tile each, and work item w takes positions [w P, (w + 1) P) of it,
// across sequence boundaries, so every work-group of a ragged batch has the
// same work. Item w holds a share of sequence b when it holds one of b's
// tiles; that share is split s = w - floor(T_b / P) of b, where T_b is the
// position of the sequence's first tile. The cursor walks the sequences an
// item touches.
struct BalancedCursor {
    int64_t lo, hi;  // the item's positions [lo, hi)
    int64_t U;       // first position of sequence b (its share cost, then its tiles)
    int64_t row0;    // first row of sequence b in a packed contiguous cache
    int b;
};

// Fills wu (and S, the sequence's split count) with the share of the item in
// the cursor's sequence, skipping empty sequences. False once the item holds
// no more tiles.
__device__ inline bool balanced_share(const int32_t* __restrict__ seq_lens, int B, int P, int len_cap, int g,
                                      BalancedCursor& c, WorkUnit& wu, int& S) {
    while (c.b < B && c.U + fd::kShareCost < c.hi) {
        const int L = max(0, min(seq_lens[c.b], len_cap));
        const int n = seq_tiles(L);
        if (n > 0) {
            const int64_t T = c.U + fd::kShareCost;
            S = balanced_splits(T, n, P);
            wu.b = c.b;
            wu.g = g;
            wu.s = (int)(c.lo / P - T / P);
            wu.t0 = (int)(max(c.lo, T) - T) * 16;
            wu.t1 = min(L, (int)(min(c.hi, T + n) - T) * 16);
            wu.L = L;
            wu.row0 = c.row0;
            return true;
        }
        ++c.b;
    }
    return false;
}

// Moves the cursor to the sequence after the current one.
__device__ inline void balanced_advance(const int32_t* __restrict__ seq_lens, int len_cap, BalancedCursor& c) {
    const int L = max(0, min(seq_lens[c.b], len_cap));
    c.U += seq_positions(seq_tiles(L));
    c.row0 += L;
    ++c.b;
}

// Starts the cursor of work item w at the first sequence whose tiles reach
// into the item (two wave-wide scans over seq_lens per 64 sequences). False
// for an item past the end of the list.
__device__ inline bool balanced_first(int64_t w, const int32_t* __restrict__ seq_lens, int B, int P, int len_cap,
                                      BalancedCursor& c) {
    const int lane = threadIdx.x & 63;
    c.lo = w * P;
    c.hi = c.lo + P;
    int64_t accU = 0, accR = 0;
    for (int base = 0; base < B; base += 64) {
        const int i = base + lane;
        const int L = i < B ? max(0, min(seq_lens[i], len_cap)) : 0;
        const int64_t u = seq_positions(seq_tiles(L));
        const int64_t inclU = wave_incl_scan(u);
        const int64_t inclL = wave_incl_scan(L);
        const int64_t totalU = __shfl(inclU, 63);
        if (c.lo < accU + totalU) {
            // the first sequence whose positions end past lo (its tiles end there)
            const int j = __builtin_ctzll(__ballot(accU + inclU > c.lo));
            c.b = uniform(base + j);
            c.U = uniform(accU + __shfl(inclU, j) - __shfl(u, j));
            c.row0 = uniform(accR + __shfl(inclL, j) - __shfl(L, j));
            return true;
        }
        accU += totalU;
        accR += __shfl(inclL, 63);
    }
    return false;
}

// Arguments every partial kernel takes. q is 16-bit (q_dt); k and v hold
// kv_dt elements; k_scale / v_scale are per-KV-head factors or NULL (1).
struct PartialArgs {
    const uint16_t* q;
    const void* k;
    const void* v;
    const float* k_scale;
    const float* v_scale;
    const int32_t* table;
    const int32_t* lens;
    float* ws_o;
    float* ws_ml;
    int batch, hq, hkv, chunk, s_max, max_pages, q_len;
    // 0: split s of a sequence holds tokens [s chunk, (s + 1) chunk) (work
    // list of locate_unit); 1: balanced list, chunk = 16 * tiles per item
    // (BalancedCursor; matrix-core kernel only).
    int split_mode;
    float qk_scale_log2;
    int kv_dt, q_dt;
    int num_pages;  // pool size of a paged cache (0: indices not checked)
    // Fused merge (fd_decode_fused): per-(sequence, KV head) arrival counters,
    // zero between calls, and the outputs. counters == nullptr: partials only.
    uint32_t* counters;
    void* out;
    float* lse;
    int out_dt;
};

// Scale of KV head g (1 when no scales are given).
__device__ __forceinline__ float head_scale(const float* __restrict__ sc, int g) { return sc ? sc[g] : 1.f; }

// Store one output element in the output type (round to nearest even).
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
// The same with the output type chosen at run time.
__device__ __forceinline__ void store_out_dt(int dt, void* out, int64_t i, float x) {
    if (dt == FD_F32)
        store_out<FD_F32>(out, i, x);
    else if (dt == FD_F16)
        store_out<FD_F16>(out, i, x);
    else
        store_out<FD_BF16>(out, i, x);
}

// Arguments of the prefill kernel (fd_prefill_attention).
struct PrefillArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* table;
    const int32_t* lens;
    void* out;
    float* lse;
    int batch, hq, hkv, q_len, max_pages;
    float qk_scale_log2;
    int num_pages;  // pool size of a paged cache (0: indices not checked)
};

// Arguments of the KV-append kernel (fd_append_kv).
struct AppendArgs {
    const void* k_new;
    const void* v_new;
    void* q;
    const float* k_scale;
    const float* v_scale;
    void* k_cache;
    void* v_cache;
    const int32_t* table;
    const int32_t* lens;
    int n, hkv, hq, d, max_pages, num_pages, style;
    float rope_base;
    double inv_freq[64];  // base^(-2i/d) for pair i < d/2 (RoPE)
};

// Launchers (each defined in the file that holds its kernel). They enqueue on
// `st` and return hipGetLastError().
hipError_t launch_partial_valu(int D, int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st);
hipError_t launch_partial_valu_heads(int D, int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st);
hipError_t launch_partial_valu_head_cols(int D, int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st);
hipError_t launch_partial_mfma(int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st);
hipError_t launch_partial_mfma_heads(int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, int q_dt, int kv_dt, int blocks, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, int dt, int out_dt, bool paged, hipStream_t st);
// form: 0 four waves per (sequence, query row), 1 one wave per row, 2 two rows
// per wave (rows per sequence even), 3 sixteen waves per row.
hipError_t launch_combine(int D, int out_dt, const float* ws_o, const float* ws_ml, const int32_t* lens,
                          void* out, float* lse, int B, int hq, int chunk, int s_max, int split_mode,
                          int len_cap, int form, hipStream_t st);

// ------------------------------------------------------------ fused merge

// The combine step run by a partial kernel's own last work-group
// (fd_decode_fused). Every work-group of a (sequence, head group) calls this
// after writing its split's (O, m, l): it makes those writes visible and bumps
// the group's arrival counter; the work-group whose arrival completes the
// count (splits x `tiles` column tiles) merges every split of the group's
// `nrows` rows, ROWS at a time, exactly as the combine kernel does
// (FlashAttention capstone §2.3 cross-chunk reduce), and sets the counter back
// to zero for the next call. No work-group waits for another. S: the
// sequence's split count under the plan's split mode. Rows:
// r = i * (nkv * G) + k for query token i and head k of the group, i.e.
// query row i * Hq + g0 * G + k. `red` is the caller's wave-merge LDS buffer,
// at least NW * ROWS * D floats for NW waves per work-group.
template <int D, int ROWS, int NW>
__device__ void fused_merge(const PartialArgs& a, int b, int S, int g0, int nkv, int nrows, int tiles, float* red) {
    constexpr int PER = D / 64;
    __shared__ int s_last;
    __shared__ float s_max[ROWS];
    __shared__ float s_l[NW][ROWS];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this work-group's partials, visible device-wide
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(a.counters + (int64_t)b * a.hkv + g0, 1u);
        s_last = (prev + 1 == (unsigned)(S * tiles));
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other work-groups' partials, not stale cache lines
    // Lane indices kept opaque: a caller that loops over several splits would
    // otherwise get this merge's lane-derived addresses hoisted out of its loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));

    const int G = a.hq / a.hkv;
    const int R = a.q_len * a.hq;
    const int per_tok = nkv * G;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    auto qrow_of = [&](int r) { return (r / per_tok) * a.hq + g0 * G + r % per_tok; };
    for (int r0 = 0; r0 < nrows; r0 += ROWS) {
        const int nr = min(ROWS, nrows - r0);
        // Row maxima: wave w takes rows w, w + NW, ...
        for (int r = wave; r < nr; r += NW) {
            const int64_t base = ((int64_t)b * R + qrow_of(r0 + r)) * a.s_max;
            float m = neg_inf();
            for (int s = lane; s < S; s += 64) m = fmaxf(m, a.ws_ml[(base + s) * 2]);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            if (lane == 0) s_max[r] = m;
        }
        __syncthreads();
        // Wave w sums splits w, w + NW, ... of every row.
        float acc[ROWS][PER], lsum[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            lsum[r] = 0.f;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[r][e] = 0.f;
        }
        for (int s = wave; s < S; s += NW) {
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                if (r < nr) {
                    const int64_t slot = ((int64_t)b * R + qrow_of(r0 + r)) * a.s_max + s;
                    const float w = __builtin_amdgcn_exp2f((a.ws_ml[slot * 2] - s_max[r]) * kLog2e);
                    lsum[r] = fmaf(w, a.ws_ml[slot * 2 + 1], lsum[r]);
#pragma unroll
                    for (int e = 0; e < PER; ++e)
                        acc[r][e] = fmaf(w, a.ws_o[slot * D + lane * PER + e], acc[r][e]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            if (r < nr) {
#pragma unroll
                for (int e = 0; e < PER; ++e) red[(wave * ROWS + r) * D + lane * PER + e] = acc[r][e];
                if (lane == 0) s_l[wave][r] = lsum[r];
            }
        }
        __syncthreads();
        for (int idx = tid; idx < nr * D; idx += blockDim.x) {
            const int r = idx / D, col = idx % D;
            float l = 0.f, o = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                l += s_l[w][r];
                o += red[(w * ROWS + r) * D + col];
            }
            const int64_t orow = (int64_t)b * R + qrow_of(r0 + r);
            store_out_dt(a.out_dt, a.out, orow * D + col, o / l);
            if (a.lse && col == 0) a.lse[orow] = s_max[r] + __builtin_amdgcn_logf(l) * kLn2;
        }
        __syncthreads();  // s_max, s_l and red are reused by the next batch of rows
    }
    if (threadIdx.x == 0) a.counters[(int64_t)b * a.hkv + g0] = 0u;  // ready for the next call
}

}  // namespace fdk
