// Split-KV decode attention kernels for gfx950 (CDNA4) and the C-ABI entry
// points that launch them.
//
// The method: a single query token per sequence attends over a long KV cache
// that is cut along the token axis into splits; every split computes its local
// softmax statistics (running max m, running sum l) and an unnormalised partial
// output, and a second small kernel merges the splits by log-sum-exp
// rescaling ("FlashAttention 全景演进与大模型 Token 生成全链路性能优化实战",
// §2.3 FlashDecoding; the merge identity is §1.2's formal proof; the tile
// recurrence is §2.2 of the lpnh.cn memory-wall article).
//
// Partial kernel, one work-group of four wave64s per (sequence, KV head,
// split):
//   * a token row of one KV head is d fp16/bf16 values = d/8 lanes x 16 bytes,
//     so one wave-wide 16-byte load covers 64/(d/8) consecutive tokens
//     (4 at d = 128, 8 at d = 64); each wave streams U such loads of K and U
//     of V per stage and issues the next stage's loads before it computes on
//     the current one (double buffering in registers: the data is used once,
//     so it never needs a trip through LDS);
//   * q.k is a packed fp16/bf16 dot product accumulating in fp32
//     (v_dot2_f32_f16 / v_dot2_f32_bf16) followed by a DPP butterfly across
//     the d/8 lanes of the row;
//   * each row of lanes keeps its own running max, sum and fp32 output slice
//     in registers (log2 domain: scores are pre-multiplied by scale*log2(e)
//     so every exponential is a hardware exp2);
//   * at the end the rows of a wave merge through lane shuffles, the four
//     waves merge through LDS, and the split's (O, m, l) go to the workspace.
// The query heads of one GQA group share every K/V load (G scores per row).
//
// Combine kernel: one wave per (sequence, query head) reads the split
// statistics and writes out = sum_s w_s O_s / sum_s w_s l_s and the LSE.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fdk {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kWaves = 4;          // waves per partial work-group
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

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

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of LPR lanes (LPR in {8, 16}); every lane of the
// group receives the sum.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror: the other quad of the 8
    if constexpr (LPR == 16) x += dpp_mov<0x140>(x);  // row_mirror: the other 8 of the 16
    return x;
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

// ------------------------------------------------------------- partial kernel

template <int D, int G, int DT, bool PAGED>
__global__ __launch_bounds__(kThreads) void partial_valu(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int hq, int hkv, int chunk, int s_max,
    int max_pages, float qk_scale_log2) {
    constexpr int LPR = D / 8;       // lanes per token row
    constexpr int RPW = 64 / LPR;    // token rows per wave-wide load
    constexpr int U = 4;             // loads of K (and of V) per stage
    constexpr int TPW = U * RPW;     // tokens per wave stage
    using E = Elt<DT>;

    const int g = blockIdx.x;
    const int s = blockIdx.y;
    const int b = blockIdx.z;
    int L = seq_lens[b];
    if constexpr (PAGED) L = min(L, max_pages * 16);  // never index past the table row
    if (L <= 0) return;
    const int nsplit = (L + chunk - 1) / chunk;
    if (s >= nsplit || s >= s_max) return;
    const int t0 = s * chunk;
    const int t1 = min(t0 + chunk, L);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane / LPR;
    const int c = lane % LPR;

    // First token row of this sequence in a packed contiguous cache.
    int64_t row0 = 0;
    if constexpr (!PAGED) {
        int64_t acc = 0;
        for (int i = lane; i < b; i += 64) acc += seq_lens[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        row0 = acc;
    }
    const int32_t* table = PAGED ? block_table + (int64_t)b * max_pages : nullptr;
    const int64_t head_off = (int64_t)g * D + c * 8;

    auto row_offset = [&](int t) -> int64_t {
        int64_t row;
        if constexpr (PAGED) {
            row = (int64_t)table[t >> 4] * 16 + (t & 15);
        } else {
            row = row0 + t;
        }
        return row * hkv * D + head_off;
    };

    // This lane's slice of the G query heads of KV head g.
    u32x4 qv[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        qv[j] = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * hq + g * G + j) * D + c * 8);

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = neg_inf();
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }

    const int ntok = t1 - t0;
    const int ntiles = (ntok + TPW - 1) / TPW;

    auto load = [&](int tile, u32x4* kb, u32x4* vb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int t = t0 + tile * TPW + u * RPW + r;
            t = min(t, t1 - 1);  // rows past the split re-read its last row; masked below
            const int64_t off = row_offset(t);
            kb[u] = *reinterpret_cast<const u32x4*>(k + off);
            vb[u] = *reinterpret_cast<const u32x4*>(v + off);
        }
    };

    auto compute = [&](int tile, const u32x4* kb, const u32x4* vb) {
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = (t0 + tile * TPW + u * RPW + r) < t1;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float dot = row_sum<LPR>(E::dot8(qv[j], kb[u]));
                sc[u][j] = valid ? dot * qk_scale_log2 : neg_inf();
            }
        }
        float vf[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) E::to_f32(vb[u], vf[u]);
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = sc[0][j];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
            const float mn = fmaxf(m[j], mx);
            const float mu = (mn == neg_inf()) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m[j] - mu);
            float p[U];
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = __builtin_amdgcn_exp2f(sc[u][j] - mu);
                ps += p[u];
            }
            l[j] = l[j] * alpha + ps;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = o[j][e] * alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) acc = fmaf(p[u], vf[u][e], acc);
                o[j][e] = acc;
            }
            m[j] = mn;
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
            float o2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[j][e], off);
            const float m2 = __shfl_xor(m[j], off);
            const float l2 = __shfl_xor(l[j], off);
            merge_stats<8>(m[j], l[j], o[j], m2, l2, o2);
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
            for (int e = 0; e < 8; ++e) sm_o[wave][j][c * 8 + e] = o[j][e];
            if (c == 0) {
                sm_m[wave][j] = m[j];
                sm_l[wave][j] = l[j];
            }
        }
    }
    __syncthreads();
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
        ws_o[slot * D + col] = acc;
        if (col == 0) {
            ws_ml[slot * 2] = M * kLn2;
            ws_ml[slot * 2 + 1] = lsum;
        }
    }
}

// ------------------------------------------------------------- combine kernel

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

// ------------------------------------------------------------------ dispatch

struct PartialArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* table;
    const int32_t* lens;
    float* ws_o;
    float* ws_ml;
    int hq, hkv, chunk, s_max, max_pages;
    float qk_scale_log2;
};

template <int D, int G, int DT, bool PAGED>
hipError_t launch_partial(const PartialArgs& a, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((partial_valu<D, G, DT, PAGED>), grid, dim3(kThreads), 0, st, a.q, a.k, a.v,
                       a.table, a.lens, a.ws_o, a.ws_ml, a.hq, a.hkv, a.chunk, a.s_max, a.max_pages,
                       a.qk_scale_log2);
    return hipGetLastError();
}

template <int D, int G, int DT>
hipError_t pick_paged(bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    return paged ? launch_partial<D, G, DT, true>(a, grid, st) : launch_partial<D, G, DT, false>(a, grid, st);
}

template <int D, int G>
hipError_t pick_dtype(int dt, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    return dt == FD_F16 ? pick_paged<D, G, FD_F16>(paged, a, grid, st)
                        : pick_paged<D, G, FD_BF16>(paged, a, grid, st);
}

template <int D>
hipError_t pick_group(int G, int dt, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: return pick_dtype<D, 1>(dt, paged, a, grid, st);
        case 2: return pick_dtype<D, 2>(dt, paged, a, grid, st);
        case 4: return pick_dtype<D, 4>(dt, paged, a, grid, st);
        default: return pick_dtype<D, 8>(dt, paged, a, grid, st);
    }
}

template <int D>
hipError_t launch_combine(int out_dt, const float* ws_o, const float* ws_ml, const int32_t* lens, void* out,
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

}  // namespace fdk

namespace fd {

fd_status query_num_cus(int32_t* out) {
    static int32_t cache[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64 && cache[dev] > 0) {
        *out = cache[dev];
        return FD_OK;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0)
        return fail(FD_ERR_HIP, "compute-unit query failed: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64) cache[dev] = n;
    *out = n;
    return FD_OK;
}

}  // namespace fd

using namespace fd;

extern "C" {

fd_status fd_decode_partial(const fd_problem* p, const fd_plan* plan, const void* q, const void* k,
                            const void* v, const int32_t* block_table, const int32_t* seq_lens_dev,
                            void* workspace, size_t workspace_bytes_avail, void* stream) {
    clear_error();
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

    fdk::PartialArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.table = block_table;
    a.lens = seq_lens_dev;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + workspace_o_bytes(p, plan->max_splits));
    a.hq = p->num_q_heads;
    a.hkv = p->num_kv_heads;
    a.chunk = plan->chunk_tokens;
    a.s_max = plan->max_splits;
    a.max_pages = p->page_size ? p->max_pages_per_seq : 0;
    a.qk_scale_log2 = scale * fdk::kLog2e;

    const int G = p->num_q_heads / p->num_kv_heads;
    dim3 grid(p->num_kv_heads, plan->max_splits, p->batch);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = p->head_dim == 64 ? fdk::pick_group<64>(G, p->kv_dtype, p->page_size != 0, a, grid, hs)
                                     : fdk::pick_group<128>(G, p->kv_dtype, p->page_size != 0, a, grid, hs);
    if (e != hipSuccess) return fail(FD_ERR_HIP, "partial kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
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
    hipError_t e = p->head_dim == 64
                       ? fdk::launch_combine<64>(p->out_dtype, ws_o, ws_ml, seq_lens_dev, out, lse, p->batch,
                                                 p->num_q_heads, plan->chunk_tokens, plan->max_splits, hs)
                       : fdk::launch_combine<128>(p->out_dtype, ws_o, ws_ml, seq_lens_dev, out, lse, p->batch,
                                                  p->num_q_heads, plan->chunk_tokens, plan->max_splits, hs);
    if (e != hipSuccess) return fail(FD_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

fd_status fd_decode_attention(const fd_problem* p, const void* q, const void* k, const void* v,
                              const int32_t* block_table, const int32_t* seq_lens_host,
                              const int32_t* seq_lens_dev, void* out, float* lse, void* workspace,
                              size_t workspace_bytes_avail, void* stream) {
    fd_plan plan;
    fd_status st = fd_plan_splits(p, seq_lens_host, 0, 0, &plan);
    if (st != FD_OK) return st;
    if (!out) return fail(FD_ERR_INVALID_ARGUMENT, "out must be non-NULL");
    if (workspace_bytes_avail < plan.workspace_bytes)
        return fail(FD_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, the plan needs %llu",
                    workspace_bytes_avail, (unsigned long long)plan.workspace_bytes);
    st = fd_decode_partial(p, &plan, q, k, v, block_table, seq_lens_dev, workspace, workspace_bytes_avail, stream);
    if (st != FD_OK) return st;
    return fd_combine(p, &plan, seq_lens_dev, workspace, workspace_bytes_avail, out, lse, stream);
}

}  // extern "C"
