// Prefill attention: the FlashAttention-2 forward pass over a sequence's new
// tokens, causal, on matrix cores.
//
// The method ("FlashAttention 全景演进与大模型 Token 生成全链路性能优化实战",
// §2.1): the outer loop runs over blocks of query rows, which stay on chip,
// and the inner loop over K/V blocks; the running max m and sum l of every
// row are updated per block and the output is divided by l once, after the
// last block (the tile recurrence of §1.2 / §1.3); K/V blocks wholly past
// every row's causal limit are not visited. The block sizes follow the same
// page's on-chip budget for d = 128: 128 query rows, K/V tiles of 64 tokens
// (the page suggests B_r = 64 or 128 with B_c = 64; measured on MI355X, 64
// beats 32 by 5-6%).
//
// Query rows are the q_len new tokens of each sequence, the last q_len
// positions of its cache: query i of sequence b sees tokens
// 0 .. L_b - q_len + i (q_len = L_b is plain causal prefill; a smaller q_len
// is a chunk of a longer prompt).
//
// One work-group of four wave64s per (sequence, query head, block of 128
// query rows); blocks with more visible tokens are dispatched first. Per
// 64-token tile:
//   * the work-group loads the K and V tile (256 threads x 16 bytes per
//     instruction, the next tile's loads in flight during the current tile's
//     compute) into LDS rows padded to 288 bytes;
//   * each wave owns 32 query rows as two 16-column MFMA tiles. Scores
//     S^T [32 tokens x 16 rows] = K_tile . Q^T as v_mfma_f32_16x16x32 with K
//     read from LDS (A operand) and Q^T held in registers (B operand); lane l
//     then holds 8 tokens of row l % 16;
//   * online softmax per row in the log2 domain, with the lazily moved
//     reference max of the decode kernel (rescale only when a row's max grows
//     by more than 2^8);
//   * O^T [128 dims x 16 rows] += V^T . P^T as v_mfma_f32_16x16x32: P^T is
//     the score layout itself (the contraction's token order is free, so the
//     A operand's token slots are matched to it), V^T comes from two
//     transposing LDS reads (ds_read_b64_tr_b16) per 16-dim block. The
//     product runs in fp16 for both cache types: P in fp16 (11 bits, where
//     bf16's 8 would show in the output), and a bf16 V tile is converted to
//     fp16 on its way into LDS. The conversion is exact for values within
//     fp16's normal range. A thread that stages a value beyond fp16's
//     largest marks the LDS buffer with the tile's number; after the staging
//     barrier the work-group sees the mark and stages that V tile again,
//     scaled by a power of two 2^-k (k from the tile's largest exponent, an
//     LDS atomic max), and the tile's products are rescaled by 2^k, so
//     nothing overflows (no vote and no extra barrier on ordinary tiles); values below fp16's normal range keep an
//     absolute error under 2^-25 times that scale (one product instead of the
//     two a high/low split of bf16 P would take);
//   * at the end each row's sum is reduced over its four lanes, O is divided
//     by l once and written with the natural-log LSE.

#include "fd_device.h"

namespace fdk {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#ifndef FD_PREFILL_BC
#define FD_PREFILL_BC 64
#endif
#ifndef FD_PREFILL_BUFS
#define FD_PREFILL_BUFS 2
#endif

constexpr int kD = 128;
constexpr int kBc = FD_PREFILL_BC;  // tokens per K/V tile (32 or 64)
constexpr int kMT = kBc / 16;       // 16-token score tiles per K/V tile
constexpr int kKS = kBc / 32;       // 32-token P.V steps per K/V tile
constexpr int kLoads = kBc / 16;    // 16-byte loads of K (and of V) per thread per tile
constexpr int kBufs = FD_PREFILL_BUFS;
constexpr int kPW = 4;              // waves per work-group
#ifndef FD_PREFILL_QW
#define FD_PREFILL_QW 32
#endif
constexpr int kQW = FD_PREFILL_QW;  // query rows per wave (16-column tiles)
constexpr int kNT = kQW / 16;       // 16-column tiles per wave
constexpr int kBr = kPW * kQW;      // query rows per work-group
constexpr int kPitch = kD + 16;     // LDS row pitch, elements

// Score products in the cache's type.
template <int DT> struct Mma;
template <> struct Mma<FD_F16> {
    static __device__ __forceinline__ f32x4_t mma(u32x4 a, u32x4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    }
};
template <> struct Mma<FD_BF16> {
    static __device__ __forceinline__ f32x4_t mma(u32x4 a, u32x4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};

// P.V products: fp16 for either cache type.
__device__ __forceinline__ f32x4_t mma_f16(u32x4 a, u32x4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, half2_t{(_Float16)a, (_Float16)b});
}
// Two bf16 values times 2^-k, as two fp16 values (exact while the products
// stay in fp16's normal range).
__device__ __forceinline__ uint32_t bf16_pair_to_f16(uint32_t w, int k) {
    const float lo = __builtin_bit_cast(float, w << 16), hi = __builtin_bit_cast(float, w & 0xffff0000u);
    return k ? pack_f16(ldexpf(lo, -k), ldexpf(hi, -k)) : pack_f16(lo, hi);
}
// Running maxima of the magnitude fields (exponent and mantissa bits) of the
// two bf16 halves of words, two 16-bit lanes at a time.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2_t bf16_pair_max_mag(u16x2_t m, uint32_t w) {
    return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w & 0x7fff7fffu));
}
__device__ __forceinline__ uint32_t max_of(u16x2_t m) { return max((uint32_t)m[0], (uint32_t)m[1]); }
constexpr uint32_t kF16MaxAsBf16 = 0x477fu;  // the largest bf16 magnitude at most fp16's 65504

__device__ __forceinline__ i16x4_t lds_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(const_cast<uint16_t*>(p)));
}

__device__ __forceinline__ u32x4 join(i16x4_t a, i16x4_t b) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t x = __builtin_bit_cast(u32x2_t, a);
    const u32x2_t y = __builtin_bit_cast(u32x2_t, b);
    return u32x4{x[0], x[1], y[0], y[1]};
}

}  // namespace

template <int DT, int OUT, bool PAGED>
__global__ __launch_bounds__(64 * kPW) void prefill_fa2(const PrefillArgs a) {
    using M = Mma<DT>;
    __shared__ __attribute__((aligned(16))) uint16_t sk[kBufs][kBc * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sv[kBufs][kBc * kPitch];
    __shared__ int s_vbad[kBufs];  // per buffer: the last tile staged there with a value past fp16's range
    __shared__ uint32_t s_vmax;

    // Work-group -> (query block, sequence, head), query blocks in descending
    // order so the longest causal rows start first.
    const int bh = a.batch * a.hq;
    const int nqb = (a.q_len + kBr - 1) / kBr;
    const int qblk = nqb - 1 - (int)(blockIdx.x / bh);
    const int b = (blockIdx.x % bh) / a.hq;
    const int h = blockIdx.x % a.hq;
    const int G = a.hq / a.hkv;
    const int g = h / G;

    const int L = PAGED ? min(a.lens[b], a.max_pages * 16) : a.lens[b];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4;
    const int col = lane & 15;

    // Packed cache: sequence b starts after the lengths before it.
    int64_t row0 = 0;
    if constexpr (!PAGED) {
        for (int i = lane; i < b; i += 64) row0 += a.lens[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) row0 += __shfl_xor(row0, off);
        // Every lane holds the same sum; keep it in scalar registers.
        row0 = ((int64_t)__builtin_amdgcn_readfirstlane((int)(row0 >> 32)) << 32) |
               (uint32_t)__builtin_amdgcn_readfirstlane((int)(row0 & 0xffffffff));
    }
    const int32_t* table = PAGED ? a.table + (int64_t)b * a.max_pages : nullptr;

    // Causal limits: query i sees tokens below L - q_len + i + 1.
    const int q_first = qblk * kBr;
    const int q_last = min(a.q_len, q_first + kBr) - 1;
    const int blk_lim = min(L, L - a.q_len + q_last + 1);  // tokens any row of the block sees
    const int ntiles = blk_lim > 0 ? (blk_lim + kBc - 1) / kBc : 0;

    // This lane's two query rows (one per 16-column tile).
    int qi[kNT], lim[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        qi[nt] = q_first + wave * kQW + 16 * nt + col;
        lim[nt] = qi[nt] < a.q_len ? max(0, L - a.q_len + qi[nt] + 1) : 0;
    }
    int wave_lim = 0;            // tokens any row of this wave sees
    int wave_min_lim = INT32_MAX;  // tokens every row of this wave sees
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        wave_lim = max(wave_lim, lim[nt]);
        wave_min_lim = min(wave_min_lim, lim[nt]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        wave_lim = max(wave_lim, __shfl_xor(wave_lim, off));
        wave_min_lim = min(wave_min_lim, __shfl_xor(wave_min_lim, off));
    }
    wave_lim = __builtin_amdgcn_readfirstlane(wave_lim);
    wave_min_lim = __builtin_amdgcn_readfirstlane(wave_min_lim);

    // Q^T as B operands: lane (grp, col) holds dims 32 j + 8 grp .. +8 of its row.
    u32x4 qb[kNT][4];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int64_t qrow = ((int64_t)b * a.q_len + min(qi[nt], a.q_len - 1)) * a.hq + h;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qb[nt][j] = qi[nt] < a.q_len ? *reinterpret_cast<const u32x4*>(a.q + qrow * kD + 32 * j + 8 * grp)
                                         : u32x4{0u, 0u, 0u, 0u};
    }

    float m_ref[kNT], m_use[kNT], l_run[kNT];
    f32x4_t acc[kNT][8];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        m_ref[nt] = neg_inf();
        m_use[nt] = 0.f;
        l_run[nt] = 0.f;
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) acc[nt][jd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Tile loads: thread t covers rows t / 16 + 16 i, dims 8 (t % 16) .. +8,
    // as buffer loads from a wave-uniform base with fixed per-lane offsets.
    // The descriptor ends at the sequence's last row, so rows past it read as
    // zeros (they are masked) and nothing past the sequence is touched. A
    // 16-row group of a tile is one page of a paged cache (tiles start on page
    // boundaries).
    const int lr = threadIdx.x >> 4;
    const int lc = threadIdx.x & 15;
    const int row_bytes = a.hkv * kD * 2;
    const uint16_t* kh = a.k + (int64_t)g * kD;  // head g of row 0
    const uint16_t* vh = a.v + (int64_t)g * kD;
    u32x4 kr[kLoads], vr[kLoads];
    // The tile's K (when WITH_K) and V pieces of this thread.
    auto load_into = [&]<bool WITH_K>(int tile, u32x4* kd, u32x4* vd) {
        const int t0 = tile * kBc;
        if constexpr (PAGED) {
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const int tg = t0 + 16 * i;  // first token of this page
                // (wave-uniform: readfirstlane keeps the descriptor in scalar registers)
                const int rows = __builtin_amdgcn_readfirstlane(max(0, min(16, L - tg)));
                const int64_t page = rows > 0 ? (int64_t)checked_page(table[tg >> 4], a.num_pages) : 0;
                const int voff = lr * row_bytes + 16 * lc;
                if constexpr (WITH_K)
                    kd[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          make_rsrc(kh + page * 16 * a.hkv * kD, rows * row_bytes), voff, 0, 0));
                vd[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      make_rsrc(vh + page * 16 * a.hkv * kD, rows * row_bytes), voff, 0, 0));
            }
        } else {
            const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kBc, L - t0)));
            const int64_t base = (row0 + t0) * a.hkv * kD;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + base, rows * row_bytes);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + base, rows * row_bytes);
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const int voff = (16 * i + lr) * row_bytes + 16 * lc;
                if constexpr (WITH_K) kd[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, voff, 0, 0));
                vd[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0));
            }
        }
    };
    auto load = [&](int tile) { load_into.template operator()<true>(tile, kr, vr); };
    // A bf16 V tile is staged as fp16. A thread holding a value beyond
    // fp16's range marks the buffer with the tile's number (s_vbad), and the
    // tile is staged again, scaled, before it is used (restage_v).
    auto stage = [&](int buf, int tile) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            *reinterpret_cast<u32x4*>(sk[buf] + (lr + 16 * i) * kPitch + 8 * lc) = kr[i];
            u32x4 w = vr[i];
            if constexpr (DT == FD_BF16) {
                u16x2_t mx = {0, 0};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mx = bf16_pair_max_mag(mx, w[e]);
                    w[e] = bf16_pair_to_f16(w[e], 0);
                }
                if (max_of(mx) > kF16MaxAsBf16) s_vbad[buf] = tile;
            }
            *reinterpret_cast<u32x4*>(sv[buf] + (lr + 16 * i) * kPitch + 8 * lc) = w;
        }
    };
    // The marked tile's V again (every thread of the work-group, after the
    // barrier that follows staging): loaded once more, scaled by 2^-k with k
    // from the tile's largest exponent so that every value stays below 2^15,
    // staged, and k returned. Rare: only tiles with values past 65504.
    auto restage_v = [&](int tile, int buf) -> int {
        u32x4 vt[kLoads];
        load_into.template operator()<false>(tile, nullptr, vt);
        u16x2_t mx = {0, 0};
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = bf16_pair_max_mag(mx, vt[i][e]);
        if (threadIdx.x == 0) s_vmax = 0;
        __syncthreads();
        atomicMax(&s_vmax, max_of(mx));
        __syncthreads();
        const int k = (int)(s_vmax >> 7) - 127 - 14;  // the largest value's binary exponent (>= 15), less 14
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            u32x4 w = vt[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = bf16_pair_to_f16(w[e], k);
            *reinterpret_cast<u32x4*>(sv[buf] + (lr + 16 * i) * kPitch + 8 * lc) = w;
        }
        __syncthreads();
        return k;
    };
    auto v_scale_of = [&](int tile, int buf) -> int {
        if constexpr (DT != FD_BF16) return 0;
        else return s_vbad[buf] == tile ? restage_v(tile, buf) : 0;
    };

    const int vrd = (4 * grp + ((lane >> 2) & 3)) * kPitch + 4 * (lane & 3);
    auto compute = [&](int tile, int buf, int vk) {
        const int t0 = tile * kBc;
        const uint16_t* K = sk[buf];
        const uint16_t* V = sv[buf];
        // Scores: S^T tile (mt, nt), lane (grp, col): tokens t0 + 16 mt + 4 grp + i of row col.
        f32x4_t s[kMT][kNT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) s[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 ka = *reinterpret_cast<const u32x4*>(K + (16 * mt + col) * kPitch + 32 * j + 8 * grp);
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) s[mt][nt] = M::mma(ka, qb[nt][j], s[mt][nt]);
            }
        }

        // The softmax below is the wave's vector-ALU phase, between its two
        // matrix-core phases: it issues at raised priority, so that while one
        // wave of a SIMD works through its exponentials the other's products
        // fill the matrix core, rather than both waves reaching the same phase
        // together (measured on MI355X, same GPU, three times: 8K-token
        // prompt 633-638 -> 621-626 us).
        __builtin_amdgcn_s_setprio(1);
        // Online softmax per row; P^T packed as the B operands of the P.V steps.
        // Only tiles that reach past some row's causal limit need the mask.
        const bool masked = t0 + kBc > wave_min_lim;
        u32x4 pp[kNT][kKS];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            // Raw scores here; the (positive) scale joins the exponent's fma below.
            // The mask is a separate (wave-uniform) branch, so that the tiles
            // wholly inside every row's limit skip its compare and select.
            if (masked) {
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (t0 + 16 * mt + 4 * grp + i >= lim[nt]) s[mt][nt][i] = neg_inf();
            }
            float p[4 * kMT];
            float mx = neg_inf();
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[4 * mt + i] = s[mt][nt][i];
                    mx = fmaxf(mx, p[4 * mt + i]);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            mx *= a.qk_scale_log2;  // log2 units
            if (__ballot(mx > m_ref[nt] + 8.f)) {
                const float mn = fmaxf(m_ref[nt], mx);
                const float mu = (mn == neg_inf()) ? 0.f : mn;
                const float alpha = __builtin_amdgcn_exp2f(m_ref[nt] - mu);
                l_run[nt] *= alpha;
#pragma unroll
                for (int jd = 0; jd < 8; ++jd) acc[nt][jd] = acc[nt][jd] * alpha;
                m_ref[nt] = mn;
                m_use[nt] = mu;
            }
            float ps = 0.f;
#pragma unroll
            for (int k = 0; k < 4 * kMT; ++k) {
                p[k] = __builtin_amdgcn_exp2f(fmaf(p[k], a.qk_scale_log2, -m_use[nt]));
                ps += p[k];
            }
            l_run[nt] += ps;
            // k-step ks covers score tiles 2 ks and 2 ks + 1: p[8 ks .. 8 ks + 7].
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    pp[nt][ks][w] = pack_f16(p[8 * ks + 2 * w], p[8 * ks + 2 * w + 1]);
                }
        }

        // O^T += V^T . P^T per 32-token step: the A operand's token slots
        // 8 grp + k are tokens 32 ks + 4 grp + k (k < 4) and 32 ks + 16 + 4 grp + k - 4,
        // the score layout; two transposing reads per 16-dim block. A tile
        // staged at 2^-vk adds its products at that scale (acc * 2^-vk, then
        // back), every step a power of two.
        if (vk) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int jd = 0; jd < 8; ++jd)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[nt][jd][i] = ldexpf(acc[nt][jd][i], -vk);
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
            for (int jd = 0; jd < 8; ++jd) {
                const u32x4 va = join(lds_tr(V + vrd + 32 * ks * kPitch + 16 * jd),
                                      lds_tr(V + vrd + (32 * ks + 16) * kPitch + 16 * jd));
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) acc[nt][jd] = mma_f16(va, pp[nt][ks], acc[nt][jd]);
            }
        }
        if (vk) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int jd = 0; jd < 8; ++jd)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[nt][jd][i] = ldexpf(acc[nt][jd][i], vk);
        }
    };

    if (ntiles > 0) {
        if (threadIdx.x < kBufs) s_vbad[threadIdx.x] = -1;
        __syncthreads();
        load(0);
        if constexpr (kBufs == 2) {
            // Two LDS buffers: tile t+1 is staged while tile t is computed; one
            // barrier per tile.
            stage(0, 0);
            if (1 < ntiles) load(1);
            __syncthreads();
            for (int tile = 0; tile < ntiles; ++tile) {
                const int cur = tile & 1;
                const int vk = v_scale_of(tile, cur);
                if (tile * kBc < wave_lim) compute(tile, cur, vk);
                if (tile + 1 < ntiles) {
                    stage(cur ^ 1, tile + 1);
                    if (tile + 2 < ntiles) load(tile + 2);
                }
                __syncthreads();
            }
        } else {
            for (int tile = 0; tile < ntiles; ++tile) {
                __syncthreads();  // every wave is done with the previous tile
                stage(0, tile);
                if (tile + 1 < ntiles) load(tile + 1);
                __syncthreads();
                const int vk = v_scale_of(tile, 0);
                if (tile * kBc < wave_lim) compute(tile, 0, vk);
            }
        }
    }

    // Finish every row: sum over its four lanes, divide once, natural-log LSE.
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        float l = l_run[nt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (qi[nt] >= a.q_len) continue;
        const int64_t orow = ((int64_t)b * a.q_len + qi[nt]) * a.hq + h;
        const bool empty = !(l > 0.f);
        const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
        for (int jd = 0; jd < 8; ++jd)
#pragma unroll
            for (int i = 0; i < 4; ++i) store_out<OUT>(a.out, orow * kD + 16 * jd + 4 * grp + i, acc[nt][jd][i] * inv);
        if (a.lse && grp == 0)
            a.lse[orow] = empty ? neg_inf() : (m_use[nt] + log2f(l)) * kLn2;
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int dt, int out_dt, bool paged, hipStream_t st) {
    const int64_t blocks = (int64_t)a.batch * a.hq * ((a.q_len + kBr - 1) / kBr);
    const dim3 grid((uint32_t)blocks), block(64 * kPW);
    auto go = [&]<int DT, int OUT>() {
        if (paged)
            hipLaunchKernelGGL((prefill_fa2<DT, OUT, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((prefill_fa2<DT, OUT, false>), grid, block, 0, st, a);
    };
    auto by_out = [&]<int DT>() {
        if (out_dt == FD_F32) go.template operator()<DT, FD_F32>();
        else if (out_dt == FD_F16) go.template operator()<DT, FD_F16>();
        else go.template operator()<DT, FD_BF16>();
    };
    if (dt == FD_F16) by_out.template operator()<FD_F16>();
    else by_out.template operator()<FD_BF16>();
    return hipGetLastError();
}

}  // namespace fdk
