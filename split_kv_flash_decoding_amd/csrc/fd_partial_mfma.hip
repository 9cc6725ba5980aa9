// Partial kernel, matrix-core form: every K/V row serves nq = q_len * G query
// rows (G query heads per KV head, q_len query tokens per sequence),
// 2 <= nq <= 64 (one work-group per 16 of them); d = 128, fp16/bf16 K/V or
// FP8 (E4M3) K/V with per-head scales, contiguous or paged.
//
// With G query heads sharing one KV head, each K row meets G queries and each
// V row is weighted by G probabilities: both products are small dense
// contractions ("FlashAttention 全景演进与大模型 Token 生成全链路性能优化实战",
// §4.2 on grouped-query attention; §2.3 for the split-KV decomposition), so
// they run on MFMA instead of the vector ALU, which would spend ~G times the
// instructions of the MHA kernel per byte read.
//
// One work-group of four wave64s per (sequence, KV head, split), or, under
// the balanced split list, per (work item, KV head): the item's shares of
// consecutive sequences then run through this same body one after the
// other. Each wave takes 16-token tiles of its split in turn (a tile is one
// page of a paged cache). Per tile, with lane l in group g = l/16 at column
// c = l%16:
//   * K and V tiles are read from HBM the same way: each 16-byte load
//     instruction covers four whole 256-byte token rows (loading K straight
//     into the MFMA operand layout instead, 16 rows x 64 bytes per
//     instruction, measured 5.3 TB/s against 6.5-7.1 TB/s for whole rows);
//     both tiles are staged in LDS (rows padded to 288 bytes; rocprofv3 counts
//     no LDS bank-conflict cycles for these reads and stores on MI355X, 16-bit
//     and FP8 caches alike, SQ_LDS_BANK_CONFLICT against SQ_LDS_IDX_ACTIVE);
//   * scores: S^T[16 tokens x 16 heads] = K_tile [16 x 128] . Q^T [128 x 16]
//     as four v_mfma_f32_16x16x32 (the A operand, K row c with 8 dims per
//     lane, is read back from LDS; Q^T is a register-resident B operand, zero
//     past head G-1). The result leaves lane l holding tokens 4g..4g+3 of
//     head c;
//   * online softmax per head, log2 domain: the tile max is reduced over the
//     four lanes of a head (two row swaps); each lane keeps a partial running
//     sum over its own tokens (summed at the end). The exponentials use a
//     reference max that only moves when a tile's max exceeds it by more than
//     8 (a wave-uniform branch), so probabilities stay <= 2^8 and the
//     accumulators are rescaled rarely instead of every tile; one final
//     rescale moves (O, l) to the split's true max, which the workspace holds;
//   * probabilities in fp32 are split into a high and a low 16-bit part
//     (p = hi + lo exactly to ~2^-17), so the 16-bit matrix product loses
//     nothing the tolerance would see;
//   * O^T [128 x 16 heads] += V^T [128 x 16 tokens] . P^T [16 tokens x 16]
//     as eight 16x16x16 MFMAs per part, or (waves owning heads) for both
//     parts at once as eight v_mfma_f32_16x16x32, whose 32-long contraction
//     takes the tile's tokens twice (high parts, then low parts of P; the
//     same V values twice). P^T is exactly the layout the score
//     MFMA produced; V^T comes from the V tile staged in LDS (row-major,
//     padded rows) and read back transposed with ds_read_b64_tr_b16, so
//     every lane's output column is its own head and the per-head rescale
//     needs no cross-lane traffic;
//   * an FP8 cache has 128-byte rows: one load instruction covers eight
//     rows, and the codes are widened exactly to the query's 16-bit type on
//     their way into LDS, so the matrix products are those of a 16-bit cache;
//     the K scale of the head joins the score scale and its V scale the
//     split's output;
//   * K/V loads are buffer loads from a per-tile scalar base with fixed
//     per-lane offsets (no per-load address arithmetic); the descriptor's
//     size ends at the split's last row, so rows past it read as zeros;
//   * the next tile's K and V loads are in flight while the current tile is
//     computed: a 16-bit tile's registers go to LDS first and then receive the
//     next tile's loads, so one tile's worth of registers suffices; FP8 tiles
//     use a two-deep register ring, so two of them are in flight;
//   * paged caches whose splits start on a page boundary look pages up once
//     per 64 tiles: lane i of a wave holds the page of its i-th next tile and
//     each tile reads its page with readlane, so no K/V load waits on a table
//     load.
// Several query tokens per sequence (capstone §4.5, speculative decoding's
// verification pass) add query rows: row n = i * G + j is head j of the group
// for query token i, which sees tokens up to L - q_len + i, so each lane
// masks its column with its own causal limit; a row that sees nothing of a
// split leaves (m, l, O) = (-inf, 0, 0).
// At the end the four waves merge through LDS by the two-block identity
// (same page, §1.2) and the split's (O, m, l) go to the workspace.

#include "fd_device.h"

namespace fdk {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kTile = 16;                  // tokens per tile (one 16-token page)
constexpr int kMW = fd::kMfmaWaves;        // waves per work-group
constexpr int kPitch = kD + 16;            // LDS row pitch of a V tile, elements (288 B)

template <int DT> struct Mfma;

template <> struct Mfma<FD_F16> {
    typedef f16x8_t v8;
    typedef f16x4_t v4;
    static __device__ __forceinline__ f32x4_t qk(u32x4 a, u32x4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv(i16x4_t a, v4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4, a), b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv2(u32x4 a, u32x4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ void split(const float* p, v4& hi, v4& lo) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const _Float16 h = (_Float16)p[e];
            hi[e] = h;
            lo[e] = (_Float16)(p[e] - (float)h);
        }
    }
};

template <> struct Mfma<FD_BF16> {
    typedef bf16x8_t v8;
    typedef bf16x4_t v4;
    static __device__ __forceinline__ f32x4_t qk(u32x4 a, u32x4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv(i16x4_t a, v4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4, a), b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv2(u32x4 a, u32x4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ void split(const float* p, v4& hi, v4& lo) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const __bf16 h = (__bf16)p[e];
            hi[e] = h;
            lo[e] = (__bf16)(p[e] - (float)h);
        }
    }
};

__device__ __forceinline__ i16x4_t lds_read_transposed(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(const_cast<uint16_t*>(p)));
}

}  // namespace

// NQ: query rows of a column tile rounded up to a power of two (2..16); the
// rows nq..NQ-1 and 16-NQ..15 of the MFMA tile are idle. PAGE_MODE: 0 contiguous
// cache; 1 paged, any split alignment (a table lookup per token); 2 paged,
// splits start on page boundaries.
// Two codes of an E4M3 word (the low or high half) widened to a 16-bit pair.
template <int QT, bool HIGH>
__device__ __forceinline__ uint32_t widen_fp8_pair(uint32_t w) {
    if constexpr (QT == FD_F16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HIGH));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HIGH));
}

// NQ: as above. KT: cache element type (QT, or FP8 E4M3); QT: q's 16-bit
// type, which the matrix products use. KEEP: several column tiles read each
// K/V row, so the loads leave it in L2 for the other tiles' work-groups
// instead of streaming it past (measured on MI355X: 64 rows, 128K tokens
// x 32 heads, 922 -> 665 us; one tile is faster with streaming loads).
// WH (waves own heads): the four waves of a work-group take 4 / NT KV heads
// times the NT column tiles of each, and every wave runs every tile of the
// work item's shares for its own (head, column tile) pair: no two waves share
// an output row, so each writes its own partial, with no merge through LDS
// and no barrier between shares, and the NT waves of a head read the same K/V
// tiles on one compute unit. Needs NT in {1, 2, 4} and Hkv a multiple of
// 4 / NT.
// NTS (WH with NT = NTS > 1 column tiles): the NT waves of a head split the
// loads of each K/V tile between them, stage it once into a tile buffer they
// share (two buffers per head, one barrier per tile) and each run their own
// column tile from it, so a K/V byte is loaded and staged once per work-group
// instead of once per column tile.
// Register budget: at most 168 VGPRs (three waves per SIMD, so three
// work-groups per compute unit can be resident), and 128 (four) for the
// shared-tile forms, which the planner gives four work-groups per compute
// unit; none spills.
template <int NQ, int KT, int QT, int PAGE_MODE, bool KEEP, bool WH = false, int NTS = 1>
__global__ __launch_bounds__(64 * kMW) __attribute__((amdgpu_waves_per_eu(NTS > 1 && PAGE_MODE != 1 ? 4 : 3))) void partial_mfma(const PartialArgs a) {
    using M = Mfma<QT>;
    constexpr bool PAGED = PAGE_MODE != 0;
    constexpr bool FP8 = KT == FD_FP8_E4M3;
    constexpr int EB = FP8 ? 1 : 2;   // bytes per cache element
    constexpr int RPI = FP8 ? 8 : 4;  // token rows per wave-wide 16-byte load
    constexpr int KL = kTile / RPI;   // loads of K (and of V) per tile
    constexpr int kPolicy = KEEP ? 0 : kBufferLoadPolicy;
    const uint16_t* __restrict__ q = a.q;
    const int32_t* __restrict__ block_table = a.table;
    const int32_t* __restrict__ seq_lens = a.lens;
    float* __restrict__ ws_o = a.ws_o;
    float* __restrict__ ws_ml = a.ws_ml;
    const int batch = a.batch, hq = a.hq, hkv = a.hkv, chunk = a.chunk, s_max = a.s_max, max_pages = a.max_pages;
    const int q_len = a.q_len;
    // The tile staging area (per wave: a K and a V tile) and, once every wave
    // is done with its tiles, the wave merge share the same LDS.
    constexpr int kStageBytes = kMW * 2 * kTile * kPitch * 2;
    constexpr int kMergeBytes = kMW * NQ * kD * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes];
    __shared__ float sm_m[kMW][NQ];
    __shared__ float sm_l[kMW][NQ];
    uint16_t (*sk)[kTile * kPitch] = reinterpret_cast<uint16_t (*)[kTile * kPitch]>(smem);
    uint16_t (*sv)[kTile * kPitch] = reinterpret_cast<uint16_t (*)[kTile * kPitch]>(smem + kStageBytes / 2);
    float (*sm_o)[NQ][kD] = reinterpret_cast<float (*)[NQ][kD]>(smem);

    // More than 16 query rows per KV head (many draft tokens of a grouped
    // head) take ceil(rows / 16) column tiles, one work-group each; the NT
    // work-groups of one work-list entry sit 8 apart in the grid, which the
    // round-robin placement of work-groups on the eight XCDs puts on one XCD,
    // so the later ones find the entry's K/V in that XCD's L2.
    const int G = hq / hkv;
    const int nq_all = q_len * G;
    const int NT = (nq_all + 15) / 16;
    int unit = blockIdx.x, ct = 0;
    if (!WH && NT > 1) {
        const int rem = blockIdx.x % (8 * NT);
        ct = rem / 8;
        unit = blockIdx.x / (8 * NT) * 8 + rem % 8;
    }
    // KV heads per work-group, and head blocks per work item.
    const int hpw = WH ? kMW / NT : 1;
    const int blocks = hkv / hpw;
    // Split mode 0: the work-list entry is one split (locate_unit). Mode 1: it
    // is work item unit / blocks of the balanced list, whose shares of
    // consecutive sequences run one after the other (the body below, once
    // per share).
    const int len_cap = PAGED ? max_pages * 16 : INT32_MAX;
    WorkUnit wu;
    int S_b = 0;
    BalancedCursor cur;
    if (a.split_mode == 0) {
        if (!locate_unit(unit, seq_lens, batch, blocks, chunk, len_cap, wu)) return;
        S_b = (wu.L + chunk - 1) / chunk;
    } else {
        if (!balanced_first(unit / blocks, seq_lens, batch, chunk >> 4, len_cap, cur) ||
            !balanced_share(seq_lens, batch, chunk >> 4, len_cap, unit % blocks, cur, wu, S_b))
            return;
    }
    int phase = 0;  // shared tile buffers (NTS > 1): the one the next tile is staged into
next_share:
    // The unit is the same in every lane, but it leaves the lookups through
    // branches the compiler takes for lane-divergent: restated as scalars, the
    // tile loop's buffer descriptors and bounds stay in scalar registers.
    uniform_unit(wu);
    S_b = uniform(S_b);
    if (wu.s >= s_max) return;
    const int s = wu.s, b = wu.b, t0 = wu.t0, t1 = wu.t1;
    const int64_t row0 = wu.row0;

    // The thread index is made opaque on every pass, so the compiler cannot
    // hoist lane-derived addresses (the epilogue's) out of the loop over
    // shares and hold them in registers across the tile loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    // The wave index is wave-uniform: taking it through a scalar register lets
    // the compiler keep the per-wave K/V buffer descriptors in scalar
    // registers (a vector-held descriptor turns every buffer load into a loop
    // over its distinct values).
    const int wave = uniform(tid >> 6);
    const int grp = lane >> 4;  // 0..3
    const int col = lane & 15;  // query row (scores, output) / token (K operand) / d-slice (V load)
    // This wave's KV head and column tile.
    const int g = WH ? wu.g * hpw + wave / NT : wu.g;
    const int ctw = WH ? wave % NT : ct;

    // Column `col` is query row c0 + col of the group: head qj for query
    // token qi; it may see tokens below `lim` (its causal limit, inside this
    // split). nq: the rows of this column tile.
    const int c0 = 16 * ctw;
    const int nq = min(16, nq_all - c0);
    const int qi = (c0 + col) / G;
    const int qj = c0 + col - qi * G;
    const int lim = min(t1, wu.L - q_len + qi + 1);
    // Tiles wholly below every active row's limit need no mask (all but the
    // last tile or two of a share).
    int lim_lo = col < nq ? lim : INT32_MAX;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lim_lo = min(lim_lo, __shfl_xor(lim_lo, off));
    lim_lo = uniform(lim_lo);

    const int32_t* table = PAGED ? block_table + (int64_t)b * max_pages : nullptr;
    const int row_bytes = hkv * kD * EB;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (int64_t)g * kD * EB;
    const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + (int64_t)g * kD * EB;
    const float qk_scale_log2 = a.qk_scale_log2 * head_scale(a.k_scale, g);

    // Q^T as the B operand of the score MFMAs: lane l holds, for d-block j,
    // dims 32 j + 8 grp .. +8 of query row col; rows past nq-1 are zero.
    const int64_t qrow = ((int64_t)b * q_len + qi) * hq + g * G + qj;
    u32x4 qb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (col < nq) {
            qb[j] = *reinterpret_cast<const u32x4*>(q + qrow * kD + 32 * j + 8 * grp);
        } else {
            qb[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    float m_ref = neg_inf();   // reference max of head `col` for the exponentials (log2 units)
    float m_use = 0.f;         // m_ref, or 0 while it is still -inf
    float m_true = neg_inf();  // running max of head `col`
    float l_run = 0.f;         // running sum (relative to m_ref) over this lane's tokens of head `col`
    f32x4_t acc[8];
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) acc[jd] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (t1 - t0 + kTile - 1) / kTile;
    uint16_t* my_sk = sk[wave];
    uint16_t* my_sv = sv[wave];
    // This lane's part of a tile load: row RPI i + lrow, bytes 16 lcol .. +16
    // (dims 8 lcol .. +8 of a 16-bit row, 16 lcol .. +16 of an FP8 row).
    const int lrow = lane / (64 / RPI);
    const int lcol = lane % (64 / RPI);
    int voff_v[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) voff_v[i] = (RPI * i + lrow) * row_bytes + 16 * lcol;

    auto row_of = [&](int t) -> int64_t {
        if constexpr (PAGED) {
            return (int64_t)checked_page(table[t >> 4], a.num_pages) * 16 + (t & 15);
        } else {
            return row0 + t;
        }
    };

    // A wave's tiles: wave, wave + kMW, ... of the split, or all of them (WH).
    const int tfirst = WH ? 0 : wave;
    constexpr int TSTEP = WH ? 1 : kMW;
    // Tile-aligned pages: lane i holds the page of this wave's tile 64 blk + i.
    int pg = 0, pg_blk = -1;
    auto tile_page = [&](int tile) -> int64_t {
        const int kk = (tile - tfirst) / TSTEP;
        const int blk = kk >> 6;
        if (blk != pg_blk) {
            const int tidx = tfirst + TSTEP * (64 * blk + lane);
            pg = tidx < ntiles ? checked_page(table[(t0 >> 4) + tidx], a.num_pages) : 0;
            pg_blk = blk;
        }
        return (int64_t)__builtin_amdgcn_readlane(pg, kk & 63) * 16;
    };

    // Where a tile's rows come from: buffer descriptors over its rows (the
    // descriptor's size ends at the split, so rows past it read as zeros), or,
    // for pages that may start mid-tile, one table lookup per row.
    struct TileSrc {
        __amdgpu_buffer_rsrc_t rk, rv;
        int tt;
    };
    auto tile_src = [&](int tile) -> TileSrc {
        TileSrc ts;
        ts.tt = t0 + tile * kTile;
        if constexpr (PAGE_MODE != 1) {
            const int64_t first = (PAGE_MODE == 2) ? tile_page(tile) : row0 + ts.tt;
            const int bytes = min(kTile, t1 - ts.tt) * row_bytes;
            ts.rk = make_rsrc(kbase + first * row_bytes, bytes);
            ts.rv = make_rsrc(vbase + first * row_bytes, bytes);
        }
        return ts;
    };
    // Load instruction i of the tile's K (or V) rows: rows RPI i .. + RPI.
    auto load_one = [&](const TileSrc& ts, int i, bool is_v) -> u32x4 {
        if constexpr (PAGE_MODE == 1) {
            // Pages may start mid-tile: one table lookup per row, clamped to the split.
            const int64_t row = row_of(min(ts.tt + RPI * i + lrow, t1 - 1)) * row_bytes;
            const uint8_t* src = (is_v ? vbase : kbase) + row + 16 * lcol;
            if constexpr (KEEP) return *reinterpret_cast<const u32x4*>(src);
            else return load16(src);
        } else {
            return buffer_load16<kPolicy>(is_v ? ts.rv : ts.rk, (RPI * i + lrow) * row_bytes + 16 * lcol);
        }
    };
    // Stage a landed load i as 16-bit rows RPI i .. + RPI of the tile at dst.
    auto stage_one = [&](u32x4 x, int i, uint16_t* dst) {
        if constexpr (FP8) {
            // codes 4 w .. 4 w + 3 sit in word w; dims 16 lcol .. +16
            u32x4 lo, hi;
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                lo[2 * w] = widen_fp8_pair<QT, false>(x[w]);
                lo[2 * w + 1] = widen_fp8_pair<QT, true>(x[w]);
                hi[2 * w] = widen_fp8_pair<QT, false>(x[w + 2]);
                hi[2 * w + 1] = widen_fp8_pair<QT, true>(x[w + 2]);
            }
            // Lane lcol's 32 bytes are chunks 2 lcol and 2 lcol + 1 of the row.
            // In dims 64..127 (lanes 4..7 of each eight) the two 8-dim halves
            // of every 16 dims trade places (dim x sits at x ^ 8), so each
            // store instruction's eight-lane groups cover 128 distinct bytes
            // modulo 128 with no per-lane data select (with the plain layout
            // every bank is hit twice: measured 0.37 conflict cycles per
            // LDS-active cycle); the tile readers apply the same swap.
            uint16_t* d = dst + (RPI * i + lrow) * kPitch + 16 * lcol;
            const int sw = (lcol & 4) * 2;
            *reinterpret_cast<u32x4*>(d + sw) = lo;
            *reinterpret_cast<u32x4*>(d + (sw ^ 8)) = hi;
        } else {
            *reinterpret_cast<u32x4*>(dst + (RPI * i + lrow) * kPitch + 8 * lcol) = x;
        }
    };

    auto load = [&](int tile, u32x4* kr, u32x4* vr) {
        const TileSrc ts = tile_src(tile);
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            kr[i] = load_one(ts, i, false);
            vr[i] = load_one(ts, i, true);
        }
    };

    // Stage a tile's K and V (landed in registers) as 16-bit rows in this
    // wave's LDS area: row RPI i + lrow.
    auto stage = [&](const u32x4* kr, const u32x4* vr) {
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            stage_one(kr[i], i, my_sk);
            stage_one(vr[i], i, my_sv);
        }
    };

    // One staged tile: scores, online softmax, P.V.
    auto compute = [&](int tile) {
        const int tt = t0 + tile * kTile;

        // V^T blocks of 16 dims: lane 16 g' + 4 e + j reads row 4 g' + e,
        // dims 16 jd + 4 j .. +4; the transposing read hands lane 16 g' + i
        // the dims-i column of rows 4 g' .. 4 g' + 3. The eight reads go out
        // first, so their latency passes under the scores and the softmax
        // (the shared-tile forms, held to 128 registers, read each block just
        // before its product instead).
        const uint16_t* rd_lo = my_sv + (4 * grp + ((lane >> 2) & 3)) * kPitch + 4 * (lane & 3);
        // dims 64..127 of an FP8 tile: 8-dim halves swapped (stage_one)
        const uint16_t* rd_hi = my_sv + (4 * grp + ((lane >> 2) & 3)) * kPitch + 4 * ((lane & 3) ^ (FP8 ? 2 : 0));
        constexpr bool kEarlyV = NTS == 1;
        auto read_v = [&](int jd) { return lds_read_transposed((jd < 4 ? rd_lo : rd_hi) + 16 * jd); };
        i16x4_t vt[8];
        if constexpr (kEarlyV) {
#pragma unroll
            for (int jd = 0; jd < 8; ++jd) vt[jd] = read_v(jd);
        }

        // A operand of d-block j: K row col, dims 32 j + 8 grp .. +8.
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // dims 64..127 of an FP8 tile: 8-dim halves swapped (stage_one)
            const int hsw = (FP8 && j >= 2) ? 8 : 0;
            const u32x4 ka = *reinterpret_cast<const u32x4*>(my_sk + col * kPitch + 32 * j + ((8 * grp) ^ hsw));
            sc = M::qk(ka, qb[j], sc);
        }

        // Shared-tile forms: the softmax (this wave's vector phase between its
        // two matrix-core phases) issues at raised priority, so the waves of a
        // SIMD tend to sit in different phases (measured on MI355X, same GPU,
        // twice: paged GQA with 8 query tokens 387.0/387.9 -> 385.2/385.0 us
        // per partial launch, 128K MHA with 64 query tokens 373.3/373.9 ->
        // 370.8/370.6 us; the single-tile forms did not move).
        if constexpr (NTS > 1) __builtin_amdgcn_s_setprio(1);
        float p[4];
        float mx = neg_inf();
        if (tt + kTile <= lim_lo) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = sc[i] * qk_scale_log2;
                mx = fmaxf(mx, p[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = (tt + 4 * grp + i < lim) ? sc[i] * qk_scale_log2 : neg_inf();
                mx = fmaxf(mx, p[i]);
            }
        }
        mx = max_lane_groups(mx);
        m_true = fmaxf(m_true, mx);
        // Move the reference only when some head's scores outgrow it by 2^8.
        if (__ballot(mx > m_ref + 8.f)) {
            const float mn = fmaxf(m_ref, mx);
            const float mu = (mn == neg_inf()) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - mu);  // 0 on the first tile
            l_run *= alpha;
#pragma unroll
            for (int jd = 0; jd < 8; ++jd) acc[jd] = acc[jd] * alpha;
            m_ref = mn;
            m_use = mu;
        }
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(p[i] - m_use);
            ps += p[i];
        }
        l_run += ps;
        typename M::v4 phi, plo;
        M::split(p, phi, plo);

        if constexpr (NTS > 1) __builtin_amdgcn_s_setprio(0);
        if constexpr (WH) {
            // Both parts in one double-rate product: the contraction runs over
            // the tile's 16 tokens twice, slots 8 g .. 8 g + 3 of lane group g
            // taking the high parts of its tokens 4 g .. 4 g + 3 and slots
            // 8 g + 4 .. 8 g + 7 the low parts, so B = [hi, lo] and A holds the
            // same four V values twice.
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t hw = __builtin_bit_cast(u32x2_t, phi), lw = __builtin_bit_cast(u32x2_t, plo);
            const u32x4 pb = {hw[0], hw[1], lw[0], lw[1]};
#pragma unroll
            for (int jd = 0; jd < 8; ++jd) {
                const u32x2_t v2 = __builtin_bit_cast(u32x2_t, kEarlyV ? vt[jd] : read_v(jd));
                acc[jd] = M::pv2(u32x4{v2[0], v2[1], v2[0], v2[1]}, pb, acc[jd]);
            }
        } else {
            // Two products (the other form's registers stay within 3 waves per SIMD).
#pragma unroll
            for (int jd = 0; jd < 8; ++jd) {
                const i16x4_t v4 = kEarlyV ? vt[jd] : read_v(jd);
                acc[jd] = M::pv(v4, plo, M::pv(v4, phi, acc[jd]));
            }
        }
    };

    int tile = tfirst;
    if constexpr (NTS > 1) {
        // The NTS waves of head hh take turns over the tile's 2 KL loads (K
        // loads first, then V): wave ctw takes loads ctw, ctw + NTS, ...
        constexpr int NL = 2 * KL / NTS;
        static_assert(2 * KL % NTS == 0, "loads per wave");
        const int hh = wave / NTS;
        const int part = uniform(ctw);
        constexpr int kTileElems = kTile * kPitch;
        u32x4 r[NL];
        auto load_part = [&](int tl) {
            const TileSrc ts = tile_src(tl);
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const int f = part + NTS * j;
                r[j] = load_one(ts, f % KL, f >= KL);
            }
        };
        if (ntiles > 0) load_part(0);
        for (; tile < ntiles; ++tile) {
            my_sk = reinterpret_cast<uint16_t*>(smem) + (hh * 2 + phase) * 2 * kTileElems;
            my_sv = my_sk + kTileElems;
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const int f = part + NTS * j;
                stage_one(r[j], f % KL, f >= KL ? my_sv : my_sk);
            }
            // The whole tile is staged; every wave of the work-group is also
            // past the tile before it, whose buffer the next tile reuses.
            __syncthreads();
            if (tile + 1 < ntiles) load_part(tile + 1);
            compute(tile);
            phase ^= 1;
        }
    } else if constexpr (!FP8) {
        // The wave's next tile loads into the registers its current tile has
        // just left for LDS, so they are in flight while the current tile is
        // computed and the register file holds one tile, not two: 3 waves per
        // SIMD instead of 2 (measured on MI355X: GQA varlen 124 -> 116 us).
        u32x4 kr[KL], vr[KL];
        if (tile < ntiles) load(tile, kr, vr);
        while (tile < ntiles) {
            stage(kr, vr);
            if (tile + TSTEP < ntiles) load(tile + TSTEP, kr, vr);
            compute(tile);
            tile += TSTEP;
        }
    } else {
        // FP8 tiles are half the registers of 16-bit ones, so a two-deep
        // register ring keeps two tiles in flight (the same bytes in flight
        // per wave as one 16-bit tile): a tile's registers go to LDS and then
        // take the loads of the tile two steps on.
        u32x4 ka[KL], va[KL], kb[KL], vb[KL];
        if (tile < ntiles) load(tile, ka, va);
        if (tile + TSTEP < ntiles) load(tile + TSTEP, kb, vb);
        while (tile < ntiles) {
            stage(ka, va);
            if (tile + 2 * TSTEP < ntiles) load(tile + 2 * TSTEP, ka, va);
            compute(tile);
            tile += TSTEP;
            if (tile >= ntiles) break;
            stage(kb, vb);
            if (tile + 2 * TSTEP < ntiles) load(tile + 2 * TSTEP, kb, vb);
            compute(tile);
            tile += TSTEP;
        }
    }

    // Each head's sum is spread over the four lanes that hold it.
    l_run = sum_lane_groups(l_run);
    // Express (O, l) relative to the true max (a factor in [2^-8, 1]).
    {
        const float mu = (m_true == neg_inf()) ? 0.f : m_true;
        const float alpha = (m_ref == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(m_ref - mu);
        l_run *= alpha;
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) acc[jd] = acc[jd] * alpha;
    }
    const float m_run = m_true;

    if constexpr (WH) {
        // This wave alone holds its rows' statistics: lane (grp, col) writes
        // O[row col][16 jd + 4 grp .. + 4] straight to the workspace.
        if (col < nq) {
            const float v_sc = head_scale(a.v_scale, g);
            const int n = c0 + col;
            const int ni = n / G;
            const int64_t slot = (((int64_t)b * q_len + ni) * hq + g * G + (n - ni * G)) * s_max + s;
#pragma unroll
            for (int jd = 0; jd < 8; ++jd)
                *reinterpret_cast<f32x4_t*>(ws_o + slot * kD + 16 * jd + 4 * grp) = acc[jd] * v_sc;
            if (grp == 0) {
                ws_ml[slot * 2] = m_run * kLn2;
                ws_ml[slot * 2 + 1] = l_run;
            }
        }
        if (a.counters)
            fused_merge<kD, (NQ < 4 ? NQ : 4), kMW>(a, b, S_b, wu.g * hpw, hpw, q_len * hpw * G, 1,
                                                    reinterpret_cast<float*>(smem));
        if (a.split_mode != 0) {
            balanced_advance(seq_lens, len_cap, cur);
            if (balanced_share(seq_lens, batch, chunk >> 4, len_cap, unit % blocks, cur, wu, S_b)) goto next_share;
        }
        return;
    }

    // Lane (grp, col) holds O[row col][16 jd + 4 grp + i]; the merge area
    // overlaps the other waves' staging tiles.
    __syncthreads();
    if (col < nq) {
#pragma unroll
        for (int jd = 0; jd < 8; ++jd)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_o[wave][col][16 * jd + 4 * grp + i] = acc[jd][i];
        if (grp == 0) {
            sm_m[wave][col] = m_run;
            sm_l[wave][col] = l_run;
        }
    }
    __syncthreads();
    const float v_sc = head_scale(a.v_scale, g);
    for (int idx = tid; idx < nq * kD; idx += 64 * kMW) {
        const int n = idx / kD;
        const int d = idx % kD;
        float Mx = sm_m[0][n];
#pragma unroll
        for (int w = 1; w < kMW; ++w) Mx = fmaxf(Mx, sm_m[w][n]);
        const float mu = (Mx == neg_inf()) ? 0.f : Mx;
        float o = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kMW; ++w) {
            const float a = __builtin_amdgcn_exp2f(sm_m[w][n] - mu);
            o += a * sm_o[w][n][d];
            lsum += a * sm_l[w][n];
        }
        const int ni = (c0 + n) / G;
        const int64_t row = ((int64_t)b * q_len + ni) * hq + g * G + (c0 + n - ni * G);
        const int64_t slot = row * s_max + s;
        ws_o[slot * kD + d] = o * v_sc;
        if (d == 0) {
            ws_ml[slot * 2] = Mx * kLn2;
            ws_ml[slot * 2 + 1] = lsum;
        }
    }
    // The fused merge takes four rows at a time: with sixteen, its accumulators
    // would cost the kernel its third wave per SIMD inside the loop over shares.
    if (a.counters) fused_merge<kD, (NQ < 4 ? NQ : 4), kMW>(a, b, S_b, g, 1, nq_all, NT, &sm_o[0][0][0]);
    if (a.split_mode != 0) {
        balanced_advance(seq_lens, len_cap, cur);
        if (balanced_share(seq_lens, batch, chunk >> 4, len_cap, unit % blocks, cur, wu, S_b)) {
            __syncthreads();  // the last share's merge area is the next share's staging area
            goto next_share;
        }
    }
}

template <int NQ, int KT, int QT, bool WH, bool KEEP = false, int NTS = 1>
hipError_t launch_nq(bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    // Paged splits that start on page boundaries read their page indices 64 at a time.
    if (!paged)
        hipLaunchKernelGGL((partial_mfma<NQ, KT, QT, 0, KEEP, WH, NTS>), grid, dim3(64 * kMW), 0, st, a);
    else if (a.chunk % 16 == 0)
        hipLaunchKernelGGL((partial_mfma<NQ, KT, QT, 2, KEEP, WH, NTS>), grid, dim3(64 * kMW), 0, st, a);
    else
        hipLaunchKernelGGL((partial_mfma<NQ, KT, QT, 1, KEEP, WH, NTS>), grid, dim3(64 * kMW), 0, st, a);
    return hipGetLastError();
}

template <int KT, int QT, bool WH>
hipError_t launch_types(int nq, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    if (nq <= 2) return launch_nq<2, KT, QT, WH>(paged, a, grid, st);
    if (nq <= 4) return launch_nq<4, KT, QT, WH>(paged, a, grid, st);
    if (nq <= 8) return launch_nq<8, KT, QT, WH>(paged, a, grid, st);
    if (nq <= 16) return launch_nq<16, KT, QT, WH>(paged, a, grid, st);
    if constexpr (WH) {
        // The column tiles of a head share each staged tile (2 or 4 of them;
        // the planner gives three-tile problems to the other form).
        if (nq <= 32) return launch_nq<16, KT, QT, true, false, 2>(paged, a, grid, st);
        return launch_nq<16, KT, QT, true, false, 4>(paged, a, grid, st);
    } else {
        return launch_nq<16, KT, QT, false, true>(paged, a, grid, st);
    }
}

template <bool WH>
hipError_t launch_mfma(int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    const int nq = G * a.q_len;  // query rows per KV head (16 per column tile)
    if (a.kv_dt == FD_FP8_E4M3)
        return a.q_dt == FD_F16 ? launch_types<FD_FP8_E4M3, FD_F16, WH>(nq, paged, a, grid, st)
                                : launch_types<FD_FP8_E4M3, FD_BF16, WH>(nq, paged, a, grid, st);
    return a.kv_dt == FD_F16 ? launch_types<FD_F16, FD_F16, WH>(nq, paged, a, grid, st)
                             : launch_types<FD_BF16, FD_BF16, WH>(nq, paged, a, grid, st);
}

hipError_t launch_partial_mfma(int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    return launch_mfma<false>(G, paged, a, grid, st);
}

hipError_t launch_partial_mfma_heads(int G, bool paged, const PartialArgs& a, dim3 grid, hipStream_t st) {
    return launch_mfma<true>(G, paged, a, grid, st);
}

}  // namespace fdk
