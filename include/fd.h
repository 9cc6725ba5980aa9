/*
 * fd.h - split-KV flash decoding for AMD Instinct MI355X (gfx950).
 *
 * Decode attention for one query token per sequence over a long KV cache:
 *     out[b,h,:] = softmax(scale * K_b q[b,h]) V_b,   lse[b,h] = ln sum_t exp(scale * <q[b,h], K_b[t]>)
 * (the definition in "FlashAttention 全景演进与大模型 Token 生成全链路性能优化实战",
 * §1.1). The cache of each sequence is cut along the token axis into splits of
 * `chunk_tokens` consecutive tokens; each split computes a running max m, a
 * running sum l and an unnormalised partial output O, and a second pass
 * merges the splits by log-sum-exp rescaling (same page, §2.3 FlashDecoding,
 * and §1.2 for the merge identity; also "注意力算子、算子融合与 CUDA Graph",
 * section on decode attention). The merged result is exactly the definition
 * up to floating-point rounding.
 *
 * Layouts (all dense, row-major):
 *   q            [B, Hq, d] (q_len = 1) or [B, q_len, Hq, d], in kv_dtype
 *                (q_dtype for an FP8 cache)
 *   k, v         contiguous: [sum_b L_b, Hkv, d]; sequence b starts at token
 *                row sum_{b'<b} L_b' (a packed variable-length batch).
 *                paged (page_size 16): pools [P, 16, Hkv, d]; token t of
 *                sequence b is at pool[block_table[b, t / 16], t % 16]
 *                (the 16-token physical blocks and per-request block table of
 *                the FlashAttention capstone, §4.1).
 *   block_table  int32 [B, max_pages_per_seq], paged only.
 *   seq_lens     int32 [B], every L_b >= 1.
 *   out          [B, q_len, Hq, d] in out_dtype;  lse  float32 [B, q_len, Hq],
 *                natural log (q_len = 1: [B, Hq, d] and [B, Hq]).
 *   Query head h reads KV head h / (Hq / Hkv) (grouped-query attention with
 *   contiguous groups, capstone §4.2).
 *   Several query tokens per sequence (q_len > 1, the verification pass of
 *   speculative decoding, capstone §4.5) are the last q_len tokens of the
 *   cache: query i of sequence b attends to tokens 0 .. L_b - q_len + i.
 *   An FP8 cache (kv_dtype FD_FP8_E4M3; FP8 attention with fp32 accumulation
 *   and scaling factors is capstone §2.2's FA-3 paragraph) holds OCP E4M3
 *   codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 *   infinities, NaN at S.1111.111, largest finite 448); element (t, g, i)
 *   stands for k_scale[g] * e4m3(k[t, g, i]) (v likewise with v_scale), one
 *   float32 scale per KV head, passed to the *_scaled calls.
 *
 * Ownership: the caller allocates every buffer (device memory for q, k, v,
 * block_table, seq_lens_dev, out, lse and the workspace; host memory for
 * seq_lens_host and the structs). The library allocates no device memory,
 * never frees anything and keeps no state except a per-device cache of the
 * compute-unit count and the fixed per-GPU buffer that
 * fd_decode_attention_noalloc uses in place of a workspace (set aside when the
 * library's code is loaded on a device). It reads the inputs and writes only
 * out, lse and the workspace (or that buffer).
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 * stream). Every call that takes one only enqueues work on it and returns;
 * results are ready once the stream is synchronised. Calls made on one stream
 * with one workspace are ordered; using one workspace from two streams at once
 * races.
 *
 * Errors: no C++ exception crosses this interface. Every call returns an
 * fd_status; on failure fd_last_error_message() (per thread) says why.
 * Argument checks happen on the host before anything is enqueued, so a call
 * that returns an error has launched nothing. The kernels bound every
 * workspace access by the plan and every paged access by max_pages_per_seq,
 * but they cannot check device lengths against the caller's contiguous cache
 * size.
 *
 * Plans and device lengths: each device length must be at least 1 and at
 * most the host length the plan was made from (equal in the common case).
 * The kernels derive every sequence's splits from the device lengths, and
 * work-groups past the resulting work list exit at once, so a plan made for
 * upper-bound lengths serves every later step within those bounds: partial +
 * combine can be captured once in a HIP graph and replayed while the
 * sequences grow, only the contents of seq_lens_dev (and of the cache)
 * changing. A contiguous cache is packed by the device lengths.
 */
#ifndef FD_H
#define FD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fd_status {
    FD_OK = 0,
    FD_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, inconsistent shapes */
    FD_ERR_UNSUPPORTED = 2,        /* valid but not built: head_dim, page size, group size */
    FD_ERR_WORKSPACE_TOO_SMALL = 3,
    FD_ERR_HIP = 4                 /* the HIP runtime reported an error (launch, device query) */
} fd_status;

typedef enum fd_dtype {
    FD_F16 = 0,
    FD_BF16 = 1,
    FD_F32 = 2,
    FD_FP8_E4M3 = 3            /* OCP E4M3 codes, KV cache only */
} fd_dtype;

/* The problem shape. q, k and v share `kv_dtype`, except that q of an FP8
 * cache is in `q_dtype`. */
typedef struct fd_problem {
    int32_t batch;             /* B >= 1 */
    int32_t num_q_heads;       /* Hq >= 1 */
    int32_t num_kv_heads;      /* Hkv >= 1, divides Hq; Hq/Hkv in {1, 2, 4, 8} */
    int32_t head_dim;          /* d in {64, 128} */
    int32_t kv_dtype;          /* FD_F16, FD_BF16 or FD_FP8_E4M3 */
    int32_t out_dtype;         /* FD_F32, FD_F16 or FD_BF16 */
    float scale;               /* softmax scale; <= 0 selects 1/sqrt(d) */
    int32_t page_size;         /* 0 = contiguous packed cache, 16 = paged */
    int32_t max_pages_per_seq; /* paged: columns of block_table; ignored otherwise */
    int32_t q_len;             /* query tokens per sequence, 0 or 1 = one; q_len > 1 needs d = 128
                                  and q_len * Hq/Hkv <= 64, and every L_b >= q_len */
    int32_t q_dtype;           /* FP8 cache: q's type, FD_F16 or FD_BF16; ignored otherwise */
    int32_t num_pages;         /* paged: pages in the pool (0 = do not check page indices); a
                                  table entry outside [0, num_pages) then reads page 0 instead */
} fd_problem;

/* How the splits are cut. Holds scalars only: nothing is uploaded per call,
 * and each kernel derives a sequence's splits from the device seq_lens.
 *
 * split_mode 0 (per sequence): split s of sequence b holds tokens
 * [s*C, min((s+1)*C, L_b)), so S_b = ceil(L_b / C).
 * split_mode 1 (balanced, ragged batches on the matrix-core kernel): the
 * sequences, in order, take consecutive positions of one list: 4 positions
 * for the cost of starting a share (pipeline start, wave merge, store), then
 * one per 16-token tile, n_b = ceil(L_b / 16) of them. So sequence b's first
 * tile sits at T_b = 4*(b+1) + n_0 + ... + n_{b-1}. Work item w takes
 * positions [w*P, (w+1)*P) of the list, P = C / 16, across sequence
 * boundaries, so every work-group has the same work whatever the length mix.
 * Split s of sequence b is its share of item floor(T_b / P) + s: tokens
 * [16*max(0, (floor(T_b/P)+s)*P - T_b), min(L_b, 16*((floor(T_b/P)+s+1)*P - T_b))),
 * and S_b = floor((T_b + n_b - 1) / P) - floor(T_b / P) + 1 <= ceil(n_b / P) + 1. */
typedef struct fd_plan {
    int32_t chunk_tokens;      /* C: tokens per split (mode 0) or per work item (mode 1, a multiple of 16) */
    int32_t max_splits;        /* S_max: workspace stride, >= every S_b (mode 0: max_b ceil(L_b / C);
                                  mode 1: ceil(max_b n_b / P) + 1) */
    int32_t total_splits;      /* work-list entries per KV-head group: sum_b ceil(L_b / C) (mode 0),
                                  or ceil(sum_b (n_b + 4) / P) work items (mode 1) */
    int32_t num_cus;           /* compute units the plan was sized for */
    int32_t partial_kernel;    /* which partial kernel runs (0 = vector ALU token rows, 1 = MFMA,
                                  2 = vector ALU head rows, 3 = vector ALU head columns,
                                  4 = MFMA with each wave owning a head) */
    int32_t split_mode;        /* 0 = per-sequence chunks, 1 = balanced list (partial_kernel 1 or 4) */
    int64_t total_tokens;      /* sum_b L_b */
    uint64_t workspace_bytes;  /* bytes the workspace must hold */
} fd_plan;

/*
 * Size the splits for one batch (host only).
 *
 * One head per processor starves a GPU with few KV heads, so each sequence is
 * cut into chunks (FlashAttention capstone §2.3, which gives 256 tokens as an
 * example chunk). The planner tries chunks that make about num_cus * k
 * work-groups (sequence, KV head, split) for k = 1, 2, 3, 4, 6, 8, ... and
 * keeps the largest one whose full-size splits alone give every compute unit
 * two work-groups (three when shorter last splits exist; twice that for the
 * token-rows kernel on an FP8 cache; four work-groups per compute unit
 * directly for the matrix-core kernel with four column tiles) while at most
 * an eighth of the tokens fall in shorter last splits. Chunks are multiples of
 * 64 and at least 256 tokens (1024 for the kernel whose work-groups cover
 * several heads, 2048 when the cache is FP8; when that kernel's
 * work-groups would be fewer than the compute units its chunk is halved, down
 * to 256 tokens, and only if that still leaves too few does the plan fall back
 * to one head per work-group).
 * A batch of unequal lengths on the matrix-core kernel (at most 4096
 * sequences, no forced split count) gets split_mode 1 instead:
 * P = max(16, ceil(sum_b (n_b + 4) * W / (num_cus * k))) positions per work
 * item (n_b = ceil(L_b / 16) tiles, W the work-groups per item), i.e. about k
 * work-groups per compute unit, all of them the same size: k = 4 for the
 * kernel with each wave owning a head and four column tiles, 1 for that
 * kernel with one column tile on a 16-bit cache, 3 for an FP8 cache on the
 * kernel whose waves share a head, 2 otherwise.
 * `force_num_splits` > 0 instead sets C = ceil(max_b L_b / force) and accepts
 * any C >= 1 (split_mode 0). `num_cus` == 0 asks the current HIP device (the only HIP call
 * here; its count is cached per device). Validates the problem and every
 * length (1 <= L_b, and L_b <= max_pages_per_seq * 16 when paged).
 * seq_lens_host: B lengths in host memory. out: receives the plan.
 * The environment variables FD_NUM_SPLITS (forces splits when the argument
 * is 0), FD_MIN_CHUNK, FD_WG_PER_CU (fixes k, or the work-groups per compute
 * unit of split_mode 1), FD_PARTIAL_KERNEL (0 to 4) and FD_SPLIT_MODE (0 or
 * 1, where the balanced mode applies) override these choices for experiments.
 */
fd_status fd_plan_splits(const fd_problem* problem, const int32_t* seq_lens_host,
                         int32_t num_cus, int32_t force_num_splits, fd_plan* out);

/*
 * Per-split partials (asynchronous on `stream`).
 *
 * For every sequence b, query row r (= i * Hq + h for query token i and head
 * h) and split s < S_b writes the split's running max
 * m_s = max_t scale*<q, k_t>, sum l_s = sum_t exp(scale*<q,k_t> - m_s) and
 * unnormalised output O_s = sum_t exp(scale*<q,k_t> - m_s) v_t over the
 * split's tokens t (with split_mode 0, [s*C, min((s+1)*C, L_b)); with
 * split_mode 1, the range fd_plan describes) that the query may see (the
 * per-chunk local softmax of capstone §2.3; the running-statistics loop of
 * the lpnh.cn memory-wall article, §2.2). A split holding no such token gets
 * m_s = -inf, l_s = 0, O_s = 0. Tokens at or past L_b are never read.
 *
 * Workspace layout (float32, all of it written by the kernels, so the caller
 * never initialises it):
 *   O  [B, q_len*Hq, S_max, d]     at byte offset 0
 *   ML [B, q_len*Hq, S_max, 2]     after O: (m_s, l_s) pairs, m_s in
 *                                  natural-log units of the scaled score.
 *   counters uint32 [B, Hkv]       at the next 16-byte boundary; used only by
 *                                  fd_decode_fused.
 * Entries of splits a sequence does not have are left untouched.
 * q, k, v, block_table (NULL when contiguous), seq_lens_dev: device pointers.
 * q, k and v must be 16-byte aligned. An FP8 cache takes fd_decode_partial_scaled.
 */
fd_status fd_decode_partial(const fd_problem* problem, const fd_plan* plan,
                            const void* q, const void* k, const void* v,
                            const int32_t* block_table, const int32_t* seq_lens_dev,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * fd_decode_partial with per-KV-head dequantisation scales: the cache element
 * (t, g, i) stands for k_scale[g] * k[t, g, i] (and v_scale[g] * v[t, g, i]).
 * k_scale, v_scale: device float32 [Hkv], finite; NULL means all ones. The
 * kernels fold k_scale[g] into the score scale and v_scale[g] into the
 * split's O_s, so m_s, l_s and O_s are those of the dequantised cache.
 * Required for kv_dtype FD_FP8_E4M3 (NULL scales are then allowed and mean
 * the codes' own values); accepted for 16-bit caches too.
 */
fd_status fd_decode_partial_scaled(const fd_problem* problem, const fd_plan* plan,
                                   const void* q, const void* k, const void* v,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, const int32_t* seq_lens_dev,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Partials and merge in one kernel launch (asynchronous on `stream`): every
 * work-group writes its split's partial exactly as fd_decode_partial does;
 * the last work-group of each (sequence, KV-head group) to finish then merges
 * that group's splits as fd_combine does and writes out and lse. "Last" is
 * decided by an arrival counter per (sequence, KV head) kept at the end of
 * the workspace (the plan's workspace_bytes includes it): the counters must
 * be zero before the first call on a workspace (fd_workspace_init), and every
 * completed call leaves them zero again, so later calls, graph replays
 * included, need no initialisation. No work-group waits for another. Calls
 * that share a workspace must not overlap. Same arguments as
 * fd_decode_partial_scaled (scales NULL for a 16-bit cache without scales),
 * plus out and lse as for fd_combine.
 * Cost: every work-group releases its partial at device scope before it
 * arrives (on gfx950 an L2 write-back per wave), which costs more than the
 * saved launch once there are more than a few dozen work-groups. Measured on
 * MI355X: 1024 tokens x 8 heads 19.2 -> 12.7 us per step; 32K-token MHA
 * 86.5 -> 105.8 us; 128K-token MHA 322.5 -> 393.8 us. Use it for small,
 * launch-bound steps; fd_decode_partial + fd_combine otherwise.
 */
fd_status fd_decode_fused(const fd_problem* problem, const fd_plan* plan,
                          const void* q, const void* k, const void* v,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_table, const int32_t* seq_lens_dev,
                          void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Zero the arrival counters of a workspace for fd_decode_fused (a small
 * kernel on `stream`, no memset, so it may be recorded in a graph). Needed
 * once per workspace allocation.
 */
fd_status fd_workspace_init(const fd_problem* problem, const fd_plan* plan, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Merge the partials (asynchronous on `stream`).
 *
 * For every (b, query row): M = max_s m_s, w_s = exp(m_s - M),
 * l = sum_s w_s l_s, out = sum_s w_s O_s / l and lse = M + ln l (the
 * cross-chunk reduce of capstone §2.3, by the two-block identity of §1.2
 * applied to every split). out: device [B, q_len, Hq, d] in out_dtype.
 * lse: device float32 [B, q_len, Hq], or NULL. Batches of 1024 query rows or
 * more (B * q_len * Hq) merge one row per wave, from 4096 rows two rows per
 * wave (when a sequence has an even number of rows), smaller batches with
 * four waves per row, or sixteen when the plan has 128 splits or more;
 * FD_COMBINE_FORM (0 four waves per row, 1 one wave per row, 2 two rows per
 * wave, 3 sixteen waves per row) forces one, for experiments.
 */
fd_status fd_combine(const fd_problem* problem, const fd_plan* plan,
                     const int32_t* seq_lens_dev, const void* workspace,
                     size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * One call: plan (with num_cus = 0 and no forced split count), partials,
 * merge. Returns FD_ERR_WORKSPACE_TOO_SMALL, having launched nothing, if
 * workspace_bytes is below the plan's need; size the workspace with
 * fd_plan_splits beforehand. seq_lens_host and seq_lens_dev hold the same B
 * lengths, in host and device memory.
 */
fd_status fd_decode_attention(const fd_problem* problem,
                              const void* q, const void* k, const void* v,
                              const int32_t* block_table,
                              const int32_t* seq_lens_host, const int32_t* seq_lens_dev,
                              void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/* fd_decode_attention with the per-KV-head scales of fd_decode_partial_scaled. */
fd_status fd_decode_attention_scaled(const fd_problem* problem,
                                     const void* q, const void* k, const void* v,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_table,
                                     const int32_t* seq_lens_host, const int32_t* seq_lens_dev,
                                     void* out, float* lse,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of partials fd_decode_attention_noalloc can hold on each GPU (64 MiB). */
#define FD_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/*
 * fd_decode_attention_scaled without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The partials go to a buffer the
 * library holds in device memory, FD_NOALLOC_WORKSPACE_BYTES on every GPU it
 * runs on, until the process ends; the call itself allocates and frees
 * nothing. Same plan, kernels and results as fd_decode_attention_scaled
 * (k_scale and v_scale NULL for a 16-bit cache without scales); the caller
 * still passes the inputs and out / lse.
 * Errors: FD_ERR_WORKSPACE_TOO_SMALL, having launched nothing, when the plan's
 * workspace_bytes (fd_plan_splits) exceed FD_NOALLOC_WORKSPACE_BYTES; FD_ERR_HIP
 * if the buffer's address cannot be found on the current device.
 * Sharing: every call on one GPU uses that GPU's one buffer. Calls on one
 * stream are ordered; calls that overlap on one GPU (two streams, or two host
 * threads with different streams) race on it. Nothing in the buffer needs
 * clearing: the partial kernel writes every slot the merge reads.
 */
fd_status fd_decode_attention_noalloc(const fd_problem* problem,
                                      const void* q, const void* k, const void* v,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table,
                                      const int32_t* seq_lens_host, const int32_t* seq_lens_dev,
                                      void* out, float* lse, void* stream);

/*
 * Prefill attention (asynchronous on `stream`): every one of the q_len query
 * tokens of each sequence attends causally to its cache, in one pass with no
 * splits and no workspace.
 *
 * The FlashAttention-2 forward pass (FlashAttention capstone, §2.1): blocks
 * of 128 query rows stay on chip while K/V tiles stream past; each row keeps
 * a running max and sum, the output is divided once at the end, and tiles
 * wholly past a block's causal limit are skipped. Query i of sequence b is at
 * position L_b - q_len + i and sees tokens 0 .. L_b - q_len + i (q_len = L_b:
 * causal self-attention over the whole prompt; smaller q_len: one chunk of a
 * longer prompt whose earlier tokens are already cached), the same reading
 * as multi-query decode. Arithmetic: q.k products in the cache's type and
 * P.V products in fp16 (P rounded to fp16; a bf16 V tile converted to fp16,
 * scaled by a power of two when it holds a value past 65504), all
 * accumulated in fp32.
 * problem: head_dim 128, fp16/bf16 cache (q of the same type), contiguous or
 *          paged, q_len >= 1 new tokens per sequence (no upper limit), every
 *          L_b >= q_len (a row with no visible token gets out = 0,
 *          lse = -inf).
 * q: device [B, q_len, Hq, d]; k, v: the cache as for fd_decode_partial;
 * out: device [B, q_len, Hq, d] in out_dtype; lse: device float32
 * [B, q_len, Hq] or NULL.
 */
fd_status fd_prefill_attention(const fd_problem* problem, const void* q, const void* k, const void* v,
                               const int32_t* block_table, const int32_t* seq_lens_dev,
                               void* out, float* lse, void* stream);

/* Rotary position embedding applied by fd_append_kv. */
typedef enum fd_rope_style {
    FD_ROPE_NONE = 0,          /* store the new keys as given */
    FD_ROPE_INTERLEAVED = 1,   /* pairs (2i, 2i+1) */
    FD_ROPE_HALF = 2           /* pairs (i, i + d/2) */
} fd_rope_style;

/*
 * Append each sequence's q_len new tokens to a paged cache (asynchronous on
 * `stream`), rotating the new keys and the queries by their positions first.
 *
 * RoPE belongs before split-KV decode, in a kernel of its own, and applies to
 * the current step's keys and queries (CUTLASS Split KV article, §5.3); the
 * cache is the capstone's 16-token paged layout (§4.1). With the lengths L_b
 * counted *after* the append (the lengths the following decode call uses),
 * new token j of sequence b is at position pos = L_b - q_len + j, stored at
 * k_cache[block_table[b, pos / 16], pos % 16] (v_cache likewise). Rotation
 * (RoFormer's rotary embedding): pair i of each head vector turns by
 * pos * rope_base^(-2i/d); computed in fp64, then rounded once to the storage
 * format (ties to even). An FP8 cache stores the E4M3 code of value / scale[g]
 * saturated at +-448 (k_scale / v_scale as for fd_decode_partial_scaled; NULL
 * means 1; 16-bit caches divide by the scales too when given).
 *
 * problem: paged (page_size 16) with batch, heads, head_dim, kv_dtype,
 *          q_dtype and q_len (new tokens per sequence, 0 or 1 = one).
 * k_new, v_new: device [B, q_len, Hkv, d] in q's type (kv_dtype for 16-bit
 *          caches, q_dtype for FP8 caches).
 * q:       device [B, q_len, Hq, d], rotated in place; NULL to leave out.
 * k_cache, v_cache: device pools [num_pages, 16, Hkv, d] in kv_dtype.
 * block_table: device int32 [B, max_pages_per_seq]; seq_lens_dev: device
 *          int32 [B] (after the append).
 * Alignment: k_new, v_new, q and 16-bit caches 16 bytes, FP8 caches 8 bytes
 * (whole rows move in 16-byte pieces); FD_ERR_INVALID_ARGUMENT otherwise.
 * Slots other than the new tokens' are not touched. A position outside the
 * block table, or a page index outside [0, num_pages), is skipped on the
 * device (nothing written) rather than trusted. rope_style FD_ROPE_NONE
 * stores keys unrotated and leaves q alone; otherwise rope_base must be a
 * positive finite number (10000 in RoFormer).
 */
fd_status fd_append_kv(const fd_problem* problem, int32_t rope_style, float rope_base,
                       const void* k_new, const void* v_new, void* q,
                       const float* k_scale, const float* v_scale,
                       void* k_cache, void* v_cache, int32_t num_pages,
                       const int32_t* block_table, const int32_t* seq_lens_dev, void* stream);

/* A static, human-readable name for a status code. */
const char* fd_status_string(fd_status status);

/* The message of the last failed call on this thread ("" if none). */
const char* fd_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_H */
