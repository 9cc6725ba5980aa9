// Internal declarations shared by the host planner (fd_host.cpp) and the
// entry points and kernel files (fd_api.hip, fd_partial_*.hip, ...). Not part
// of the public interface.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fd.h"

namespace fd {

// Largest batch (the combine kernel's grid y extent) and largest number of
// splits of one sequence (the workspace's split stride) accepted.
constexpr int32_t kMaxGridYZ = 65535;
// Token rows a partial-kernel work-group consumes per pass (the planner keeps
// automatic chunks a multiple of it).
constexpr int32_t kChunkGranule = 64;
constexpr int32_t kDefaultMinChunk = 256;
constexpr int32_t kHeadRowsMinChunk = 1024;
// The shortest head-rows split the planner takes to give every CU a
// work-group before it falls back to token rows.
constexpr int32_t kHeadRowsFloorChunk = 256;
constexpr int32_t kPageSize = 16;
// Balanced split mode (fd_plan.split_mode 1): tokens per tile of the list,
// the smallest work item in tiles (256 tokens), the work-groups per compute
// unit it aims at, and the largest batch it is chosen for (the combine walks
// the lengths before its sequence). Work-groups per compute unit: two, fewer
// and longer items, for the matrix-core kernel whose waves own heads, 16-bit
// and FP8 caches alike (an FP8 wave keeps two tiles in flight; measured on
// MI355X, same GPU, three against two: GQA varlen 66.6 -> 62.3 us, paged GQA
// 177.4 -> 172.6 us); three for an FP8 cache on the kernel whose waves share
// a head (its occupancy).
constexpr int32_t kTileTokens = 16;
constexpr int32_t kBalancedMinTiles = 16;
constexpr int32_t kBalancedWgPerCu16 = 2;
constexpr int32_t kBalancedWgPerCuFp8 = 3;
// One work-group per compute unit (one wave per SIMD) for that kernel with a
// single column tile on a 16-bit cache: half as many, twice as long items,
// so half the share starts and splits to merge (measured on MI355X, same GPU,
// one against two: paged GQA 318.2 against 328.8 us per step, the same with 2
// query tokens 330.3 against 343.2, GQA varlen 110.7 against 111.9, with 2 and
// 4 query tokens 113.2 against 116.0 and 116.7 against 121.5-121.9). FP8
// caches (GQA varlen with 2 query tokens 74.9 against 67.4 us) and two column
// tiles (paged GQA with 4 query tokens 460.1 against 349.6 us) keep two.
constexpr int32_t kBalancedWgPerCuSingle16 = 1;
// The matrix-core kernel with waves owning heads and four column tiles (49 to
// 64 query rows per KV head) does four times the matrix work per byte of a
// single tile and fits four work-groups per compute unit: it wants them all,
// whatever the split mode (measured on MI355X, same GPU, three against four:
// paged GQA with 8 query tokens 406.7 -> 388.8 us, 128K-token MHA with 64
// query tokens 402.8 -> 382.1 us; two column tiles lose with more than two:
// GQA varlen with 8 query tokens 121.3 -> 123.2 (three) and 128.2 us (four)).
constexpr int32_t kWideMultiQueryWgPerCu = 4;
constexpr int32_t kBalancedMaxBatch = 4096;
// List positions a sequence takes before its tiles in the balanced list: the
// cost of starting a share (the pipeline's first loads, the wave merge and the
// partial's store), in tiles, so an item that holds many short sequences gets
// fewer tiles.
#ifndef FD_SHARE_COST
#define FD_SHARE_COST 4
#endif
constexpr int32_t kShareCost = FD_SHARE_COST;

// Records `msg` as this thread's last error and returns `st`.
fd_status fail(fd_status st, const char* fmt, ...);
void clear_error();

// Checks the problem fields (not the lengths). Resolves the scale.
fd_status check_problem(const fd_problem* p, float* scale_out);
// Checks a plan against the problem it is used with.
fd_status check_plan(const fd_problem* p, const fd_plan* plan);

// Workspace layout: O [B, q_len*Hq, S_max, d] then ML [B, q_len*Hq, S_max, 2],
// float32, then the fused merge's arrival counters, uint32 [B, Hkv], at a
// 16-byte aligned offset.
uint64_t workspace_o_bytes(const fd_problem* p, int32_t max_splits);
uint64_t workspace_counters_offset(const fd_problem* p, int32_t max_splits);
uint64_t workspace_bytes(const fd_problem* p, int32_t max_splits);

// The combine's form: 0 four waves per (sequence, query row); 3 sixteen waves
// per row, for those batches when rows have kCombineWideSplits splits or more;
// 1 one wave per row, for batches of at least kCombinePerWaveRows rows
// (measured on MI355X: 512 rows of up to 25 splits merge in 2.0-2.6 us with
// four waves per row, 3.7-4.5 us with one)
// (B * q_len * Hq), where four waves per row would take several rounds of the
// chip's wave slots; 2 two rows per wave, from kCombineTwoRowRows rows when a
// sequence has an even number of rows. FD_COMBINE_FORM=0/1/2/3 overrides (2
// only with even rows per sequence).
constexpr int64_t kCombinePerWaveRows = 1024;
constexpr int64_t kCombineTwoRowRows = 4096;
constexpr int32_t kCombineWideSplits = 128;
int32_t combine_form(const fd_problem* p, int32_t max_splits);

// Compute units of the current HIP device, cached per device (fd_api.hip).
fd_status query_num_cus(int32_t* out);

// Partial kernels a plan can select.
enum PartialKernel : int32_t {
    kPartialTokenRows = 0,  // vector ALU, lane rows are tokens of one KV head
    kPartialMfma = 1,       // matrix cores, grouped-query heads
    kPartialHeadRows = 2,   // vector ALU, lane rows are consecutive KV heads, waves split the tokens
    kPartialHeadCols = 3,   // vector ALU, lane rows are consecutive KV heads, waves split the heads
    kPartialMfmaHeads = 4,  // matrix cores, each wave owns one (KV head, column tile) of the work-group
};

// Whether a kernel is one of the two matrix-core forms.
inline bool is_mfma_kernel(int32_t kernel) { return kernel == kPartialMfma || kernel == kPartialMfmaHeads; }

// Query tokens per sequence (a q_len of 0 means one).
inline int32_t problem_q_len(const fd_problem* p) { return p->q_len > 1 ? p->q_len : 1; }
// Largest q_len * Hq/Hkv the matrix-core kernel handles (up to four 16-column
// MFMA tiles, one work-group each).
constexpr int32_t kMaxQueryRows = 64;
// Waves per work-group of the matrix-core kernel (fd_partial_mfma.hip).
constexpr int32_t kMfmaWaves = 4;

// Bytes of one cache element (2 for fp16/bf16, 1 for E4M3).
inline int32_t kv_elem_bytes(const fd_problem* p) { return p->kv_dtype == FD_FP8_E4M3 ? 1 : 2; }
// q's element type: the cache's, or q_dtype for an FP8 cache.
inline int32_t q_dtype_of(const fd_problem* p) { return p->kv_dtype == FD_FP8_E4M3 ? p->q_dtype : p->kv_dtype; }

// Token rows (head rows) one 16-byte wave-wide load covers: 64 lanes over
// d * bytes / 16 lanes per row.
inline int32_t rows_per_load(const fd_problem* p) { return 64 / (p->head_dim * kv_elem_bytes(p) / 16); }

// Waves per work-group of the head-columns kernel (fd_partial_valu.hip):
// eight for 16-bit caches, four for FP8. (Head rows always run eight; a
// head-rows work-group covers rows_per_load heads whatever its waves.)
inline int32_t head_cols_waves(const fd_problem* p) { return kv_elem_bytes(p) == 1 ? 4 : 8; }

// Whether the matrix-core partial kernel covers this problem: d = 128 and
// 2 <= q_len * Hq/Hkv <= kMaxQueryRows query rows per KV head.
bool mfma_applicable(const fd_problem* p);
// Whether the matrix-core kernel with waves owning heads covers it: as the
// matrix-core kernel, with 1, 2 or 4 column tiles (so the four waves of a
// work-group hold whole heads) and Hkv a multiple of the heads per work-group.
bool mfma_heads_applicable(const fd_problem* p);
// Whether the head-rows kernel covers it: one query token, G <= 2 and Hkv a
// multiple of the rows one load covers.
bool head_rows_applicable(const fd_problem* p);
// Whether the head-columns kernel covers it: as head rows, with Hkv a multiple
// of the heads all waves of a work-group cover together.
bool head_cols_applicable(const fd_problem* p);
// KV heads one work-group of `kernel` handles.
int32_t heads_per_workgroup(const fd_problem* p, int32_t kernel);
// Work-groups per split of one sequence: KV-head groups times the matrix-core
// kernel's column tiles.
int32_t workgroups_per_split(const fd_problem* p, int32_t kernel);
// Column tiles (16 query rows each) of the matrix-core kernel.
inline int32_t mfma_column_tiles(const fd_problem* p) {
    return (problem_q_len(p) * (p->num_q_heads / p->num_kv_heads) + 15) / 16;
}

}  // namespace fd
