// Host-side launchers implemented next to their kernels and called by the
// C ABI in rts_api.cpp after argument validation.  Each returns an rts_status.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace rts {

// A rank's owned physical KV rows, emitted by a packed select next to (or
// instead of) the global ids (kernels page: DCPTopkSelectKernel docstring on
// emit_rows, dcp_topk_merge_rows).  rows_out == nullptr: not requested.
struct RowsArgs {
    const int32_t* req_id;       // [rows]
    const int32_t* block_table;  // [table_rows, ld_table]
    int32_t* rows_out;           // [rows, out_cols]
    int32_t* valid_out;          // [rows]
    int64_t table_rows, ld_table, stride_rows;
    int32_t dcp_rank, table_cols, block_size, out_cols;
};

// Launch geometry of topk_rows for one problem shape.
struct TopkPlan {
    int e;          // sorted-list length per lane (list = 64 * e >= k)
    int waves;      // waves per workgroup sharing one row
    int groups;     // workgroups per row (> 1 needs a workspace)
    size_t ws_bytes;
    int block_kpt;  // > 0: whole rows in one workgroup's registers, block_kpt keys per thread
};

// Largest workspace a topk_rows plan uses: partial lists of split rows beyond
// this take fewer groups.  Also the size of topk_rows_noalloc's static scratch.
constexpr size_t kMaxSplitBytes = size_t(16) << 20;

TopkPlan plan_topk_rows(int dtype, int64_t rows, int64_t cols, int32_t k, bool allow_split);

// topk_rows_noalloc's scratch on the current device (its address there, taken
// on the first call on the device) and its size in bytes.
int scratch_of_current_device(void** ptr, size_t* bytes);

int launch_topk_rows(const void* logits, int dtype, int64_t rows, int64_t cols, int64_t ld,
                     const int32_t* row_ends, int32_t k, int32_t* out, int64_t ld_out,
                     const TopkPlan& plan, void* workspace, hipStream_t stream);

int launch_pack_candidates(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                           const int32_t* local_idx, int32_t n, int64_t ld_idx,
                           const int32_t* row_ends, int32_t* packed, hipStream_t stream);

int launch_pack_pairs(const float* x, int64_t rows, int64_t cols, int64_t ld,
                      const int32_t* local_idx, int32_t kc, int64_t ld_idx,
                      const int32_t* row_ends, int32_t rank, int32_t world, int32_t* pairs,
                      hipStream_t stream);

// row_major: gathered is [rows, world, n + n/32] instead of [world, rows, n + n/32].
int launch_merge_packed(const int32_t* gathered, bool row_major, int32_t world, int64_t rows,
                        int32_t n, int32_t k, int32_t* out_ids, int32_t* sat_word,
                        const RowsArgs* rows_args, hipStream_t stream);

// Candidate slots of one rescued row: world * n round-1 words plus k words
// for each of at most min((k-1)/n, world) receive slots.
int rescue_candidates(int32_t world, int32_t n, int32_t k);

int launch_rescue_push(const int32_t* local_packed, int32_t rank, int32_t world, int64_t rows,
                       int32_t n, int32_t k, const int32_t* sat_word, int32_t* recv,
                       hipStream_t stream);

int launch_merge_rescue(const int32_t* gathered, const int32_t* recv, int32_t world, int64_t rows,
                        int32_t n, int32_t k, const int32_t* sat_word, int32_t* out_ids,
                        const RowsArgs* rows_args, hipStream_t stream);

int launch_emit_rows(const int32_t* ids, int64_t rows, int32_t k, int32_t world, int32_t dcp_rank,
                     const int32_t* req_id, const int32_t* block_table, int64_t table_rows,
                     int32_t table_cols, int64_t ld_table, int32_t block_size, int64_t stride_rows,
                     int32_t* rows_out, int32_t out_cols, int32_t* valid_out, hipStream_t stream);

// row_major: pairs is [rows, world * kc, 2] instead of [world, rows, kc, 2].
int launch_merge_pairs(const int32_t* pairs, bool row_major, int32_t world, int64_t rows,
                       int32_t kc, int32_t k, int32_t* out_ids, hipStream_t stream);

}  // namespace rts
