// The C ABI of row_top_select: argument validation on the host (nothing is
// launched on a bad call, in the spirit of the host checks of _check_exact on
// the kernels page of vllm.models.kimi_k3.nvidia.ops.dcp_topk_merge), then the
// launchers next to the kernels.  No allocation, no synchronisation.
#include "../../include/row_top_select.h"

#include <stdint.h>

#include "rts_internal.h"

namespace {

constexpr int32_t kMaxK = 2048;
constexpr int64_t kMaxGrid = 0x7FFFFFFFll;
constexpr int64_t kMaxCandidates = 32768;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

const char* rts_status_string(int status) {
    switch (status) {
        case RTS_OK: return "RTS_OK";
        case RTS_EINVAL: return "RTS_EINVAL: invalid argument";
        case RTS_EUNSUPPORTED: return "RTS_EUNSUPPORTED: request outside this build's limits";
        case RTS_EWORKSPACE: return "RTS_EWORKSPACE: workspace smaller than required";
        case RTS_EHIP: return "RTS_EHIP: HIP launch failed";
        default: return "unknown rts_status";
    }
}

size_t topk_rows_workspace_size(int dtype, int64_t rows, int64_t cols, int32_t k) {
    if ((dtype != RTS_F32 && dtype != RTS_BF16) || rows < 0 || cols < 0 || k < 1 || k > kMaxK)
        return 0;
    return rts::plan_topk_rows(dtype, rows, cols, k, true).ws_bytes;
}

int topk_rows(const void* logits, int dtype, int64_t rows, int64_t cols, int64_t ld_logits,
              const int32_t* row_ends, int32_t k, int32_t* out_idx, int64_t ld_out, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
    if (dtype != RTS_F32 && dtype != RTS_BF16) return RTS_EINVAL;
    if (rows < 0 || cols < 0 || ld_logits < cols || ld_logits < 0 || k < 1 || ld_out < k)
        return RTS_EINVAL;
    if (k > kMaxK || cols > 0x7FFFFFFFll) return RTS_EUNSUPPORTED;
    if (rows == 0) return RTS_OK;
    if (!out_idx || (cols > 0 && !logits)) return RTS_EINVAL;
    const size_t esz = dtype == RTS_F32 ? 4 : 2;
    if (!aligned(logits, esz) || !aligned(out_idx, 4) || (row_ends && !aligned(row_ends, 4)))
        return RTS_EINVAL;
    if (workspace_bytes > 0 && !workspace) return RTS_EINVAL;
    const bool have_ws = workspace != nullptr;
    rts::TopkPlan plan = rts::plan_topk_rows(dtype, rows, cols, k, have_ws);
    if (have_ws && workspace_bytes < plan.ws_bytes) return RTS_EWORKSPACE;
    if (have_ws && !aligned(workspace, 8)) return RTS_EINVAL;
    if (rows * plan.groups > kMaxGrid) return RTS_EUNSUPPORTED;
    return rts::launch_topk_rows(logits, dtype, rows, cols, ld_logits, row_ends, k, out_idx, ld_out,
                                 plan, workspace, stream);
}

int topk_rows_noalloc(const void* logits, int dtype, int64_t rows, int64_t cols, int64_t ld_logits,
                      const int32_t* row_ends, int32_t k, int32_t* out_idx, int64_t ld_out,
                      hipStream_t stream) {
    if (dtype != RTS_F32 && dtype != RTS_BF16) return RTS_EINVAL;
    if (rows < 0 || cols < 0 || ld_logits < cols || ld_logits < 0 || k < 1 || ld_out < k)
        return RTS_EINVAL;
    if (k > kMaxK || cols > 0x7FFFFFFFll) return RTS_EUNSUPPORTED;
    if (rows == 0) return RTS_OK;
    if (!out_idx || (cols > 0 && !logits)) return RTS_EINVAL;
    const size_t esz = dtype == RTS_F32 ? 4 : 2;
    if (!aligned(logits, esz) || !aligned(out_idx, 4) || (row_ends && !aligned(row_ends, 4)))
        return RTS_EINVAL;
    rts::TopkPlan plan = rts::plan_topk_rows(dtype, rows, cols, k, true);
    void* scratch = nullptr;
    if (plan.groups > 1) {
        size_t bytes = 0;
        const int rc = rts::scratch_of_current_device(&scratch, &bytes);
        if (rc != RTS_OK) return rc;
        if (plan.ws_bytes > bytes) return RTS_EWORKSPACE;
    }
    if (rows * plan.groups > kMaxGrid) return RTS_EUNSUPPORTED;
    return rts::launch_topk_rows(logits, dtype, rows, cols, ld_logits, row_ends, k, out_idx, ld_out,
                                 plan, scratch, stream);
}

int pack_candidates(const uint16_t* logits_bf16, int64_t rows, int64_t cols, int64_t ld_logits,
                    const int32_t* local_idx, int32_t n, int64_t ld_idx, const int32_t* row_ends,
                    int32_t* packed, hipStream_t stream) {
    if (rows < 0 || cols < 0 || ld_logits < cols || n < 32 || n % 32 != 0 || ld_idx < n)
        return RTS_EINVAL;
    if (rows == 0) return RTS_OK;
    if (!logits_bf16 || !local_idx || !packed) return RTS_EINVAL;
    if (!aligned(logits_bf16, 2) || !aligned(local_idx, 4) || !aligned(packed, 4) ||
        (row_ends && !aligned(row_ends, 4)))
        return RTS_EINVAL;
    if ((rows * (int64_t)n + 255) / 256 > kMaxGrid) return RTS_EUNSUPPORTED;
    return rts::launch_pack_candidates(logits_bf16, rows, cols, ld_logits, local_idx, n, ld_idx,
                                       row_ends, packed, stream);
}

namespace {
int merge_packed_checked(const int32_t* gathered, bool row_major, int32_t world, int64_t rows,
                         int32_t n, int32_t k, int32_t* out_ids, int32_t* sat_word,
                         hipStream_t stream) {
    if (world < 1 || world > 16 || rows < 0 || n < 32 || n % 32 != 0 || k < 1) return RTS_EINVAL;
    if (k > kMaxK || (int64_t)world * n > kMaxCandidates || rows > kMaxGrid) return RTS_EUNSUPPORTED;
    if (rows == 0) return RTS_OK;
    if (!gathered || !out_ids) return RTS_EINVAL;
    if (!aligned(gathered, 4) || !aligned(out_ids, 4) || (sat_word && !aligned(sat_word, 4)))
        return RTS_EINVAL;
    return rts::launch_merge_packed(gathered, row_major, world, rows, n, k, out_ids, sat_word, nullptr,
                                    stream);
}

int merge_pairs_checked(const int32_t* gathered_pairs, bool row_major, int32_t world, int64_t rows,
                        int32_t kc, int32_t k, int32_t* out_ids, hipStream_t stream) {
    if (world < 1 || rows < 0 || kc < 1 || k < 1) return RTS_EINVAL;
    if (k > kMaxK || (int64_t)world * kc > kMaxCandidates || rows > kMaxGrid) return RTS_EUNSUPPORTED;
    if (rows == 0) return RTS_OK;
    if (!gathered_pairs || !out_ids) return RTS_EINVAL;
    if (!aligned(gathered_pairs, 8) || !aligned(out_ids, 4)) return RTS_EINVAL;
    return rts::launch_merge_pairs(gathered_pairs, row_major, world, rows, kc, k, out_ids, stream);
}
}  // namespace

int merge_select_rank_major(const int32_t* gathered, int32_t world, int64_t rows, int32_t n,
                            int32_t k, int32_t* out_ids, int32_t* sat_word, hipStream_t stream) {
    return merge_packed_checked(gathered, false, world, rows, n, k, out_ids, sat_word, stream);
}

int merge_select_row_major(const int32_t* gathered, int32_t world, int64_t rows, int32_t n, int32_t k,
                           int32_t* out_ids, int32_t* sat_word, hipStream_t stream) {
    return merge_packed_checked(gathered, true, world, rows, n, k, out_ids, sat_word, stream);
}

int rescue_push(const int32_t* local_packed, int32_t rank, int32_t world, int64_t rows, int32_t n,
                int32_t k, const int32_t* sat_word, int32_t* recv, hipStream_t stream) {
    if (world < 1 || world > 16 || rank < 0 || rank >= world || rows < 0 || n < 32 || n % 32 != 0 ||
        k < 32 || k % 32 != 0)
        return RTS_EINVAL;
    if (k > kMaxK || (rows + 3) / 4 > kMaxGrid) return RTS_EUNSUPPORTED;
    if (rows == 0 || (k - 1) / n == 0) return RTS_OK;
    if (!local_packed || !sat_word || !recv) return RTS_EINVAL;
    if (!aligned(local_packed, 4) || !aligned(sat_word, 4) || !aligned(recv, 4)) return RTS_EINVAL;
    return rts::launch_rescue_push(local_packed, rank, world, rows, n, k, sat_word, recv, stream);
}

int merge_rescue_rank_major(const int32_t* gathered, const int32_t* recv, int32_t world, int64_t rows,
                            int32_t n, int32_t k, const int32_t* sat_word, int32_t* out_ids,
                            hipStream_t stream) {
    if (world < 1 || world > 16 || rows < 0 || n < 32 || n % 32 != 0 || k < 32 || k % 32 != 0)
        return RTS_EINVAL;
    if (k > kMaxK || rts::rescue_candidates(world, n, k) > kMaxCandidates || rows > kMaxGrid)
        return RTS_EUNSUPPORTED;
    if (rows == 0 || (k - 1) / n == 0) return RTS_OK;
    if (!gathered || !recv || !sat_word || !out_ids) return RTS_EINVAL;
    if (!aligned(gathered, 4) || !aligned(recv, 4) || !aligned(sat_word, 4) || !aligned(out_ids, 4))
        return RTS_EINVAL;
    return rts::launch_merge_rescue(gathered, recv, world, rows, n, k, sat_word, out_ids, nullptr, stream);
}

int emit_rows(const int32_t* ids, int64_t rows, int32_t k, int32_t world, int32_t dcp_rank,
              const int32_t* req_id, const int32_t* block_table, int64_t table_rows, int32_t table_cols,
              int64_t ld_table, int32_t block_size, int64_t stride_rows, int32_t* rows_out,
              int32_t out_cols, int32_t* valid_out, hipStream_t stream) {
    if (rows < 0 || k < 1 || world < 1 || dcp_rank < 0 || dcp_rank >= world || table_rows < 0 ||
        table_cols < 0 || ld_table < table_cols || block_size < 1 || out_cols < k)
        return RTS_EINVAL;
    if (k > kMaxK || (rows + 3) / 4 > kMaxGrid) return RTS_EUNSUPPORTED;
    if (rows == 0) return RTS_OK;
    if (!ids || !req_id || !rows_out || !valid_out || (table_rows > 0 && table_cols > 0 && !block_table))
        return RTS_EINVAL;
    if (!aligned(ids, 4) || !aligned(req_id, 4) || !aligned(rows_out, 4) || !aligned(valid_out, 4) ||
        (block_table && !aligned(block_table, 4)))
        return RTS_EINVAL;
    return rts::launch_emit_rows(ids, rows, k, world, dcp_rank, req_id, block_table, table_rows,
                                 table_cols, ld_table, block_size, stride_rows, rows_out, out_cols,
                                 valid_out, stream);
}

namespace {
// Validates an rts_kv_rows against k and world and converts it.
int kv_rows_args(const rts_kv_rows* kv, int32_t k, int32_t world, rts::RowsArgs& ra) {
    if (!kv || kv->dcp_rank < 0 || kv->dcp_rank >= world || kv->table_rows < 0 || kv->table_cols < 0 ||
        kv->ld_table < kv->table_cols || kv->block_size < 1 || kv->out_cols < k)
        return RTS_EINVAL;
    if (!kv->req_id || !kv->rows_out || !kv->valid_out ||
        (kv->table_rows > 0 && kv->table_cols > 0 && !kv->block_table))
        return RTS_EINVAL;
    if (!aligned(kv->req_id, 4) || !aligned(kv->rows_out, 4) || !aligned(kv->valid_out, 4) ||
        (kv->block_table && !aligned(kv->block_table, 4)))
        return RTS_EINVAL;
    ra = rts::RowsArgs{kv->req_id, kv->block_table, kv->rows_out, kv->valid_out, kv->table_rows,
                       kv->ld_table, kv->stride_rows, kv->dcp_rank, kv->table_cols, kv->block_size,
                       kv->out_cols};
    return RTS_OK;
}
}  // namespace

int merge_select_rank_major_rows(const int32_t* gathered, int32_t world, int64_t rows, int32_t n,
                                 int32_t k, const rts_kv_rows* kv, int32_t* out_ids, int32_t* sat_word,
                                 hipStream_t stream) {
    if (world < 1 || world > 16 || rows < 0 || n < 32 || n % 32 != 0 || k < 1) return RTS_EINVAL;
    if (k > kMaxK || (int64_t)world * n > kMaxCandidates || rows > kMaxGrid) return RTS_EUNSUPPORTED;
    rts::RowsArgs ra;
    const int rc = kv_rows_args(kv, k, world, ra);
    if (rc != RTS_OK) return rc;
    if (rows == 0) return RTS_OK;
    if (!gathered || !aligned(gathered, 4) || (out_ids && !aligned(out_ids, 4)) ||
        (sat_word && !aligned(sat_word, 4)))
        return RTS_EINVAL;
    return rts::launch_merge_packed(gathered, false, world, rows, n, k, out_ids, sat_word, &ra, stream);
}

int merge_rescue_rank_major_rows(const int32_t* gathered, const int32_t* recv, int32_t world,
                                 int64_t rows, int32_t n, int32_t k, const int32_t* sat_word,
                                 const rts_kv_rows* kv, int32_t* out_ids, hipStream_t stream) {
    if (world < 1 || world > 16 || rows < 0 || n < 32 || n % 32 != 0 || k < 32 || k % 32 != 0)
        return RTS_EINVAL;
    if (k > kMaxK || rts::rescue_candidates(world, n, k) > kMaxCandidates || rows > kMaxGrid)
        return RTS_EUNSUPPORTED;
    rts::RowsArgs ra;
    const int rc = kv_rows_args(kv, k, world, ra);
    if (rc != RTS_OK) return rc;
    if (rows == 0 || (k - 1) / n == 0) return RTS_OK;
    if (!gathered || !recv || !sat_word) return RTS_EINVAL;
    if (!aligned(gathered, 4) || !aligned(recv, 4) || !aligned(sat_word, 4) ||
        (out_ids && !aligned(out_ids, 4)))
        return RTS_EINVAL;
    return rts::launch_merge_rescue(gathered, recv, world, rows, n, k, sat_word, out_ids, &ra, stream);
}

int pack_pairs(const float* logits, int64_t rows, int64_t cols, int64_t ld_logits,
               const int32_t* local_idx, int32_t kc, int64_t ld_idx, const int32_t* row_ends,
               int32_t rank, int32_t world, int32_t* pairs, hipStream_t stream) {
    if (rows < 0 || cols < 0 || ld_logits < cols || kc < 1 || ld_idx < kc || world < 1 ||
        rank < 0 || rank >= world)
        return RTS_EINVAL;
    if (cols * (int64_t)world > 0x7FFFFFFFll) return RTS_EUNSUPPORTED;
    if (rows == 0) return RTS_OK;
    if (!logits || !local_idx || !pairs) return RTS_EINVAL;
    if (!aligned(logits, 4) || !aligned(local_idx, 4) || !aligned(pairs, 8) ||
        (row_ends && !aligned(row_ends, 4)))
        return RTS_EINVAL;
    if ((rows * (int64_t)kc + 255) / 256 > kMaxGrid) return RTS_EUNSUPPORTED;
    return rts::launch_pack_pairs(logits, rows, cols, ld_logits, local_idx, kc, ld_idx, row_ends,
                                  rank, world, pairs, stream);
}

int merge_select_pairs_rank_major(const int32_t* gathered_pairs, int32_t world, int64_t rows,
                                  int32_t kc, int32_t k, int32_t* out_ids, hipStream_t stream) {
    return merge_pairs_checked(gathered_pairs, false, world, rows, kc, k, out_ids, stream);
}

int merge_select_pairs_row_major(const int32_t* gathered_pairs, int32_t world, int64_t rows,
                                 int32_t kc, int32_t k, int32_t* out_ids, hipStream_t stream) {
    return merge_pairs_checked(gathered_pairs, true, world, rows, kc, k, out_ids, stream);
}

}  // extern "C"
