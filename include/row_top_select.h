/*
 * row_top_select -- batched per-row exact top-K selection over indexer logits,
 * and the one-round candidate merge of a token-sharded (DCP) indexer, for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources: the three pages this library follows.
 *   [P1] vLLM pull request 65178 (rank-major DCP top-k merge): "Overview" and
 *        "Details" -- (score, global id) candidates all-gathered along dim 0
 *        into [W, R, K, 2] and selected in place.
 *   [P2] vLLM API page vllm.models.kimi_k3.nvidia.ops.dcp_topk_merge.kernels:
 *        module docstring (B' word and bit plane, exactness, saturation word),
 *        DCPTopkPackKernel, DCPTopkSelectKernel, DCPTopkRescueKernel,
 *        DCPTopkRescueWorkspace, _decode_key, _ord16, dcp_topk_pack_indices,
 *        dcp_topk_select, dcp_topk_merge_rows, _check_exact.
 *   [P3] vLLM pull request 57206, "Use DeepSelect for eligible sparse-indexer
 *        prefill chunks": "Purpose" (causal per-row end, KV from column 0,
 *        preallocated output) and "Test Plan" (short rows, -1 tails, strided
 *        output, untouched padding, graph replay after updating row ends).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains memory and keeps no state,
 *     except the static device scratch of topk_rows_noalloc (one array per
 *     GPU, its address cached on the first call there).
 *   - Every call only validates its arguments on the host and enqueues work on
 *     `stream` (0 = the null stream); it never synchronises, so calls are
 *     stream-ordered and may be captured into a HIP graph.  Data the kernels
 *     read (row_ends included) is read on the device at execution time.
 *   - Errors are reported by the return value (rts_status) before anything is
 *     launched; a failed launch returns RTS_EHIP.  Data-dependent oddities
 *     (NaN, out-of-range local ids, duplicate candidates) are defined
 *     behaviour and never cause an out-of-bounds access.
 *   - Scores order as IEEE values, descending, with -0.0 below +0.0 (the
 *     order of the order-preserving key of [P2] _ord16); NaN is never a
 *     candidate; +inf and -inf are ordinary candidates.  Equal scores are
 *     resolved toward the lower id.
 */
#ifndef ROW_TOP_SELECT_H
#define ROW_TOP_SELECT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RTS_OK = 0,
    RTS_EINVAL = -1,       /* a null pointer, a negative size, a stride below its row, ... */
    RTS_EUNSUPPORTED = -2, /* valid request outside what this build implements (e.g. k > 2048) */
    RTS_EWORKSPACE = -3,   /* a workspace was given but is smaller than required */
    RTS_EHIP = -4          /* the HIP runtime rejected the launch */
} rts_status;

typedef enum {
    RTS_F32 = 0,  /* IEEE binary32 */
    RTS_BF16 = 1  /* bfloat16 bit patterns (uint16_t) */
} rts_dtype;

/* Human-readable name of an rts_status value (static storage). */
const char* rts_status_string(int status);

/*
 * Bytes of device workspace that lets topk_rows split long rows of a small
 * batch over several workgroups (0 when no split is used for this shape).
 * Passing less than this (but not 0) to topk_rows is RTS_EWORKSPACE; passing
 * no workspace at all is allowed and runs every row in one workgroup.
 */
size_t topk_rows_workspace_size(int dtype, int64_t rows, int64_t cols, int32_t k);

/*
 * topk_rows -- exact top-k of every row ([P3] Purpose and Test Plan; selection
 * rule of [P2] module docstring and DCPTopkSelectKernel docstring).
 *
 * logits    [rows, ld_logits] row-major, dtype RTS_F32 (float) or RTS_BF16
 *           (uint16_t bits); only columns [0, cols) are ever read, and of row i
 *           only columns [0, e_i).  Must be aligned to its element size.
 * row_ends  int32 [rows] or NULL.  e_i = clamp(row_ends[i], 0, cols): the
 *           exclusive causal end of row i, the row starting at column 0.
 *           NULL means e_i = cols for every row.
 * k         1 <= k <= 2048.
 * out_idx   int32 [rows, ld_out], ld_out >= k.  Row i receives the column ids
 *           of its m_i = min(k, #non-NaN in [0, e_i)) best entries in
 *           (score desc, id asc) order, then -1 in columns [m_i, k).  Columns
 *           [k, ld_out) are never written.
 * workspace optional device scratch (see topk_rows_workspace_size), may be
 *           NULL with workspace_bytes == 0.
 * Errors: RTS_EINVAL (bad sizes/strides/pointers/dtype/alignment),
 *         RTS_EUNSUPPORTED (k > 2048, cols >= 2^31), RTS_EWORKSPACE, RTS_EHIP.
 */
/* `dtype` is a plain int holding an rts_dtype value (RTS_F32 or RTS_BF16), so
 * the symbol keeps one fixed C signature for foreign-function callers; any
 * other value is RTS_EINVAL. */
int topk_rows(const void* logits, int dtype, int64_t rows, int64_t cols, int64_t ld_logits,
              const int32_t* row_ends, int32_t k, int32_t* out_idx, int64_t ld_out,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * topk_rows_noalloc -- topk_rows for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments (minus the workspace), outputs and
 * errors as topk_rows, and the same result.
 *
 * Where topk_rows would split long rows of a small batch over several
 * workgroups with a caller workspace, this call keeps the partial lists in a
 * static device array of the library instead: 16 MiB (every launch plan of
 * this library fits in it), one per GPU, held from the first call on that
 * GPU until the process ends.  The array's address on the current device is
 * taken on the first call there (make that first call outside graph
 * capture); no call allocates or frees memory.  Nothing in the array needs
 * clearing between calls: each launch writes every list it reads.  Calls on
 * one GPU share its array, so two calls whose executions overlap on that GPU
 * (different streams without ordering between them) race; calls ordered on
 * one stream do not.  A plan that needed more than the array holds would be
 * refused with RTS_EWORKSPACE.  `stream` must belong to the current device.
 */
int topk_rows_noalloc(const void* logits, int dtype, int64_t rows, int64_t cols, int64_t ld_logits,
                      const int32_t* row_ends, int32_t k, int32_t* out_idx, int64_t ld_out,
                      hipStream_t stream);

/*
 * pack_candidates -- a rank's local top-n as B' words ([P2] module docstring
 * step 1, DCPTopkPackKernel, dcp_topk_pack_indices).
 *
 * logits_bf16 [rows, ld_logits] bf16 bits; cols columns.
 * local_idx   int32 [rows, ld_idx], ld_idx >= n: local column ids, -1 padded,
 *             any order.
 * n           number of slots, a positive multiple of 32.
 * row_ends    int32 [rows] or NULL (= cols).
 * packed      int32 [rows, n + n/32], contiguous.  For slot j with
 *             l = local_idx[t, j] and end = min(row_end_t, cols, 2^17):
 *               0 <= l < end and score not NaN:
 *                 packed[t, j] = (ord16(score) << 16) | (0xFFFF - (l & 0xFFFF)),
 *                 bit j%32 of packed[t, n + j/32] = bit 16 of l;
 *               otherwise packed[t, j] = 0 (empty) and the plane bit is 0.
 *             ord16(b) = b & 0x8000 ? ~b & 0xFFFF : b | 0x8000.
 * Errors: RTS_EINVAL, RTS_EHIP.
 */
int pack_candidates(const uint16_t* logits_bf16, int64_t rows, int64_t cols, int64_t ld_logits,
                    const int32_t* local_idx, int32_t n, int64_t ld_idx, const int32_t* row_ends,
                    int32_t* packed, hipStream_t stream);

/*
 * merge_select_rank_major -- round-1 select of the packed merge ([P2] module
 * docstring steps 2-3 and saturation, DCPTopkSelectKernel, _decode_key; the
 * gathered buffer is read in place, rank-major, as in [P1]).
 *
 * gathered  int32 [world, rows, n + n/32], contiguous: rank r's packed rows.
 *           A nonzero word w at (r, t, j) is the candidate
 *             local = (0xFFFF - (w & 0xFFFF)) | (bit j%32 of gathered[r, t, n + j/32]) << 16,
 *             gid = local * world + r, score key ord16 = w >> 16.
 * world     1..16 ranks; n a positive multiple of 32; world * n <= 32768.
 * k         1 <= k <= 2048.
 * out_ids   int32 [rows, k], contiguous: the gids of the first min(k, count)
 *           candidates under (ord16 desc, gid asc), listed in candidate order
 *           (rank, then slot), then -1.
 * sat_word  int32 [rows] or NULL: (mask << 16) | tau16, tau16 = ord16 of the
 *           k-th selected (0 when fewer than k candidates), mask bit r set iff
 *           all n words of rank r are nonzero with ord16 > tau16; a mask with
 *           more than (k - 1) / n bits is cleared.  mask == 0 means round 1 is
 *           exact.
 * Candidates are expected to have distinct gids; with repeated words the
 * output stays in bounds and deterministic but is not specified further.
 * Limits are wider than the kernels page's (which takes k in {512, 1024,
 * 2048} and n < k without its second-round state): any k in [1, 2048] and
 * any n, since sat_word tells the caller whether round 1 was exact.
 * Errors: RTS_EINVAL, RTS_EUNSUPPORTED, RTS_EHIP.
 */
int merge_select_rank_major(const int32_t* gathered, int32_t world, int64_t rows, int32_t n,
                            int32_t k, int32_t* out_ids, int32_t* sat_word, hipStream_t stream);

/*
 * merge_select_row_major -- merge_select_rank_major on the row-major layout
 * gathered int32 [rows, world, n + n/32] (rank r's words of row t at
 * gathered[t, r]), the layout an all-gather along dim 1 (or a reorder copy of
 * the dim-0 result) produces ([P1] Overview, "Before").  Same arguments,
 * limits, candidate order, outputs and errors; for the same words the outputs
 * are identical to merge_select_rank_major's.
 */
int merge_select_row_major(const int32_t* gathered, int32_t world, int64_t rows, int32_t n, int32_t k,
                           int32_t* out_ids, int32_t* sat_word, hipStream_t stream);

/*
 * Second round of the packed merge, with the world ranks on one device
 * ([P2] module docstring on exactness, DCPTopkRescueKernel,
 * DCPTopkRescueWorkspace).  A row enters it iff its sat_word mask is nonzero,
 * names only ranks below world and has at most S = (k - 1) / n bits (round 1
 * writes no other nonzero mask); every other row is neither read past its
 * sat_word nor written.  When S == 0 (n >= k) no row can enter and both calls
 * return RTS_OK without launching.  The receive buffer
 *   recv  int32 [rows, S, k + k/32], contiguous
 * holds, in slot s of row t, the packed local top-k of the s-th saturated
 * rank (ascending rank order), in the word and plane format of
 * pack_candidates with n = k.
 *
 * rescue_push -- rank `rank`'s push: for every row whose mask enters the
 * second round and has bit `rank`, copy local_packed[t] (int32 [rows,
 * k + k/32], contiguous: that rank's pack_candidates of its local top-k) into
 * recv[t, popc(mask & ((1 << rank) - 1))].  Other slots are not written.
 * 0 <= rank < world <= 16; n, k positive multiples of 32, k <= 2048.
 * Errors: RTS_EINVAL, RTS_EUNSUPPORTED, RTS_EHIP.
 */
int rescue_push(const int32_t* local_packed, int32_t rank, int32_t world, int64_t rows, int32_t n,
                int32_t k, const int32_t* sat_word, int32_t* recv, hipStream_t stream);

/*
 * merge_rescue_rank_major -- the rescue select.  For every row that enters
 * the second round the candidates are, at flat position r * n + j, the
 * round-1 words gathered[r, t, j] (layout of merge_select_rank_major) of the
 * ranks whose bit is clear and whose ord16 >= tau16 (sat_word & 0xFFFF), then
 * at world * n + s * k + j the words of recv[t, s] for s < popc(mask), owned
 * by the s-th set bit.  out_ids[t] (int32 [rows, k], contiguous) is
 * overwritten with the gids of the first min(k, count) under (ord16 desc,
 * gid asc), in flat position order, then -1.  With the pushes of a valid
 * round 1 the selected scores equal the top-k of the union as a multiset.
 * world <= 16; n, k positive multiples of 32, k <= 2048;
 * world * n + min(S, world) * k <= 32768.
 * Errors: RTS_EINVAL, RTS_EUNSUPPORTED, RTS_EHIP.
 */
int merge_rescue_rank_major(const int32_t* gathered, const int32_t* recv, int32_t world, int64_t rows,
                            int32_t n, int32_t k, const int32_t* sat_word, int32_t* out_ids,
                            hipStream_t stream);

/*
 * emit_rows -- this rank's owned physical KV rows of the selected ids ([P2]
 * DCPTopkSelectKernel docstring on emit_rows, dcp_topk_merge_rows: rows_out,
 * valid_out), the format sparse attention reads.
 *
 * ids         int32 [rows, k], contiguous: global ids as the selects write
 *             them (negative = empty slot).
 * world, dcp_rank  0 <= dcp_rank < world: a gid is owned iff
 *             gid % world == dcp_rank; its local index is gid / world.
 * req_id      int32 [rows]: the request (block-table row) of each row.
 * block_table int32 [table_rows, ld_table], first table_cols columns used:
 *             KV block ids of each request.
 * block_size  tokens per KV block (>= 1); stride_rows physical rows per block.
 * rows_out    int32 [rows, out_cols], contiguous, out_cols >= k: for each
 *             owned id, in the order ids lists them, the physical row
 *               block_table[req, b] * stride_rows + local % block_size,
 *             b = local / block_size (computed in 64 bits, stored as its low
 *             32 bits); then -1.  An id whose block b >= table_cols is
 *             dropped; a row whose req_id is outside [0, table_rows) owns
 *             nothing.
 * valid_out   int32 [rows]: the number of rows written for each row.
 * k <= 2048.  Errors: RTS_EINVAL, RTS_EUNSUPPORTED, RTS_EHIP.
 */
int emit_rows(const int32_t* ids, int64_t rows, int32_t k, int32_t world, int32_t dcp_rank,
              const int32_t* req_id, const int32_t* block_table, int64_t table_rows, int32_t table_cols,
              int64_t ld_table, int32_t block_size, int64_t stride_rows, int32_t* rows_out,
              int32_t out_cols, int32_t* valid_out, hipStream_t stream);

/*
 * rts_kv_rows -- where the fused selects below write this rank's owned
 * physical KV rows; the fields mean what the arguments of emit_rows of the
 * same names mean (all pointers device pointers, owned by the caller).
 */
typedef struct {
    int32_t dcp_rank;           /* 0 <= dcp_rank < world */
    const int32_t* req_id;      /* [rows] */
    const int32_t* block_table; /* [table_rows, ld_table], first table_cols columns used */
    int64_t table_rows;
    int32_t table_cols;
    int64_t ld_table;           /* >= table_cols */
    int32_t block_size;         /* >= 1 */
    int64_t stride_rows;
    int32_t* rows_out;          /* [rows, out_cols], contiguous, out_cols >= k */
    int32_t out_cols;
    int32_t* valid_out;         /* [rows] */
} rts_kv_rows;

/*
 * merge_select_rank_major_rows -- merge_select_rank_major that writes this
 * rank's owned physical rows straight from the select ([P2]
 * DCPTopkSelectKernel docstring: emit_ids and/or emit_rows;
 * dcp_topk_merge_rows).  For the same words, kv->rows_out and kv->valid_out
 * are exactly what emit_rows writes for the ids merge_select_rank_major
 * returns, and out_ids (optional, NULL = not written) and sat_word (NULL =
 * not written) are what merge_select_rank_major writes.
 * Errors: those of merge_select_rank_major; RTS_EINVAL for an invalid kv.
 */
int merge_select_rank_major_rows(const int32_t* gathered, int32_t world, int64_t rows, int32_t n,
                                 int32_t k, const rts_kv_rows* kv, int32_t* out_ids, int32_t* sat_word,
                                 hipStream_t stream);

/*
 * merge_rescue_rank_major_rows -- merge_rescue_rank_major that also (or
 * only: out_ids may be NULL) rewrites kv->rows_out and kv->valid_out of the
 * rows that enter the second round, as emit_rows would for their new ids.
 * Rows that do not enter are not written.
 * Errors: those of merge_rescue_rank_major; RTS_EINVAL for an invalid kv.
 */
int merge_rescue_rank_major_rows(const int32_t* gathered, const int32_t* recv, int32_t world,
                                 int64_t rows, int32_t n, int32_t k, const int32_t* sat_word,
                                 const rts_kv_rows* kv, int32_t* out_ids, hipStream_t stream);

/*
 * pack_pairs -- a rank's local top-kc as (score, global id) pairs ([P1]
 * Overview: "pack(local_topk)" into [R, K, 2]).
 *
 * logits    float [rows, ld_logits]; cols columns.
 * local_idx int32 [rows, ld_idx], ld_idx >= kc: local column ids, -1 padded.
 * row_ends  int32 [rows] or NULL (= cols).
 * rank, world  0 <= rank < world; cols * world < 2^31.
 * pairs     int32 [rows, kc, 2], contiguous: for l = local_idx[t, j] with
 *           0 <= l < clamp(row_end_t, 0, cols) and x[t, l] not NaN:
 *           (bits of x[t, l], l * world + rank); otherwise (0, -1).
 * Errors: RTS_EINVAL, RTS_EHIP.
 */
int pack_pairs(const float* logits, int64_t rows, int64_t cols, int64_t ld_logits,
               const int32_t* local_idx, int32_t kc, int64_t ld_idx, const int32_t* row_ends,
               int32_t rank, int32_t world, int32_t* pairs, hipStream_t stream);

/*
 * merge_select_pairs_rank_major -- select from (score, global id) pairs read
 * in place from the rank-major all-gather buffer ([P1] Overview and Details).
 *
 * gathered_pairs int32 [world, rows, kc, 2], contiguous: [..., 0] fp32 score
 *           bits, [..., 1] global id; a negative id is an empty slot, a NaN
 *           score is dropped.
 * world >= 1, kc >= 1, world * kc <= 32768.  k: 1 <= k <= 2048.
 * out_ids   int32 [rows, k], contiguous: the ids of the first min(k, count)
 *           candidates under (score desc, -0 below +0, id asc), listed in
 *           candidate order (rank, then slot), then -1.
 * Ids are expected to be distinct within a row (as all-gathered local top-k
 * lists are); repeated ids stay in bounds but are not specified further.
 * Errors: RTS_EINVAL, RTS_EUNSUPPORTED, RTS_EHIP.
 */
int merge_select_pairs_rank_major(const int32_t* gathered_pairs, int32_t world, int64_t rows,
                                  int32_t kc, int32_t k, int32_t* out_ids, hipStream_t stream);

/*
 * merge_select_pairs_row_major -- merge_select_pairs_rank_major on the
 * row-major layout gathered_pairs int32 [rows, world * kc, 2] (candidate
 * r * kc + j of row t is rank r's slot j), the [R, W*K, 2] buffer of [P1]
 * Overview, "Before".  Same arguments, limits, order and errors; for the same
 * pairs the ids are identical to merge_select_pairs_rank_major's.
 */
int merge_select_pairs_row_major(const int32_t* gathered_pairs, int32_t world, int64_t rows,
                                 int32_t kc, int32_t k, int32_t* out_ids, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROW_TOP_SELECT_H */
