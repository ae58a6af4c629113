/*
 * Reference oracle for the row top-K select and the candidate merge.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow CPU definition that
 * the GPU library is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the library never calls it and it
 * shares no code, header or table with the library.
 *
 * Every selection here is "collect the valid candidates, sort them with the C
 * library's qsort under the stated order, take the first K".  Scores are
 * compared as IEEE values (bf16 widened exactly to float); the only departure
 * from IEEE equality is that -0.0 ranks below +0.0, which is what the
 * order-preserving bf16 key of the kernels page does (section "_ord16": the key
 * of -0 is 0x7FFF, the key of +0 is 0x8000).
 *
 * Sources (the three pages of the reference):
 *   [P1] vLLM pull request 65178, rank-major DCP top-k merge: "Overview" and
 *        "Details" (the [W, R, K, 2] (score, global id) buffer read in place).
 *   [P2] vLLM API page vllm.models.kimi_k3.nvidia.ops.dcp_topk_merge.kernels:
 *        module docstring (B' word, bit plane, saturation word),
 *        DCPTopkPackKernel, DCPTopkSelectKernel, DCPTopkRescueKernel,
 *        DCPTopkRescueWorkspace, _decode_key, _ord16,
 *        assert_packed_merge_contract, dcp_topk_pack_indices,
 *        dcp_topk_merge_rows.
 *   [P3] vLLM pull request 57206, "Use DeepSelect for eligible sparse-indexer
 *        prefill chunks": "Purpose" (causal end bound, KV starts at column 0)
 *        and "Test Plan" (short rows, -1 tails, untouched padding).
 *
 * Parity pins for each function live in tests/ (brute force, closed forms,
 * invariants); none of them re-call this file to produce an expected value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Scores                                                              */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> float (exact: bf16 is the top half of an fp32). */
static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float bits_to_float(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* One candidate: score, the id it is reported under, and its position in
 * the input (used only to break exact duplicates deterministically). */
typedef struct {
    float v;
    int64_t id;
    int64_t pos;
} cand_t;

/* Order of [P2] DCPTopkSelectKernel docstring / [P3] Purpose:
 * score descending, -0 below +0, then id ascending. */
static int cand_cmp(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    int sa = signbit(a->v) ? 1 : 0;
    int sb = signbit(b->v) ? 1 : 0;
    if (sa != sb) return sa ? 1 : -1; /* the negative zero goes after */
    if (a->id < b->id) return -1;
    if (a->id > b->id) return 1;
    if (a->pos < b->pos) return -1;
    if (a->pos > b->pos) return 1;
    return 0;
}

static int64_t clamp_end(const int32_t* row_ends, int64_t row, int64_t cols) {
    int64_t e = row_ends ? (int64_t)row_ends[row] : cols;
    if (e < 0) e = 0;
    if (e > cols) e = cols;
    return e;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* O1: per-row exact top-K ([P3] Purpose + Test Plan, [P2] module doc) */
/* ------------------------------------------------------------------ */
/*
 * For row i, e = clamp(row_ends[i], 0, cols) (cols when row_ends is NULL).
 * Candidates are (x[i, j], j) for j < e with x not NaN; +-inf are ordinary.
 * out[i, 0:m] = ids of the first m = min(k, #candidates) in the order above,
 * out[i, m:k] = -1, out[i, k:ld_out] untouched.
 * dtype 0 = fp32, 1 = bf16 (bit patterns as uint16).
 */
int oracle_topk_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                     int64_t ld, const int32_t* row_ends, int32_t k,
                     int32_t* out, int64_t ld_out, int nthreads) {
    if (rows < 0 || cols < 0 || ld < cols || k < 1 || ld_out < k) return -1;
    if (dtype != 0 && dtype != 1) return -1;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)(cols > 0 ? cols : 1));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < rows; ++i) {
            if (!buf) continue;
            int64_t e = clamp_end(row_ends, i, cols);
            int64_t n = 0;
            for (int64_t j = 0; j < e; ++j) {
                float v = dtype == 0 ? ((const float*)x)[i * ld + j]
                                     : bf16_to_float(((const uint16_t*)x)[i * ld + j]);
                if (isnan(v)) continue;
                buf[n].v = v;
                buf[n].id = j;
                buf[n].pos = j;
                ++n;
            }
            qsort(buf, (size_t)n, sizeof(cand_t), cand_cmp);
            int32_t* o = out + i * ld_out;
            for (int64_t t = 0; t < k; ++t) o[t] = t < n ? (int32_t)buf[t].id : -1;
        }
        free(buf);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------ */
/* O2: pack a local top-N into B' words ([P2] module doc step 1,      */
/*     DCPTopkPackKernel, dcp_topk_pack_indices)                       */
/* ------------------------------------------------------------------ */

/* [P2] _ord16: flip a negative bf16, set the sign bit of a non-negative. */
static uint32_t ord16_of(uint16_t b) {
    return (b & 0x8000u) ? (uint32_t)(~b & 0xFFFFu) : (uint32_t)(b | 0x8000u);
}

/*
 * packed[t] is n words then n/32 bit-plane words.  Slot j holds local id
 * l = local_idx[t, j]; with end = min(row_end or cols, cols, 2^17):
 *   0 <= l < end and bf16 x[t, l] not NaN  ->  word = (ord16 << 16) | (0xFFFF - (l & 0xFFFF)),
 *                                              plane bit j%32 of word n + j/32 = (l >> 16) & 1
 *   otherwise                              ->  word = 0, plane bit 0.
 */
int oracle_pack_candidates(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                           const int32_t* local_idx, int32_t n, int64_t ld_idx,
                           const int32_t* row_ends, int32_t* packed) {
    if (rows < 0 || cols < 0 || ld < cols || n < 32 || n % 32 != 0 || ld_idx < n) return -1;
    int64_t width = (int64_t)n + n / 32;
    for (int64_t t = 0; t < rows; ++t) {
        int64_t end = cols;
        if (end > (1 << 17)) end = 1 << 17;
        if (row_ends && row_ends[t] < end) end = row_ends[t];
        int32_t* p = packed + t * width;
        for (int32_t q = 0; q < n / 32; ++q) p[n + q] = 0;
        for (int32_t j = 0; j < n; ++j) {
            int64_t l = local_idx[t * ld_idx + j];
            uint32_t word = 0;
            if (l >= 0 && l < end) {
                uint16_t b = x[t * ld + l];
                if ((b & 0x7FFFu) <= 0x7F80u) {
                    word = (ord16_of(b) << 16) | (0xFFFFu - ((uint32_t)l & 0xFFFFu));
                    if (((uint32_t)l >> 16) & 1u)
                        p[n + j / 32] = (int32_t)((uint32_t)p[n + j / 32] | (1u << (j % 32)));
                }
            }
            p[j] = (int32_t)word;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O3: select from the rank-major gathered B' buffer ([P2] module doc */
/*     steps 2-3 + saturation, DCPTopkSelectKernel, _decode_key)      */
/* ------------------------------------------------------------------ */

typedef struct {
    uint32_t o;   /* ord16 */
    int64_t gid;  /* global id */
    int64_t pos;  /* flat candidate position r * n + j */
} mcand_t;

static int mcand_cmp(const void* pa, const void* pb) {
    const mcand_t* a = (const mcand_t*)pa;
    const mcand_t* b = (const mcand_t*)pb;
    if (a->o > b->o) return -1;
    if (a->o < b->o) return 1;
    if (a->gid < b->gid) return -1;
    if (a->gid > b->gid) return 1;
    if (a->pos < b->pos) return -1;
    if (a->pos > b->pos) return 1;
    return 0;
}

static int popcount32(uint32_t v) {
    int c = 0;
    while (v) {
        c += (int)(v & 1u);
        v >>= 1;
    }
    return c;
}

/*
 * gathered is int32 [world, rows, n + n/32] (row-contiguous, rank-major).
 * For each row: every nonzero word w at (r, j) decodes to
 *   o = w >> 16, local = (0xFFFF - (w & 0xFFFF)) | (plane bit j of rank r) << 16,
 *   gid = local * world + r.
 * The K selected are the first min(K, count) under (o desc, gid asc).
 * out_ids[row] lists their gids in candidate order (r, then j ascending),
 * then -1 up to k.
 * sat_word[row] = (mask << 16) | tau16, tau16 = o of the K-th selected (0 when
 * fewer than K), mask bit r set iff all n words of rank r are nonzero with
 * o > tau16; a mask with more than (k - 1) / n bits is cleared.
 * sat_word may be NULL.
 */
int oracle_merge_select_rank_major(const int32_t* gathered, int32_t world, int64_t rows,
                                   int32_t n, int32_t k, int32_t* out_ids, int32_t* sat_word) {
    if (world < 1 || world > 16 || rows < 0 || n < 32 || n % 32 != 0 || k < 1) return -1;
    int64_t width = (int64_t)n + n / 32;
    int64_t total = (int64_t)world * n;
    mcand_t* buf = (mcand_t*)malloc(sizeof(mcand_t) * (size_t)total);
    unsigned char* sel = (unsigned char*)malloc((size_t)total);
    if (!buf || !sel) {
        free(buf);
        free(sel);
        return -2;
    }
    for (int64_t t = 0; t < rows; ++t) {
        int64_t cnt = 0;
        for (int32_t r = 0; r < world; ++r) {
            const int32_t* p = gathered + ((int64_t)r * rows + t) * width;
            for (int32_t j = 0; j < n; ++j) {
                uint32_t w = (uint32_t)p[j];
                if (w == 0) continue;
                uint32_t plane = (uint32_t)p[n + j / 32];
                int64_t local = (int64_t)(0xFFFFu - (w & 0xFFFFu)) |
                                ((int64_t)((plane >> (j % 32)) & 1u) << 16);
                buf[cnt].o = w >> 16;
                buf[cnt].gid = local * world + r;
                buf[cnt].pos = (int64_t)r * n + j;
                ++cnt;
            }
        }
        qsort(buf, (size_t)cnt, sizeof(mcand_t), mcand_cmp);
        int64_t m = cnt < k ? cnt : k;
        memset(sel, 0, (size_t)total);
        for (int64_t q = 0; q < m; ++q) sel[buf[q].pos] = 1;
        uint32_t tau16 = cnt >= k ? buf[k - 1].o : 0u;

        int32_t* o = out_ids + t * k;
        int64_t w_at = 0;
        for (int32_t r = 0; r < world; ++r) {
            const int32_t* p = gathered + ((int64_t)r * rows + t) * width;
            for (int32_t j = 0; j < n; ++j) {
                if (!sel[(int64_t)r * n + j]) continue;
                uint32_t w = (uint32_t)p[j];
                uint32_t plane = (uint32_t)p[n + j / 32];
                int64_t local = (int64_t)(0xFFFFu - (w & 0xFFFFu)) |
                                ((int64_t)((plane >> (j % 32)) & 1u) << 16);
                o[w_at++] = (int32_t)(local * world + r);
            }
        }
        for (int64_t q = w_at; q < k; ++q) o[q] = -1;

        if (sat_word) {
            uint32_t mask = 0;
            for (int32_t r = 0; r < world; ++r) {
                const int32_t* p = gathered + ((int64_t)r * rows + t) * width;
                int full = 1;
                for (int32_t j = 0; j < n; ++j) {
                    uint32_t w = (uint32_t)p[j];
                    if (w == 0 || (w >> 16) <= tau16) {
                        full = 0;
                        break;
                    }
                }
                if (full) mask |= 1u << r;
            }
            if (popcount32(mask) > (k - 1) / n) mask = 0;
            sat_word[t] = (int32_t)((mask << 16) | tau16);
        }
    }
    free(buf);
    free(sel);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O3b: second round of the exact packed merge, all W ranks on one     */
/*      device ([P2] module docstring on exactness, DCPTopkRescueKernel, */
/*      DCPTopkRescueWorkspace, the select's exact flag)                */
/* ------------------------------------------------------------------ */

/* A row enters the second round iff its mask is nonzero, names only ranks
 * below world, and has at most S = (k-1)/n bits (the receive slots per row).
 * Round 1 never writes any other nonzero mask; such a row is left alone. */
static int mcand_pos_cmp(const void* pa, const void* pb) {
    const mcand_t* a = (const mcand_t*)pa;
    const mcand_t* b = (const mcand_t*)pb;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

static int rescue_row_mask(uint32_t sw, int32_t world, int32_t n, int32_t k) {
    uint32_t mask = sw >> 16;
    if (mask == 0 || (world < 32 && (mask >> world) != 0)) return 0;
    if (popcount32(mask) > (k - 1) / n) return 0;
    return 1;
}

/* A saturated rank's push: its local top-k of the row, packed into k words
 * and k/32 plane words, lands in receive slot popc(mask & ((1 << rank) - 1))
 * of recv [rows, S, k + k/32].  local_packed [rows, k + k/32] is that rank's
 * pack of its local top-k for every row; only rows whose mask has the rank's
 * bit are copied. */
int oracle_rescue_push(const int32_t* local_packed, int32_t rank, int32_t world, int64_t rows,
                       int32_t n, int32_t k, const int32_t* sat_word, int32_t* recv) {
    if (world < 1 || world > 16 || rank < 0 || rank >= world || rows < 0 || n < 32 ||
        n % 32 != 0 || k < 32 || k % 32 != 0)
        return -1;
    const int64_t pw = (int64_t)k + k / 32, slots = (k - 1) / n;
    for (int64_t t = 0; t < rows; ++t) {
        const uint32_t sw = (uint32_t)sat_word[t];
        if (!rescue_row_mask(sw, world, n, k) || !(((sw >> 16) >> rank) & 1u)) continue;
        const int64_t slot = popcount32((sw >> 16) & ((1u << rank) - 1u));
        memcpy(recv + (t * slots + slot) * pw, local_packed + t * pw, sizeof(int32_t) * (size_t)pw);
    }
    return 0;
}

/* The rescue: for each row that enters the second round, the candidates are,
 * at flat positions r * n + j, the round-1 words of the ranks whose bit is
 * clear with ord16 >= tau16 (sat_word's low half), then at W * n + s * k + j
 * the words of receive slot s, owned by the s-th set bit of the mask.  The
 * top k under (ord16 desc, gid asc) overwrite out_ids[t] as gids in flat
 * position order, then -1.  Other rows are not written. */
int oracle_merge_rescue_rank_major(const int32_t* gathered, const int32_t* recv, int32_t world,
                                   int64_t rows, int32_t n, int32_t k, const int32_t* sat_word,
                                   int32_t* out_ids) {
    if (world < 1 || world > 16 || rows < 0 || n < 32 || n % 32 != 0 || k < 32 || k % 32 != 0)
        return -1;
    const int64_t gw = (int64_t)n + n / 32, pw = (int64_t)k + k / 32, slots = (k - 1) / n;
    const int64_t ncand = (int64_t)world * n + slots * k;
    mcand_t* buf = (mcand_t*)malloc(sizeof(mcand_t) * (size_t)ncand);
    if (!buf) return -2;
    for (int64_t t = 0; t < rows; ++t) {
        const uint32_t sw = (uint32_t)sat_word[t];
        if (!rescue_row_mask(sw, world, n, k)) continue;
        const uint32_t mask = sw >> 16, tau16 = sw & 0xFFFFu;
        int32_t owner[16];
        int32_t nsat = 0;
        for (int32_t r = 0; r < world; ++r)
            if ((mask >> r) & 1u) owner[nsat++] = r;
        int64_t cnt = 0;
        for (int64_t f = 0; f < ncand; ++f) {
            const int32_t* p;
            int32_t j, len, r;
            if (f < (int64_t)world * n) {
                r = (int32_t)(f / n);
                j = (int32_t)(f % n);
                if ((mask >> r) & 1u) continue;
                p = gathered + ((int64_t)r * rows + t) * gw;
                len = n;
            } else {
                int64_t s = (f - (int64_t)world * n) / k;
                if (s >= nsat) continue;
                r = owner[s];
                j = (int32_t)((f - (int64_t)world * n) % k);
                p = recv + (t * slots + s) * pw;
                len = k;
            }
            uint32_t w = (uint32_t)p[j];
            if (w == 0) continue;
            if (f < (int64_t)world * n && (w >> 16) < tau16) continue;
            uint32_t plane = (uint32_t)p[len + j / 32];
            int64_t local = (int64_t)(0xFFFFu - (w & 0xFFFFu)) |
                            ((int64_t)((plane >> (j % 32)) & 1u) << 16);
            buf[cnt].o = w >> 16;
            buf[cnt].gid = local * world + r;
            buf[cnt].pos = f;
            ++cnt;
        }
        qsort(buf, (size_t)cnt, sizeof(mcand_t), mcand_cmp);
        const int64_t m = cnt < k ? cnt : k;
        /* emit the chosen in flat position order */
        qsort(buf, (size_t)m, sizeof(mcand_t), mcand_pos_cmp);
        const mcand_t* chosen = buf;
        int32_t* o = out_ids + t * k;
        for (int64_t q = 0; q < m; ++q) o[q] = (int32_t)chosen[q].gid;
        for (int64_t q = m; q < k; ++q) o[q] = -1;
    }
    free(buf);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O4: pair candidates and their select ([P1] Overview + Details)      */
/* ------------------------------------------------------------------ */

/*
 * pairs[t, j] = (fp32 bits of x[t, l], l * world + rank) for l = local_idx[t, j]
 * with 0 <= l < min(row_end or cols, cols) and x[t, l] not NaN;
 * otherwise (0, -1), the empty pair.
 */
int oracle_pack_pairs(const float* x, int64_t rows, int64_t cols, int64_t ld,
                      const int32_t* local_idx, int32_t kc, int64_t ld_idx,
                      const int32_t* row_ends, int32_t rank, int32_t world, int32_t* pairs) {
    if (rows < 0 || cols < 0 || ld < cols || kc < 1 || ld_idx < kc || world < 1 ||
        rank < 0 || rank >= world)
        return -1;
    for (int64_t t = 0; t < rows; ++t) {
        int64_t end = clamp_end(row_ends, t, cols);
        for (int32_t j = 0; j < kc; ++j) {
            int64_t l = local_idx[t * ld_idx + j];
            int32_t* p = pairs + (t * kc + j) * 2;
            p[0] = 0;
            p[1] = -1;
            if (l >= 0 && l < end) {
                float v = x[t * ld + l];
                if (!isnan(v)) {
                    memcpy(&p[0], &v, sizeof v);
                    p[1] = (int32_t)(l * world + rank);
                }
            }
        }
    }
    return 0;
}

/*
 * pairs is int32 [world, rows, kc, 2]: [..., 0] the fp32 score bits,
 * [..., 1] the global id (negative = empty).  NaN scores are dropped.
 * The K selected are the first min(K, count) under (score desc, -0 below +0,
 * gid asc); out_ids[row] lists their gids in candidate order (r, then j),
 * then -1 up to k.
 */
int oracle_merge_select_pairs_rank_major(const int32_t* pairs, int32_t world, int64_t rows,
                                         int32_t kc, int32_t k, int32_t* out_ids) {
    if (world < 1 || rows < 0 || kc < 1 || k < 1) return -1;
    int64_t total = (int64_t)world * kc;
    cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)total);
    unsigned char* sel = (unsigned char*)malloc((size_t)total);
    if (!buf || !sel) {
        free(buf);
        free(sel);
        return -2;
    }
    for (int64_t t = 0; t < rows; ++t) {
        int64_t cnt = 0;
        for (int32_t r = 0; r < world; ++r) {
            const int32_t* p = pairs + (((int64_t)r * rows + t) * kc) * 2;
            for (int32_t j = 0; j < kc; ++j) {
                int32_t gid = p[2 * j + 1];
                float v = bits_to_float((uint32_t)p[2 * j]);
                if (gid < 0 || isnan(v)) continue;
                buf[cnt].v = v;
                buf[cnt].id = gid;
                buf[cnt].pos = (int64_t)r * kc + j;
                ++cnt;
            }
        }
        qsort(buf, (size_t)cnt, sizeof(cand_t), cand_cmp);
        int64_t m = cnt < k ? cnt : k;
        memset(sel, 0, (size_t)total);
        for (int64_t q = 0; q < m; ++q) sel[buf[q].pos] = 1;
        int32_t* o = out_ids + t * k;
        int64_t w_at = 0;
        for (int64_t f = 0; f < total; ++f) {
            if (!sel[f]) continue;
            int32_t r = (int32_t)(f / kc), j = (int32_t)(f % kc);
            o[w_at++] = pairs[(((int64_t)r * rows + t) * kc + j) * 2 + 1];
        }
        for (int64_t q = w_at; q < k; ++q) o[q] = -1;
    }
    free(buf);
    free(sel);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O5: a rank's owned physical KV rows of the selected ids ([P2]      */
/*     DCPTopkSelectKernel docstring on emit_rows, dcp_topk_merge_rows) */
/* ------------------------------------------------------------------ */

/* For each row t, walk ids[t, 0:k) in order; a gid >= 0 is owned by
 * dcp_rank when gid % world == dcp_rank.  Its local index local = gid / world
 * lies in KV block b = local / block_size of request req_id[t]; when b is a
 * column of the block table (b < table_cols) the token's physical row
 *   block_table[req_id[t], b] * stride_rows + local % block_size
 * (wrapped to int32) is appended to rows_out[t].  Then -1 up to out_cols and
 * valid_out[t] = the number appended.  A req_id outside [0, table_rows)
 * owns nothing. */
int oracle_emit_rows(const int32_t* ids, int64_t rows, int32_t k, int32_t world, int32_t dcp_rank,
                     const int32_t* req_id, const int32_t* block_table, int64_t table_rows,
                     int32_t table_cols, int32_t block_size, int64_t stride_rows, int32_t* rows_out,
                     int32_t out_cols, int32_t* valid_out) {
    if (rows < 0 || k < 1 || world < 1 || dcp_rank < 0 || dcp_rank >= world || table_rows < 0 ||
        table_cols < 0 || block_size < 1 || out_cols < k)
        return -1;
    for (int64_t t = 0; t < rows; ++t) {
        const int64_t req = req_id[t];
        int32_t cnt = 0;
        int32_t* o = rows_out + t * out_cols;
        if (req >= 0 && req < table_rows) {
            for (int32_t j = 0; j < k; ++j) {
                const int32_t gid = ids[t * k + j];
                if (gid < 0 || gid % world != dcp_rank) continue;
                const int32_t local = gid / world;
                const int32_t b = local / block_size;
                if (b >= table_cols) continue;
                const int64_t phys = (int64_t)block_table[req * table_cols + b] * stride_rows +
                                     (local - b * block_size);
                o[cnt++] = (int32_t)(uint32_t)((uint64_t)phys & 0xFFFFFFFFu);
            }
        }
        valid_out[t] = cnt;
        for (int32_t j = cnt; j < out_cols; ++j) o[j] = -1;
    }
    return 0;
}
