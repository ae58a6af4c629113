// Candidate packing and the rank-major merge selects, for gfx950.
//
// Sources (the kernels page of vllm.models.kimi_k3.nvidia.ops.dcp_topk_merge
// and vLLM PR 65178 "rank-major DCP top-k merge"):
//   * pack: B' word (ord16(score) << 16) | (0xFFFF - local[15:0]) plus a bit
//     plane holding local[16], one plane word per 32 slots; ids outside
//     [0, min(row_end, S, 2^17)) and NaN scores pack as 0 (module docstring
//     step 1, DCPTopkPackKernel, dcp_topk_pack_indices).
//   * packed select: decode every nonzero word to gid = local * W + r and the
//     score key ord16, keep the top k under (ord16 desc, gid asc), and derive
//     sat_word = (mask << 16) | tau16 (module docstring, DCPTopkSelectKernel,
//     _decode_key).
//   * pair select: (score, gid) candidates of the all-gathered [W, R, K, 2]
//     buffer read in place (PR 65178 Overview and Details).
// The packed select runs one wave per row when a row's candidates fit in 64
// registers per lane and world is a power of two up to 16
// (merge_packed_wave_kernel).  The pair select runs one wave per rank of a
// row, with one radix level on the registers and the rest on an LDS list of
// the boundary bin and above (merge_pairs_wave_kernel, up to 2048 pairs per
// rank).  Otherwise (and for the second round) one 512-thread workgroup per
// row holds every candidate in registers as a 64-bit composite
// (key << 32) | (0xFFFFFFFF - gid).  The k-th
// composite is found by a radix select whose 256 bins at each level span
// [min, max] of the composites still in play (so a narrow score range still
// spreads over the bins); histogram atomics go to 16 lane-striped LDS copies
// at a 257-word stride, so lanes that share a digit mostly hit different
// addresses and banks.  Selected ids are written in candidate order (rank,
// then slot), a fixed order that does not depend on the launch geometry.
#include "rts_device.hpp"
#include "rts_levels.hpp"
#include "rts_internal.h"
#include "../../include/row_top_select.h"

namespace rts {

constexpr int kSelBlock = 512;
constexpr int kSelWaves = kSelBlock / kWave;
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;
constexpr int kMaxTab = 64 * kSelWaves;  // KPT * waves entries of the emission table

// Where rank r's candidates of row t start, in units of one rank-row (n + n/32
// words, or kc pairs): r * rank_stride + t * row_stride.  Rank-major
// [W, R, .] (the dim-0 all-gather read in place) is {rows, 1}; row-major
// [R, W, .] (the reordered buffer) is {1, W}.
struct Layout {
    int64_t rank_stride, row_stride;
    __host__ __device__ int64_t at(int64_t r, int64_t row) const { return r * rank_stride + row * row_stride; }
};

// The block-table row of `row` (nullptr: the request is outside the table,
// so the row owns nothing).
__device__ __forceinline__ const int32_t* rows_table_of(const RowsArgs& ra, int64_t row) {
    const int64_t req = ra.req_id[row];
    return (req >= 0 && req < ra.table_rows) ? ra.block_table + req * ra.ld_table : nullptr;
}

// Physical row of local index `local` when its KV block is inside the table.
__device__ __forceinline__ bool owned_phys(const RowsArgs& ra, const int32_t* bt, uint32_t local,
                                           int32_t& phys) {
    const uint32_t b = local / (uint32_t)ra.block_size;
    if (bt == nullptr || b >= (uint32_t)ra.table_cols) return false;
    const int64_t v = (int64_t)bt[b] * ra.stride_rows + (int64_t)(local - b * (uint32_t)ra.block_size);
    phys = (int32_t)(uint32_t)(uint64_t)v;
    return true;
}

struct SelectSmem {
    uint32_t hist[kHistCopies][kHistStride];
    uint32_t bins[256];
    uint64_t red_lo[kSelWaves];
    uint64_t red_hi[kSelWaves];
    uint32_t red_n[kSelWaves];
    uint32_t scal[4];
    uint32_t tab[kMaxTab];
    uint32_t wsum[kSelWaves];
    uint32_t notsat;
};

// ---------------------------------------------------------------------------
// Block-level pieces (all threads of the workgroup call them)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t block_sum(uint32_t v, SelectSmem& sm) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    v = wave_sum32(v);
    if (lane == 0) sm.red_n[wave] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) t += sm.red_n[w];
    __syncthreads();
    return t;
}

// Exclusive scan of one value per thread (thread order); returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& excl, SelectSmem& sm) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan32(v);
    if (lane == kWave - 1) sm.wsum[wave] = incl;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t s = sm.wsum[w];
        off += w < wave ? s : 0u;
        tot += s;
    }
    __syncthreads();
    excl = off + incl - v;
    return tot;
}

// The smallest composite T such that exactly k nonzero keys are >= T (keys
// distinct); requires k <= number of nonzero keys.  With repeated keys more
// than k may be >= T.
template <int KPT>
__device__ uint64_t block_radix_kth(const uint64_t (&key)[KPT], int k, SelectSmem& sm) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    uint64_t lo_edge = 1, hi_edge = ~0ull;
    int need = k;
    // Each level narrows the range by at least 2^7; the cap only bounds the
    // loop if the count invariant were ever broken.
    for (int level = 0;; ++level) {
        uint64_t mn = ~0ull, mx = 0;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const bool in = key[i] >= lo_edge && key[i] <= hi_edge;
            mn = in ? umin64(mn, key[i]) : mn;
            mx = in ? umax64(mx, key[i]) : mx;
        }
        mn = wave_min64(mn);
        mx = wave_max64(mx);
        if (lane == 0) {
            sm.red_lo[wave] = mn;
            sm.red_hi[wave] = mx;
        }
        __syncthreads();
        mn = ~0ull;
        mx = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) {
            mn = umin64(mn, sm.red_lo[w]);
            mx = umax64(mx, sm.red_hi[w]);
        }
        if (mn == mx) return mn;
        const uint64_t d = mx - mn;
        const int bl = 64 - __clzll((long long)d);
        const int s = bl > 8 ? bl - 8 : 0;
        uint32_t* hcopy = sm.hist[lane & (kHistCopies - 1)];
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            if (key[i] >= lo_edge && key[i] <= hi_edge)
                __hip_atomic_fetch_add(&hcopy[(uint32_t)((key[i] - mn) >> s)], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        __syncthreads();
        if (threadIdx.x < 256) {
            uint32_t t = 0;
#pragma unroll
            for (int c = 0; c < kHistCopies; ++c) {
                t += sm.hist[c][threadIdx.x];
                sm.hist[c][threadIdx.x] = 0u;
            }
            sm.bins[threadIdx.x] = t;
        }
        __syncthreads();
        if (wave == 0) {
            uint32_t c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = sm.bins[255 - 4 * lane - j];
            const uint32_t tot = c[0] + c[1] + c[2] + c[3];
            uint32_t run = wave_incl_scan32(tot) - tot;
            bool found = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (run < (uint32_t)need && run + c[j] >= (uint32_t)need) {
                    sm.scal[0] = 255u - 4u * (uint32_t)lane - (uint32_t)j;
                    sm.scal[1] = run;
                    sm.scal[2] = c[j];
                    found = true;
                }
                run += c[j];
            }
            // Defensive: with the count invariant broken, end at the range minimum.
            if (__ballot(found) == 0ull && lane == 0) {
                sm.scal[0] = 0u;
                sm.scal[1] = 0u;
                sm.scal[2] = (uint32_t)need;
            }
        }
        __syncthreads();
        const uint32_t bin = sm.scal[0];
        const uint32_t above = sm.scal[1];
        const uint32_t cb = sm.scal[2];
        need -= (int)above;
        const uint64_t blo = mn + ((uint64_t)bin << s);
        if ((int)cb == need || level >= 12) return blo;
        lo_edge = blo;
        hi_edge = bin == (uint32_t)(d >> s) ? mx : blo + ((1ull << s) - 1ull);
    }
}

// Selection of the keys >= T, written in flat candidate order
// (f = i * kSelBlock + thread) into out[0, k), then -1 up to k.
template <int KPT>
__device__ void block_emit(const uint64_t (&key)[KPT], uint64_t T, int k, int32_t* __restrict__ out,
                           SelectSmem& sm) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    uint64_t m[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        m[i] = __ballot(key[i] != 0ull && key[i] >= T);
        if (lane == 0) sm.tab[i * kSelWaves + wave] = (uint32_t)__popcll(m[i]);
    }
    __syncthreads();
    const int t = threadIdx.x;
    static_assert(KPT * kSelWaves <= kSelBlock, "one table entry per thread");
    const uint32_t v = t < KPT * kSelWaves ? sm.tab[t] : 0u;
    uint32_t excl;
    const uint32_t total = block_excl_scan(v, excl, sm);
    if (t < KPT * kSelWaves) sm.tab[t] = excl;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if ((m[i] >> lane) & 1ull) {
            const uint32_t pos = sm.tab[i * kSelWaves + wave] + mbcnt64(m[i]);
            if (pos < (uint32_t)k) out[pos] = (int32_t)composite_id(key[i]);
        }
    }
    const int filled = total < (uint32_t)k ? (int)total : k;
    for (int p = filled + t; p < k; p += kSelBlock) out[p] = -1;
}

// The owned physical rows of the keys >= T (gid = composite id; owned iff
// gid % world == dcp_rank), in the same flat order as block_emit, then -1 up
// to out_cols, and their count.
template <int KPT>
__device__ void block_emit_rows(const uint64_t (&key)[KPT], uint64_t T, int32_t world, int64_t row,
                                const RowsArgs& ra, SelectSmem& sm) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    __syncthreads();  // block_emit may still be reading sm.tab
    const int32_t* bt = rows_table_of(ra, row);
    uint64_t m[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const uint32_t gid = composite_id(key[i]);
        const uint32_t local = gid / (uint32_t)world;
        int32_t phys;
        const bool own = key[i] != 0ull && key[i] >= T && gid - local * (uint32_t)world == (uint32_t)ra.dcp_rank &&
                         owned_phys(ra, bt, local, phys);
        m[i] = __ballot(own);
        if (lane == 0) sm.tab[i * kSelWaves + wave] = (uint32_t)__popcll(m[i]);
    }
    __syncthreads();
    const int t = threadIdx.x;
    const uint32_t v = t < KPT * kSelWaves ? sm.tab[t] : 0u;
    uint32_t excl;
    const uint32_t total = block_excl_scan(v, excl, sm);
    if (t < KPT * kSelWaves) sm.tab[t] = excl;
    __syncthreads();
    // With distinct composites at most k keys are >= T; repeated candidates
    // (outside the contract) can select more, so every position is bounded
    // by the row's out_cols.
    const uint32_t cap = (uint32_t)ra.out_cols;
    int32_t* orow = ra.rows_out + row * (int64_t)ra.out_cols;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if ((m[i] >> lane) & 1ull) {
            const uint32_t gid = composite_id(key[i]);
            const uint32_t local = gid / (uint32_t)world;
            int32_t phys = -1;
            owned_phys(ra, bt, local, phys);
            const uint32_t pos = sm.tab[i * kSelWaves + wave] + mbcnt64(m[i]);
            if (pos < cap) orow[pos] = phys;
        }
    }
    const uint32_t filled = total < cap ? total : cap;
    for (int p = (int)filled + t; p < ra.out_cols; p += kSelBlock) orow[p] = -1;
    if (t == 0) ra.valid_out[row] = (int32_t)filled;
    __syncthreads();  // sm.tab is reused by the caller
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// One thread per slot; a half-wave covers 32 consecutive slots of one row
// (n is a multiple of 32), so its ballot half is the plane word.
__global__ __launch_bounds__(256) void pack_candidates_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const int32_t* __restrict__ local_idx, int32_t n, int64_t ld_idx,
    const int32_t* __restrict__ row_ends, int32_t* __restrict__ packed) {
    const int64_t gidx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool in = gidx < rows * (int64_t)n;
    const int64_t t = in ? gidx / n : 0;
    const int32_t j = in ? (int32_t)(gidx - t * n) : 0;
    const int64_t width = (int64_t)n + n / 32;
    uint32_t word = 0;
    bool high = false;
    if (in) {
        int64_t end = cols < (1 << 17) ? cols : (1 << 17);
        if (row_ends && (int64_t)row_ends[t] < end) end = row_ends[t];
        const int32_t l = local_idx[t * ld_idx + j];
        if (l >= 0 && (int64_t)l < end) {
            const uint32_t b = x[t * ld + l];
            if ((b & 0x7FFFu) <= 0x7F80u) {
                const uint32_t o = (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
                word = (o << 16) | (0xFFFFu - ((uint32_t)l & 0xFFFFu));
                high = (((uint32_t)l >> 16) & 1u) != 0u;
            }
        }
        packed[t * width + j] = (int32_t)word;
    }
    const uint64_t m = __ballot(high);
    const int lane = lane_id();
    if (in && (lane & 31) == 0)
        packed[t * width + n + j / 32] = (int32_t)(lane < 32 ? (uint32_t)m : (uint32_t)(m >> 32));
}

__global__ __launch_bounds__(256) void pack_pairs_kernel(
    const float* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const int32_t* __restrict__ local_idx, int32_t kc, int64_t ld_idx,
    const int32_t* __restrict__ row_ends, int32_t rank, int32_t world, int32_t* __restrict__ pairs) {
    const int64_t gidx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gidx >= rows * (int64_t)kc) return;
    const int64_t t = gidx / kc;
    const int32_t j = (int32_t)(gidx - t * kc);
    int64_t end = row_ends ? (int64_t)row_ends[t] : cols;
    end = end < 0 ? 0 : (end > cols ? cols : end);
    const int32_t l = local_idx[t * ld_idx + j];
    int32_t s = 0, id = -1;
    if (l >= 0 && (int64_t)l < end) {
        const uint32_t u = __float_as_uint(x[t * ld + l]);
        if (!f32_bits_is_nan(u)) {
            s = (int32_t)u;
            id = l * world + rank;
        }
    }
    typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
    i32x2 pr;
    pr[0] = s;
    pr[1] = id;
    reinterpret_cast<i32x2*>(pairs)[gidx] = pr;
}

// flat candidate index f = i * kSelBlock + thread  ->  (rank r, slot j)
struct FlatWalk {
    int32_t r, j, q0, r0, n;
    __device__ FlatWalk(int32_t n_, int32_t t) : n(n_) {
        r = t / n_;
        j = t - r * n_;
        q0 = kSelBlock / n_;
        r0 = kSelBlock - q0 * n_;
    }
    __device__ void next() {
        r += q0;
        j += r0;
        if (j >= n) {
            j -= n;
            ++r;
        }
    }
};

template <int KPT, bool ROWS>
__global__ __launch_bounds__(kSelBlock) void merge_packed_kernel(
    const int32_t* __restrict__ gathered, Layout lay, int32_t world, int64_t rows, int32_t n,
    int32_t k, int32_t* __restrict__ out_ids, int32_t* __restrict__ sat_word, RowsArgs ra) {
    __shared__ SelectSmem sm;
    const int t = threadIdx.x, lane = lane_id();
    const int64_t row = blockIdx.x;
    const int64_t width = (int64_t)n + n / 32;
    const int32_t total = world * n;

    for (int q = t; q < kHistCopies * kHistStride; q += kSelBlock) (&sm.hist[0][0])[q] = 0u;
    if (t == 0) sm.notsat = 0u;

    uint64_t key[KPT];
    {
        FlatWalk w(n, t);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            key[i] = 0ull;
            if (i * kSelBlock + t < total) {
                const int32_t* rowp = gathered + lay.at(w.r, row) * width;
                const uint32_t word = (uint32_t)rowp[w.j];
                const uint32_t plane = (uint32_t)rowp[n + (w.j >> 5)];
                if (word != 0u) {
                    const uint32_t local =
                        (0xFFFFu - (word & 0xFFFFu)) | (((plane >> (w.j & 31)) & 1u) << 16);
                    const uint32_t gid = local * (uint32_t)world + (uint32_t)w.r;
                    key[i] = composite(word >> 16, gid);
                }
            }
            w.next();
        }
    }
    uint32_t nz = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) nz += key[i] != 0ull;
    __syncthreads();
    const uint32_t nvalid = block_sum(nz, sm);

    uint64_t T = 1ull;
    if (nvalid > (uint32_t)k) T = block_radix_kth<KPT>(key, k, sm);
    if (out_ids) block_emit<KPT>(key, T, k, out_ids + row * (int64_t)k, sm);
    if constexpr (ROWS) block_emit_rows<KPT>(key, T, world, row, ra, sm);

    if (sat_word) {
        // tau16: ord16 of the k-th selected composite (the smallest selected).
        uint64_t mn = ~0ull;
#pragma unroll
        for (int i = 0; i < KPT; ++i) mn = (key[i] != 0ull && key[i] >= T) ? umin64(mn, key[i]) : mn;
        mn = wave_min64(mn);
        const int wave = t / kWave;
        if (lane == 0) sm.red_lo[wave] = mn;
        __syncthreads();
        mn = ~0ull;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) mn = umin64(mn, sm.red_lo[w]);
        const uint32_t tau = nvalid >= (uint32_t)k ? (uint32_t)(mn >> 32) : 0u;
        // Rank r is saturated iff all its n words are nonzero with ord16 > tau.
        FlatWalk w(n, t);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const bool cand = i * kSelBlock + t < total;
            const bool bad = cand && (key[i] == 0ull || (uint32_t)(key[i] >> 32) <= tau);
            const uint32_t bits = wave_or32(bad ? (1u << w.r) : 0u);
            if (lane == 0 && bits)
                __hip_atomic_fetch_or(&sm.notsat, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            w.next();
        }
        __syncthreads();
        if (t == 0) {
            uint32_t mask = ~sm.notsat & ((1u << world) - 1u);
            if (__popc(mask) > (k - 1) / n) mask = 0u;
            sat_word[row] = (int32_t)((mask << 16) | tau);
        }
    }
}

// ---------------------------------------------------------------------------
// Second round of the packed merge (kernels page: module docstring on
// exactness, DCPTopkRescueKernel, DCPTopkRescueWorkspace), with every rank's
// push landing in one receive buffer recv [rows, S, k + k/32], S = (k-1)/n.
//
// A row takes part iff its mask is nonzero, names only ranks below world and
// has at most S bits; round 1 writes no other nonzero mask, and other rows are
// left as they are (a mask check is all they cost).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool rescue_row(uint32_t sw, int32_t world, int32_t slots) {
    const uint32_t mask = sw >> 16;
    return mask != 0u && (mask >> world) == 0u && __popc(mask) <= slots;
}

// The push of one saturated rank: its packed local top-k of the row into
// receive slot popc(mask & ((1 << rank) - 1)).  One wave per row.
__global__ __launch_bounds__(256) void rescue_push_kernel(
    const int32_t* __restrict__ local_packed, int32_t rank, int32_t world, int64_t rows, int32_t n,
    int32_t k, const int32_t* __restrict__ sat_word, int32_t* __restrict__ recv) {
    const int64_t row = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
    if (row >= rows) return;
    const uint32_t sw = (uint32_t)sat_word[row];
    const int32_t slots = (k - 1) / n;
    if (!rescue_row(sw, world, slots) || !((sw >> 16) >> rank & 1u)) return;
    const int64_t pw = (int64_t)k + k / 32;
    const int64_t slot = __popc((sw >> 16) & ((1u << rank) - 1u));
    const int32_t* src = local_packed + row * pw;
    int32_t* dst = recv + (row * slots + slot) * pw;
    for (int64_t q = lane_id(); q < pw; q += kWave) dst[q] = src[q];
}

// The rescue select of one row (all threads of the workgroup).  Flat
// candidate f = i * kSelBlock + thread: f < world * n is round-1 slot
// (r, j) = (f / n, f % n), a candidate when rank r is not saturated and its
// ord16 >= tau16; f >= world * n is slot j of receive slot s,
// (s, j) = ((f - world*n) / k, (f - world*n) % k), owned by the s-th set bit
// of the mask.  Selection and emission in flat order are the round-1 block
// kernel's.
template <int KPT, bool IN_LOOP, bool ROWS>
__device__ __forceinline__ void rescue_one_row(const int32_t* __restrict__ gathered,
                                               const int32_t* __restrict__ recv, int32_t world,
                                               int64_t rows, int32_t n, int32_t k, int64_t row,
                                               uint32_t sw, int32_t* __restrict__ out_ids,
                                               const RowsArgs& ra, SelectSmem& sm) {
    // Inside a row loop, an opaque copy of the thread index renewed per row:
    // without it the compiler hoists the per-register slot arithmetic out of
    // the loop and keeps all of it live across rows.
    int t = threadIdx.x;
    if constexpr (IN_LOOP) asm volatile("" : "+v"(t));
    const int32_t slots = (k - 1) / n;
    const uint32_t mask = sw >> 16, tau16 = sw & 0xFFFFu;
    const int32_t nsat = __popc(mask);
    const int64_t gw = (int64_t)n + n / 32, pw = (int64_t)k + k / 32;
    const uint32_t r1 = (uint32_t)(world * n);
    const uint32_t total = r1 + (uint32_t)nsat * (uint32_t)k;

    // Candidate words and their plane words are loaded a batch of KB
    // registers at a time, every load of a batch in flight before the first
    // is used (the plane load does not wait for the word's test).
    constexpr int KB = KPT < 8 ? KPT : 8;
    uint64_t key[KPT];
#pragma unroll
    for (int ib = 0; ib < KPT; ib += KB) {
        uint32_t wv[KB], pv[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const uint32_t f = (uint32_t)((ib + b) * kSelBlock + t);
            wv[b] = 0u;
            pv[b] = 0u;
            if (f < r1) {
                const uint32_t r = f / (uint32_t)n, j = f - r * (uint32_t)n;
                if (!((mask >> r) & 1u)) {
                    const int32_t* rowp = gathered + ((int64_t)r * rows + row) * gw;
                    wv[b] = (uint32_t)rowp[j];
                    pv[b] = (uint32_t)rowp[n + (j >> 5)];
                }
            } else if (f < total) {
                const uint32_t fr = f - r1, s = fr / (uint32_t)k, j = fr - s * (uint32_t)k;
                const int32_t* slotp = recv + (row * slots + (int64_t)s) * pw;
                wv[b] = (uint32_t)slotp[j];
                pv[b] = (uint32_t)slotp[k + (j >> 5)];
            }
        }
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const int i = ib + b;
            const uint32_t f = (uint32_t)(i * kSelBlock + t);
            const uint32_t word = wv[b];
            key[i] = 0ull;
            if (f < r1) {
                const uint32_t r = f / (uint32_t)n, j = f - r * (uint32_t)n;
                // words of saturated ranks were not loaded (0)
                if (word != 0u && (word >> 16) >= tau16) {
                    const uint32_t local = (0xFFFFu - (word & 0xFFFFu)) | (((pv[b] >> (j & 31)) & 1u) << 16);
                    key[i] = composite(word >> 16, local * (uint32_t)world + r);
                }
            } else if (f < total) {
                const uint32_t fr = f - r1, s = fr / (uint32_t)k, j = fr - s * (uint32_t)k;
                // owner: the s-th set bit of the mask
                uint32_t m = mask;
                for (uint32_t c = 0; c < s; ++c) m &= m - 1u;
                const uint32_t owner = (uint32_t)__builtin_ctz(m);
                if (word != 0u) {
                    const uint32_t local = (0xFFFFu - (word & 0xFFFFu)) | (((pv[b] >> (j & 31)) & 1u) << 16);
                    key[i] = composite(word >> 16, local * (uint32_t)world + owner);
                }
            }
        }
    }
    uint32_t nz = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) nz += key[i] != 0ull;
    __syncthreads();
    const uint32_t nvalid = block_sum(nz, sm);

    uint64_t T = 1ull;
    if (nvalid > (uint32_t)k) T = block_radix_kth<KPT>(key, k, sm);
    if (out_ids) block_emit<KPT>(key, T, k, out_ids + row * (int64_t)k, sm);
    if constexpr (ROWS) block_emit_rows<KPT>(key, T, world, row, ra, sm);
    if constexpr (IN_LOOP) __syncthreads();  // block_emit's table is reused by the next row
}

// One workgroup per row (grid = rows); a row that does not enter returns at once.
template <int KPT, bool ROWS>
__global__ __launch_bounds__(kSelBlock) void merge_rescue_row_kernel(
    const int32_t* __restrict__ gathered, const int32_t* __restrict__ recv, int32_t world,
    int64_t rows, int32_t n, int32_t k, const int32_t* __restrict__ sat_word,
    int32_t* __restrict__ out_ids, RowsArgs ra) {
    __shared__ SelectSmem sm;
    const int64_t row = blockIdx.x;
    const uint32_t sw = (uint32_t)sat_word[row];
    if (!rescue_row(sw, world, (k - 1) / n)) return;
    for (int q = threadIdx.x; q < kHistCopies * kHistStride; q += kSelBlock) (&sm.hist[0][0])[q] = 0u;
    rescue_one_row<KPT, false, ROWS>(gathered, recv, world, rows, n, k, row, sw, out_ids, ra, sm);
}

// Rows dealt to workgroups with stride gridDim.x.  A workgroup reads the
// sat_words of up to kSelBlock of its rows at once (one per thread), lists
// those that enter the second round in LDS, then selects them one by one, so
// a row that does not enter costs one word load and no workgroup launch.
// Held to 4 waves per SIMD (two workgroups per compute unit).
template <int KPT, bool ROWS>
__global__ __launch_bounds__(kSelBlock) __attribute__((amdgpu_waves_per_eu(4)))
void merge_rescue_kernel(const int32_t* __restrict__ gathered, const int32_t* __restrict__ recv,
                         int32_t world, int64_t rows, int32_t n, int32_t k,
                         const int32_t* __restrict__ sat_word, int32_t* __restrict__ out_ids,
                         RowsArgs ra) {
    __shared__ SelectSmem sm;
    __shared__ uint32_t todo[kSelBlock];
    __shared__ uint32_t todo_sw[kSelBlock];
    const int t = threadIdx.x, lane = lane_id(), wave = t / kWave;
    const int32_t slots = (k - 1) / n;
    bool hist_clear = false;
    for (int64_t base = blockIdx.x; base < rows; base += (int64_t)gridDim.x * kSelBlock) {
        const int64_t my = base + (int64_t)t * gridDim.x;
        const uint32_t sw = my < rows ? (uint32_t)sat_word[my] : 0u;
        const bool need = my < rows && rescue_row(sw, world, slots);
        const uint64_t bal = __ballot(need);
        if (lane == 0) sm.wsum[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t off = 0, cnt = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) {
            off += w < wave ? sm.wsum[w] : 0u;
            cnt += sm.wsum[w];
        }
        if (need) {
            const uint32_t p = off + mbcnt64(bal);
            todo[p] = (uint32_t)t;
            todo_sw[p] = sw;
        }
        __syncthreads();
        if (cnt != 0u && !hist_clear) {
            for (int q = t; q < kHistCopies * kHistStride; q += kSelBlock) (&sm.hist[0][0])[q] = 0u;
            hist_clear = true;  // every radix level leaves the copies zeroed
        }
        for (uint32_t q = 0; q < cnt; ++q) {
            const int64_t row = base + (int64_t)todo[q] * gridDim.x;
            rescue_one_row<KPT, true, ROWS>(gathered, recv, world, rows, n, k, row, todo_sw[q], out_ids,
                                            ra, sm);
        }
    }
}

// ---------------------------------------------------------------------------
// A rank's owned physical KV rows of the selected ids (kernels page:
// DCPTopkSelectKernel docstring on emit_rows, dcp_topk_merge_rows).  One wave
// per row: lane l holds ids[t, c*64 + l] in register c; owned ids (gid % W ==
// dcp_rank, KV block inside the table) are compacted in id order with a
// ballot prefix, so the rows come out in the order the ids list them.
// ---------------------------------------------------------------------------
constexpr int kEmitRegs = 32;  // 32 * 64 = 2048 ids per row at most

__global__ __launch_bounds__(256) void emit_rows_kernel(
    const int32_t* __restrict__ ids, int64_t rows, int32_t k, int32_t world, int32_t dcp_rank,
    const int32_t* __restrict__ req_id, const int32_t* __restrict__ block_table, int64_t table_rows,
    int32_t table_cols, int64_t ld_table, int32_t block_size, int64_t stride_rows,
    int32_t* __restrict__ rows_out, int32_t out_cols, int32_t* __restrict__ valid_out) {
    const int64_t row = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
    if (row >= rows) return;
    const int lane = lane_id();
    const int64_t req = req_id[row];
    const bool req_ok = req >= 0 && req < table_rows;
    const int32_t* idr = ids + row * (int64_t)k;
    int32_t* outr = rows_out + row * (int64_t)out_cols;
    const int32_t* bt = block_table + (req_ok ? req : 0) * ld_table;

    int32_t g[kEmitRegs];
#pragma unroll
    for (int c = 0; c < kEmitRegs; ++c) {
        const int j = c * kWave + lane;
        g[c] = (req_ok && j < k) ? idr[j] : -1;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int c = 0; c < kEmitRegs; ++c) {
        if (c * kWave < k) {  // uniform
            const int32_t gid = g[c];
            const int32_t local = gid / world;
            const int32_t b = local / block_size;
            const bool own = gid >= 0 && gid - local * world == dcp_rank && b < table_cols;
            const uint64_t m = __ballot(own);
            if (own) {
                const int64_t phys = (int64_t)bt[b] * stride_rows + (local - b * block_size);
                outr[cnt + mbcnt64(m)] = (int32_t)(uint32_t)(uint64_t)phys;
            }
            cnt += (uint32_t)__popcll(m);
        }
    }
    for (int32_t j = (int32_t)cnt + lane; j < out_cols; j += kWave) outr[j] = -1;
    if (lane == 0) valid_out[row] = (int32_t)cnt;
}

// ---------------------------------------------------------------------------
// Packed select, one wave per row, no barriers (world * ceil(n/64) <= 64).
//
// Lane l holds, for rank r and q = 0 .. qn-1, the word of slot j = q*64 + l in
// register i = r*qn + q, and bit i of hb holds that slot's plane bit (local
// bit 16).  Register order then lane order is candidate order (r*n + j), so a
// running count plus the lane's rank among the register's selected lanes is
// the output position.
//   1. ord16 threshold: 256-bin levels over the score half of the words in
//      [min, max] of the nonzero ones (one level when the scores span fewer
//      than 256 ord16 values, two at most).  The bins are counted in four
//      lane-striped copies: bf16 scores crowd into a few bins of the first
//      level (a bin is a binade there), and lanes sharing a bin then mostly
//      hit different addresses.
//   2. Ties at tau16 (the k-th score): the candidates tied there are taken by
//      ascending gid; up to 64 of them are sorted in one register, more go
//      through 256-bin levels over the gid.
//   3. Emission in candidate order, -1 tail; tau16 and the saturation mask
//      come out of the same pass.  A score test on the whole word: ord16 >
//      thr  <=>  word > (thr << 16 | 0xFFFF), and "empty or ord16 <= tau16"
//      <=>  word < (tau16 + 1) << 16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t packed_gid(uint32_t word, uint32_t hibit, uint32_t world, uint32_t r) {
    const uint32_t local = (0xFFFFu - (word & 0xFFFFu)) | (hibit << 16);
    return local * world + r;
}

template <int QN, int W, bool ROWS>
__global__ __launch_bounds__(kWave) void merge_packed_wave_kernel(
    const int32_t* __restrict__ gathered, Layout lay, int32_t world_, int64_t rows, int32_t n,
    int32_t k, int32_t* __restrict__ out_ids, int32_t* __restrict__ sat_word, RowsArgs ra) {
    constexpr int NR = QN * W;  // registers: rank r = i / QN, q = i % QN
    constexpr int32_t world = W;
    (void)world_;
    __shared__ __attribute__((aligned(16))) uint32_t hist[kStripedWords];
    __shared__ uint32_t tied[kWave];
    const int lane = lane_id();
    const int64_t row = blockIdx.x;
    const int64_t width = (int64_t)n + n / 32;

    uint32_t w[NR];
    uint32_t hb0 = 0u, hb1 = 0u;  // bit i (hb1: i - 32): the slot's plane bit (local bit 16)
    // A rank's n/32 plane words are read one per lane (a vector load, not
    // n/32 scalar registers per rank); slot q*64 + l takes bit l % 32 of word
    // 2q + l/32, fetched from the lane that holds it.  A rank whose plane is
    // all zero (local ids below 2^16, the common case) skips the fetches.
    const int npw = n / 32;
#pragma unroll
    for (int r = 0; r < W; ++r) {
        const int32_t* rp = gathered + lay.at(r, row) * width;
        const uint32_t pw = lane < npw ? (uint32_t)rp[n + lane] : 0u;
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int i = r * QN + q;
            // Only the last register of a rank can reach past n (n % 64 == 32).
            const bool in = q < QN - 1 || q * kWave + lane < n;
            const uint32_t word = (uint32_t)rp[in ? q * kWave + lane : 0];
            w[i] = in ? word : 0u;
        }
        if (__ballot(pw != 0u)) {
#pragma unroll
            for (int q = 0; q < QN; ++q) {
                const int i = r * QN + q;
                const bool in = q < QN - 1 || q * kWave + lane < n;
                const int src = 2 * q + (lane >> 5);
                const uint32_t pword = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)pw);
                const uint32_t bit = in ? (pword >> (lane & 31)) & 1u : 0u;
                if (i < 32) hb0 |= bit << i;
                else hb1 |= bit << (i - 32);
            }
        }
    }
    auto hibit = [&](int i) -> uint32_t { return i < 32 ? (hb0 >> i) & 1u : (hb1 >> (i - 32)) & 1u; };
    // Each pass recomputes what it derives from w[] (a shift, a compare): kept
    // from pass to pass, those values would hold ~NR more registers and NR mask
    // pairs.  An empty asm per register makes every pass start from w[].
    auto fresh = [&]() {
#pragma unroll
        for (int i = 0; i < NR; ++i) asm volatile("" : "+v"(w[i]));
    };

    // Valid count and the ord16 range of the nonzero words (ord16 >= 0x7F
    // for every packed score, so 0 marks an empty slot).
    uint32_t nz = 0, mn = 0xFFFFu, mx = 0u;
    fresh();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const uint32_t o = w[i] >> 16;
        nz += (uint32_t)__popcll(__ballot(w[i] != 0u));
        mn = (w[i] != 0u && o < mn) ? o : mn;
        mx = o > mx ? o : mx;
    }
    mn = wave_min32(mn);
    mx = wave_max32(mx);

    // Selection rule: ord16 > thr_gt, or ord16 == tie16 and gid <= gid_cut.
    // Every pass below starts with fresh() outside its (uniform) condition, so
    // w[] has one version throughout and branches only decide scalars.
    uint32_t thr_gt = 0u, tie16 = 0u, gid_cut = 0u;
    uint32_t tau16 = nz == (uint32_t)k ? mn : 0u;  // the k-th selected score (0: fewer than k)
    bool tau_from_min = false;
    int need = k;
    bool open = nz > (uint32_t)k;  // the score threshold is still to be found
    uint32_t wlo = mn, span = mx - mn;
    const int bl = span ? 32 - __clz((int)span) : 0;
    uint32_t sh = bl > 8 ? (uint32_t)(bl - 8) : 0u;
    bool ties = false;  // the k-th score is tied: take `need` of the tied ones by gid
    uint32_t ntied = 0u;
#pragma unroll
    for (int level = 0; level < 2; ++level) {  // a 16-bit score needs two levels at most
        fresh();
        if (open) {
            striped_clear(hist);
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const uint32_t x = (w[i] >> 16) - wlo;  // empty: wraps past span
                if (x <= span) striped_add(hist, x >> sh);
            }
            wave_lds_sync();
            uint32_t bin, cb;
            if (!striped_find(hist, need, bin, cb)) {  // only if counts were inconsistent
                thr_gt = wlo - 1u;
                tau_from_min = true;
                open = false;
            } else {
                const uint32_t blo = wlo + (bin << sh);
                if ((int)cb == need) {  // every entry of the bin is taken
                    thr_gt = blo - 1u;
                    tau_from_min = sh > 0;
                    tau16 = blo;
                    open = false;
                } else if (sh == 0) {
                    thr_gt = blo;
                    tie16 = blo;
                    tau16 = blo;
                    ties = true;
                    ntied = cb;
                    open = false;
                } else {
                    wlo = blo;
                    const uint32_t top = mx - blo, width1 = (1u << sh) - 1u;
                    span = width1 < top ? width1 : top;
                    sh = sh > 8 ? sh - 8 : 0u;
                }
            }
        }
    }
    if (open) {  // not reached: two levels always resolve a 16-bit score
        thr_gt = wlo - 1u;
        tau_from_min = true;
    }
    // Up to 64 tied candidates: sort their gids in one register.  A register
    // with no tied lane (most of them) costs a compare and a ballot.
    fresh();
    if (ties && ntied <= (uint32_t)kWave) {
        int base = 0;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const bool t = (w[i] >> 16) == tie16;
            const uint64_t m = __ballot(t);
            if (m) {
                if (t) tied[base + (int)mbcnt64(m)] =
                    packed_gid(w[i], hibit(i), (uint32_t)world, (uint32_t)(i / QN));
                base += (int)__popcll(m);
            }
        }
        wave_lds_sync();
        uint64_t sv[1] = {lane < (int)ntied ? (uint64_t)tied[lane] : ~0ull};
        wave_bitonic_sort<1, false>(sv);
        gid_cut = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)sv[0], need - 1);
    }
    // More: 256-bin levels over key = 2^21-1-gid among the tied candidates.
    {
        bool gopen = ties && ntied > (uint32_t)kWave;
        uint32_t gw = 0u, gspan = (1u << 21) - 1u, gs = 13u;
#pragma unroll
        for (int gl = 0; gl < 3; ++gl) {
            fresh();
            if (gopen) {
                striped_clear(hist);
                wave_lds_sync();
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    if ((w[i] >> 16) == tie16) {
                        const uint32_t key = ((1u << 21) - 1u) -
                            packed_gid(w[i], hibit(i), (uint32_t)world, (uint32_t)(i / QN));
                        const uint32_t x = key - gw;
                        if (x <= gspan) striped_add(hist, x >> gs);
                    }
                }
                wave_lds_sync();
                uint32_t gbin, gcb;
                if (!striped_find(hist, need, gbin, gcb)) {
                    gopen = false;
                } else {
                    gw += gbin << gs;
                    if ((int)gcb == need || gs == 0) {
                        gopen = false;
                    } else {
                        gspan = (1u << gs) - 1u;
                        gs = gs > 8 ? gs - 8 : 0u;
                    }
                }
            }
        }
        if (ties && ntied > (uint32_t)kWave) gid_cut = ((1u << 21) - 1u) - gw;
    }
    fresh();
    if (tau_from_min) {
        uint32_t t = 0xFFFFu;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const uint32_t o = w[i] >> 16;
            t = (w[i] != 0u && o > thr_gt && o < t) ? o : t;
        }
        tau16 = wave_min32(t);
    }
    if (nz <= (uint32_t)k) thr_gt = 0u;  // every nonzero word is selected

    // Emission in candidate order; saturation: rank r keeps its bit iff all n
    // of its words are nonzero with a score above tau16.  Owned physical rows
    // (when requested) are the selected words of rank dcp_rank, in the same
    // order.  thr_gt <= 0xFF80 (the largest ord16) and tau16 <= 0xFF80, so
    // neither word bound overflows.
    int32_t* o_row = out_ids ? out_ids + row * (int64_t)k : nullptr;
    constexpr bool want_rows = ROWS;
    const int32_t* bt = want_rows ? rows_table_of(ra, row) : nullptr;
    int32_t* r_row = want_rows ? ra.rows_out + row * (int64_t)ra.out_cols : nullptr;
    const uint32_t sel_w = (thr_gt << 16) | 0xFFFFu;  // word > sel_w  <=>  ord16 > thr_gt
    const uint32_t sat_w = (tau16 + 1u) << 16;        // word < sat_w  <=>  empty or ord16 <= tau16
    int base = 0, rbase = 0;
    uint32_t notsat = 0u;
    // One emission loop for both cases (without ties, tie16 = 0 matches no
    // nonzero word): two specialised loops would let the compiler hoist the
    // gids of every register above the branch.
    fresh();
#pragma unroll
    for (int r = 0; r < W; ++r) {
        uint64_t bad = 0ull;
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int i = r * QN + q;
            const uint32_t gid = packed_gid(w[i], hibit(i), (uint32_t)world, (uint32_t)r);
            const bool sel = w[i] > sel_w || ((w[i] >> 16) == tie16 && gid <= gid_cut);
            const uint64_t m = __ballot(sel);
            const int pos = base + (int)mbcnt64(m);
            if (o_row && sel && pos < k) o_row[pos] = (int32_t)gid;
            base += (int)__popcll(m);
            bad |= __ballot((q < QN - 1 || q * kWave + lane < n) && w[i] < sat_w);
            if (want_rows && r == ra.dcp_rank) {  // uniform
                int32_t phys = -1;
                const bool own = sel && owned_phys(ra, bt, gid / (uint32_t)world, phys);
                const uint64_t om = __ballot(own);
                const int rp = rbase + (int)mbcnt64(om);
                if (own && rp < ra.out_cols) r_row[rp] = phys;
                rbase += (int)__popcll(om);
            }
        }
        if (bad) notsat |= 1u << r;
    }
    if (o_row)
        for (int p = (base < k ? base : k) + lane; p < k; p += kWave) o_row[p] = -1;
    if (want_rows) {
        // rbase exceeds out_cols only with repeated candidates (outside the
        // contract); the rows written stop at out_cols.
        const int filled = rbase < ra.out_cols ? rbase : ra.out_cols;
        for (int p = filled + lane; p < ra.out_cols; p += kWave) r_row[p] = -1;
        if (lane == 0) ra.valid_out[row] = filled;
    }
    if (sat_word && lane == 0) {
        uint32_t mask = ~notsat & ((1u << world) - 1u);
        if (__popc(mask) > (k - 1) / n) mask = 0u;
        sat_word[row] = (int32_t)((mask << 16) | tau16);
    }
}

// ---------------------------------------------------------------------------
// Pair select: one wave per rank, the `world` waves of a workgroup share a
// row.  Lane l of wave r holds
// candidate j = q*64 + l of rank r as a 32-bit score key (0 = empty) and its
// gid in key[q], gid[q]; wave order, register order, lane order is candidate
// order.  Per row:
//   1. One 256-bin level over the keys in [min, max] of the valid ones
//      (atomics into 8 lane-striped copies) finds the bin B holding the k-th
//      key.
//   2. The candidates in bin B or above (the k - need above it plus B's own)
//      are compacted in candidate order into an LDS list; the rest of the row
//      runs on the list (about k entries instead of world * kc registers).
//   3. Further levels over the list entries inside B; ties at the k-th key
//      are sorted by gid in one wave (up to 64) or resolved by levels over
//      the gid.
//   4. Emission in candidate order: each wave emits its own list segment at
//      an offset from the selected counts of the waves before it.
// A row with at most k valid candidates, or whose list would not fit (heavy
// ties), runs the same levels, tie rule and emission over the row re-read
// from memory, so that no candidate registers are held across them.
// ---------------------------------------------------------------------------
constexpr int kPairListCap = 3072;

struct PairSmem {
    static constexpr bool kWave0Find = true;
    uint32_t hist[kLevelCopies][kLevelStride];
    uint32_t bins[256];
    uint32_t red[16][4];
    uint32_t bc[4];
    uint32_t tied[kWave];
    uint32_t ntied;
    uint32_t woff[16];  // per-wave list entries
    uint32_t wsel[16];  // per-wave selected entries
    uint32_t lkey[kPairListCap];
    uint32_t lgid[kPairListCap];
};

// The k selected candidates: key > thr_gt, or key == tie_key and gid <= gid_cut.
struct PairCut {
    uint32_t thr_gt, tie_key, gid_cut;
};

__device__ __forceinline__ bool pair_selected(uint32_t key, uint32_t gid, const PairCut& c) {
    return key != 0u && (key > c.thr_gt || (key == c.tie_key && gid <= c.gid_cut));
}

// Emission in candidate order from a visitor that hands out this lane's
// candidates register by register in a uniform loop (so ballots see the whole
// wave); -1 after the selected ones.
template <typename Visit>
__device__ __forceinline__ void pair_emit_visit(PairSmem& sm, Visit visit, const PairCut& c, int world,
                                                int k, int32_t* __restrict__ o_row) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    uint32_t cnt = 0;
    visit([&](uint32_t key, uint32_t gid) __attribute__((always_inline)) {
        cnt += (uint32_t)__popcll(__ballot(pair_selected(key, gid, c)));
    });
    if (lane == 0) sm.red[wave][3] = cnt;
    lds_barrier();
    uint32_t base = 0, total = 0;
    for (int w = 0; w < world; ++w) {
        const uint32_t n = sm.red[w][3];
        base += w < wave ? n : 0u;
        total += n;
    }
    visit([&](uint32_t key, uint32_t gid) __attribute__((always_inline)) {
        const bool sel = pair_selected(key, gid, c);
        const uint64_t m = __ballot(sel);
        const uint32_t pos = base + mbcnt64(m);
        if (sel && pos < (uint32_t)k) o_row[pos] = (int32_t)gid;
        base += (uint32_t)__popcll(m);
    });
    for (int p = (int)(total < (uint32_t)k ? total : (uint32_t)k) + (int)threadIdx.x; p < k;
         p += kWave * world)
        o_row[p] = -1;
}

// Emission from the LDS list in candidate order: wave w's segment holds its
// rank's listed candidates; -1 after the selected ones (not reached when the
// counts are consistent).
__device__ __forceinline__ void pair_emit_list(PairSmem& sm, const PairCut& c, int world, int k,
                                               int32_t* __restrict__ o_row) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    uint32_t off = 0;
    for (int w = 0; w < wave; ++w) off += sm.woff[w];
    const uint32_t n = sm.woff[wave];
    uint32_t cnt = 0;
#pragma unroll 1
    for (uint32_t b = 0; b < n; b += kWave) {
        const bool in = b + (uint32_t)lane < n && off + b + (uint32_t)lane < (uint32_t)kPairListCap;
        const uint32_t i = in ? off + b + (uint32_t)lane : 0u;
        const bool sel = in && pair_selected(sm.lkey[i], sm.lgid[i], c);
        cnt += (uint32_t)__popcll(__ballot(sel));
    }
    if (lane == 0) sm.wsel[wave] = cnt;
    lds_barrier();
    uint32_t base = 0, total = 0;
    for (int w = 0; w < world; ++w) {
        const uint32_t s = sm.wsel[w];
        base += w < wave ? s : 0u;
        total += s;
    }
#pragma unroll 1
    for (uint32_t b = 0; b < n; b += kWave) {
        const bool in = b + (uint32_t)lane < n && off + b + (uint32_t)lane < (uint32_t)kPairListCap;
        const uint32_t i = in ? off + b + (uint32_t)lane : 0u;
        const uint32_t gid = sm.lgid[i];
        const bool sel = in && pair_selected(sm.lkey[i], gid, c);
        const uint64_t m = __ballot(sel);
        const uint32_t pos = base + mbcnt64(m);
        if (sel && pos < (uint32_t)k) o_row[pos] = (int32_t)gid;
        base += (uint32_t)__popcll(m);
    }
    for (int p = (int)(total < (uint32_t)k ? total : (uint32_t)k) + (int)threadIdx.x; p < k;
         p += kWave * world)
        o_row[p] = -1;
}

template <int QK>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8))) void merge_pairs_wave_kernel(
    const int32_t* __restrict__ pairs, Layout lay, int32_t world, int64_t rows, int32_t kc,
    int32_t k, int32_t* __restrict__ out_ids) {
    __shared__ PairSmem sm;
    typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // the rank (uniform)
    const int nthreads = kWave * world;

    for (int q = threadIdx.x; q < kLevelCopies * kLevelStride; q += nthreads) (&sm.hist[0][0])[q] = 0u;
    if (threadIdx.x == 0) sm.ntied = 0u;

    const int64_t row = blockIdx.x;
    const i32x2* src = reinterpret_cast<const i32x2*>(pairs) + lay.at(wave, row) * kc;
    // Pairs are loaded a batch of 8 registers at a time, all of a batch in
    // flight together (left to itself the compiler waits after every load).
    uint32_t key[QK];
    {
        constexpr int QL = QK < 8 ? QK : 8;
#pragma unroll
        for (int qb = 0; qb < QK; qb += QL) {
            i32x2 pr[QL];
#pragma unroll
            for (int b = 0; b < QL; ++b) {
                const int j = (qb + b) * kWave + lane;
                pr[b] = src[j < kc ? j : 0];  // QK may exceed ceil(kc / 64)
            }
#pragma unroll
            for (int b = 0; b < QL; ++b) {
                const int j = (qb + b) * kWave + lane;
                const uint32_t u = (uint32_t)pr[b][0];
                const bool valid = j < kc && pr[b][1] >= 0 && !__builtin_isnan(__uint_as_float(u));
                key[qb + b] = valid ? key32_of_bits(u) : 0u;
            }
        }
    }
    auto fresh = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < QK; ++q) asm volatile("" : "+v"(key[q]));
    };

    // Valid count and key range (every valid key is >= key32(-inf) > 0).
    // The minimum is taken over key - 1, which sends empty slots (0) to the
    // top of the unsigned range.
    // Per-lane figures, the wave's, then lane w < world combines wave w's.
    uint32_t nv = 0, mn = 0xFFFFFFFFu, mx = 0u;
    fresh();
#pragma unroll
    for (int q = 0; q < QK; ++q) {
        nv += key[q] != 0u ? 1u : 0u;
        const uint32_t km1 = key[q] - 1u;
        mn = km1 < mn ? km1 : mn;
        mx = key[q] > mx ? key[q] : mx;
    }
    nv = wave_sum32(nv);
    mn = wave_min32(mn);
    mx = wave_max32(mx);
    if (lane == 0) {
        sm.red[wave][0] = nv;
        sm.red[wave][1] = mn;
        sm.red[wave][2] = mx;
    }
    lds_barrier();
    {
        const bool wl = lane < world;
        nv = wave_sum32(wl ? sm.red[lane][0] : 0u);
        mn = wave_min32(wl ? sm.red[lane][1] : 0xFFFFFFFFu);
        mx = wave_max32(wl ? sm.red[lane][2] : 0u);
    }
    mn += 1u;  // the smallest valid key (used only when there are more than k)
    int32_t* o_row = out_ids + row * (int64_t)k;
    // The row re-read from memory (cached) for the rare paths, so that no
    // candidate registers are held across their barriers.
    auto visit_mem = [&](auto f) __attribute__((always_inline)) {
        constexpr int QC = QK < 8 ? QK : 8;  // registers per step
#pragma unroll 1
        for (int q0 = 0; q0 < QK; q0 += QC) {
#pragma unroll
            for (int q = 0; q < QC; ++q) {
                const int j = (q0 + q) * kWave + lane;
                const i32x2 v = src[j < kc ? j : 0];
                const uint32_t u = (uint32_t)v[0];
                const bool valid = j < kc && v[1] >= 0 && !f32_bits_is_nan(u);
                f(valid ? key32_of_bits(u) : 0u, (uint32_t)v[1]);
            }
        }
    };

    if (nv <= (uint32_t)k) {  // every valid candidate is selected
        pair_emit_visit(sm, visit_mem, PairCut{0u, 0u, 0u}, world, k, o_row);
        return;
    }

    // First level on the registers.
    const uint32_t span0 = mx - mn;
    const int bl = span0 ? 32 - __clz((int)span0) : 0;
    const uint32_t sh0 = bl > 8 ? (uint32_t)(bl - 8) : 0u;
    int need = k;
    fresh();
#pragma unroll
    for (int q = 0; q < QK; ++q) level_hist_add(sm, key[q], mn, span0, sh0);
    uint32_t bin, cb;
    const bool ok = level_hist_find(sm, need, bin, cb);
    const uint32_t blo = mn + (bin << sh0);
    const uint32_t nlist = (uint32_t)(k - need) + cb;  // keys >= blo

    if (ok && nlist <= (uint32_t)kPairListCap) {
        // Compact the keys >= blo into the list, in candidate order.
        uint32_t c = 0;
        fresh();
#pragma unroll
        for (int q = 0; q < QK; ++q) c += key[q] >= blo ? 1u : 0u;
        c = wave_sum32(c);
        if (lane == 0) sm.woff[wave] = c;
        lds_barrier();
        const uint32_t wincl = wave_incl_scan32(lane < world ? sm.woff[lane] : 0u);
        uint32_t off = wave == 0 ? 0u : (uint32_t)__builtin_amdgcn_readlane((int)wincl, wave - 1);
        // The listed entries' gids are read back from memory (mostly cached:
        // the row was just read), a batch of registers' loads in flight
        // together rather than one round trip per register.
        constexpr int QB = QK < 8 ? QK : 8;
        fresh();
#pragma unroll
        for (int qb = 0; qb < QK; qb += QB) {
            uint32_t g[QB];
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const int q = qb + b;
                g[b] = key[q] >= blo ? (uint32_t)src[q * kWave + lane][1] : 0u;
            }
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const int q = qb + b;
                const bool in = key[q] >= blo;
                const uint64_t m = __ballot(in);
                const uint32_t p = off + mbcnt64(m);
                if (in && p < (uint32_t)kPairListCap) {
                    sm.lkey[p] = key[q];
                    sm.lgid[p] = g[b];
                }
                off += (uint32_t)__popcll(m);
            }
        }
        lds_barrier();

        auto visit_list = [&](auto f) __attribute__((always_inline)) {
#pragma unroll 1
            for (int i = threadIdx.x; i < (int)nlist; i += nthreads) f(sm.lkey[i], sm.lgid[i]);
        };
        PairCut cut{blo - 1u, 0u, 0u};
        if ((int)cb != need) {
            bool ties;
            uint32_t ntie;
            if (sh0 == 0) {
                ties = true;
                cut.thr_gt = blo;
                cut.tie_key = blo;
                ntie = cb;
            } else {
                const uint32_t top = mx - blo, width1 = (1u << sh0) - 1u;
                radix_levels(sm, visit_list, need, blo, width1 < top ? width1 : top,
                            sh0 > 8 ? sh0 - 8 : 0u, mx, cut.thr_gt, ties, cut.tie_key, ntie);
            }
            if (ties) cut.gid_cut = tie_cut(sm, visit_list, cut.tie_key, ntie, need);
        }
        pair_emit_list(sm, cut, world, k, o_row);
    } else {
        // Rare (heavy ties, or a boundary bin too full for the list):
        // levels from the full window over the row re-read from memory.
        need = k;
        PairCut cut{0u, 0u, 0u};
        bool ties;
        uint32_t ntie;
        radix_levels(sm, visit_mem, need, mn, span0, sh0, mx, cut.thr_gt, ties, cut.tie_key, ntie);
        if (ties) cut.gid_cut = tie_cut(sm, visit_mem, cut.tie_key, ntie, need);
        pair_emit_visit(sm, visit_mem, cut, world, k, o_row);
    }
}

template <int KPT>
__global__ __launch_bounds__(kSelBlock) void merge_pairs_kernel(
    const int32_t* __restrict__ pairs, Layout lay, int32_t world, int64_t rows, int32_t kc,
    int32_t k, int32_t* __restrict__ out_ids) {
    __shared__ SelectSmem sm;
    typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int32_t total = world * kc;

    for (int q = t; q < kHistCopies * kHistStride; q += kSelBlock) (&sm.hist[0][0])[q] = 0u;

    uint64_t key[KPT];
    {
        FlatWalk w(kc, t);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            key[i] = 0ull;
            if (i * kSelBlock + t < total) {
                const i32x2 pr =
                    reinterpret_cast<const i32x2*>(pairs)[lay.at(w.r, row) * kc + w.j];
                const uint32_t u = (uint32_t)pr[0];
                if (pr[1] >= 0 && !f32_bits_is_nan(u)) key[i] = composite(key32_of_bits(u), (uint32_t)pr[1]);
            }
            w.next();
        }
    }
    uint32_t nz = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) nz += key[i] != 0ull;
    __syncthreads();
    const uint32_t nvalid = block_sum(nz, sm);

    uint64_t T = 1ull;
    if (nvalid > (uint32_t)k) T = block_radix_kth<KPT>(key, k, sm);
    block_emit<KPT>(key, T, k, out_ids + row * (int64_t)k, sm);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

int pick_kpt(int64_t total) {
    const int64_t need = (total + kSelBlock - 1) / kSelBlock;
    static const int choices[] = {1, 2, 4, 6, 8, 12, 16, 24, 32, 48, 64};
    for (int c : choices)
        if (c >= need) return c;
    return -1;
}

template <template <int> class L, typename... A>
int dispatch_kpt(int kpt, A... args) {
    switch (kpt) {
        case 1: L<1>::run(args...); break;
        case 2: L<2>::run(args...); break;
        case 4: L<4>::run(args...); break;
        case 6: L<6>::run(args...); break;
        case 8: L<8>::run(args...); break;
        case 12: L<12>::run(args...); break;
        case 16: L<16>::run(args...); break;
        case 24: L<24>::run(args...); break;
        case 32: L<32>::run(args...); break;
        case 48: L<48>::run(args...); break;
        case 64: L<64>::run(args...); break;
        default: return RTS_EUNSUPPORTED;
    }
    return RTS_OK;
}

template <int KPT>
struct PackedLaunch {
    static void run(const int32_t* g, Layout lay, int32_t world, int64_t rows, int32_t n, int32_t k,
                    int32_t* ids, int32_t* sat, RowsArgs ra, hipStream_t s) {
        if (ra.rows_out)
            hipLaunchKernelGGL((merge_packed_kernel<KPT, true>), dim3((unsigned)rows), dim3(kSelBlock), 0,
                               s, g, lay, world, rows, n, k, ids, sat, ra);
        else
            hipLaunchKernelGGL((merge_packed_kernel<KPT, false>), dim3((unsigned)rows), dim3(kSelBlock), 0,
                               s, g, lay, world, rows, n, k, ids, sat, ra);
    }
};

// Workgroups of the strided rescue: two per compute unit.
constexpr int64_t kRescueGrid = 512;

template <int KPT>
struct RescueLaunch {
    static void run(const int32_t* g, const int32_t* recv, int32_t world, int64_t rows, int32_t n,
                    int32_t k, const int32_t* sat, int32_t* ids, RowsArgs ra, hipStream_t s) {
        if (ra.rows_out)
            go<true>(g, recv, world, rows, n, k, sat, ids, ra, s);
        else
            go<false>(g, recv, world, rows, n, k, sat, ids, ra, s);
    }
    template <bool ROWS>
    static void go(const int32_t* g, const int32_t* recv, int32_t world, int64_t rows, int32_t n,
                   int32_t k, const int32_t* sat, int32_t* ids, RowsArgs ra, hipStream_t s) {
        if constexpr (KPT >= 48) {
            hipLaunchKernelGGL((merge_rescue_row_kernel<KPT, ROWS>), dim3((unsigned)rows), dim3(kSelBlock),
                               0, s, g, recv, world, rows, n, k, sat, ids, ra);
        } else {
            const unsigned grid = (unsigned)(rows < kRescueGrid ? rows : kRescueGrid);
            hipLaunchKernelGGL((merge_rescue_kernel<KPT, ROWS>), dim3(grid), dim3(kSelBlock), 0, s, g,
                               recv, world, rows, n, k, sat, ids, ra);
        }
    }
};

template <int KPT>
struct PairsLaunch {
    static void run(const int32_t* p, Layout lay, int32_t world, int64_t rows, int32_t kc, int32_t k,
                    int32_t* ids, hipStream_t s) {
        hipLaunchKernelGGL((merge_pairs_kernel<KPT>), dim3((unsigned)rows), dim3(kSelBlock), 0, s, p,
                           lay, world, rows, kc, k, ids);
    }
};

template <int QN, int W>
void launch_packed_wave(const int32_t* g, Layout lay, int64_t rows, int32_t n, int32_t k,
                        int32_t* ids, int32_t* sat, const RowsArgs& ra, hipStream_t s) {
    if constexpr (QN * W <= 64) {
        if (ra.rows_out)
            hipLaunchKernelGGL((merge_packed_wave_kernel<QN, W, true>), dim3((unsigned)rows), dim3(kWave),
                               0, s, g, lay, W, rows, n, k, ids, sat, ra);
        else
            hipLaunchKernelGGL((merge_packed_wave_kernel<QN, W, false>), dim3((unsigned)rows), dim3(kWave),
                               0, s, g, lay, W, rows, n, k, ids, sat, ra);
    }
}

template <int QN>
bool packed_wave_w(int world, const int32_t* g, Layout lay, int64_t rows, int32_t n, int32_t k,
                   int32_t* ids, int32_t* sat, const RowsArgs& ra, hipStream_t s) {
    if (QN * world > 64) return false;
    switch (world) {
        case 1: launch_packed_wave<QN, 1>(g, lay, rows, n, k, ids, sat, ra, s); return true;
        case 2: launch_packed_wave<QN, 2>(g, lay, rows, n, k, ids, sat, ra, s); return true;
        case 4: launch_packed_wave<QN, 4>(g, lay, rows, n, k, ids, sat, ra, s); return true;
        case 8: launch_packed_wave<QN, 8>(g, lay, rows, n, k, ids, sat, ra, s); return true;
        case 16: launch_packed_wave<QN, 16>(g, lay, rows, n, k, ids, sat, ra, s); return true;
        default: return false;
    }
}

// One wave per row for world in {1, 2, 4, 8, 16} and qn = ceil(n/64) slot
// registers per rank, with qn * world <= 64; false: use the block kernel.
bool dispatch_packed_wave(int qn, int world, const int32_t* g, Layout lay, int64_t rows, int32_t n,
                          int32_t k, int32_t* ids, int32_t* sat, const RowsArgs& ra, hipStream_t s) {
    switch (qn) {
        case 1: return packed_wave_w<1>(world, g, lay, rows, n, k, ids, sat, ra, s);
        case 2: return packed_wave_w<2>(world, g, lay, rows, n, k, ids, sat, ra, s);
        case 3: return packed_wave_w<3>(world, g, lay, rows, n, k, ids, sat, ra, s);
        case 4: return packed_wave_w<4>(world, g, lay, rows, n, k, ids, sat, ra, s);
        case 5: return packed_wave_w<5>(world, g, lay, rows, n, k, ids, sat, ra, s);
        case 6: return packed_wave_w<6>(world, g, lay, rows, n, k, ids, sat, ra, s);
        case 7: return packed_wave_w<7>(world, g, lay, rows, n, k, ids, sat, ra, s);
        case 8: return packed_wave_w<8>(world, g, lay, rows, n, k, ids, sat, ra, s);
        default: return false;
    }
}

}  // namespace

int launch_pack_candidates(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                           const int32_t* local_idx, int32_t n, int64_t ld_idx,
                           const int32_t* row_ends, int32_t* packed, hipStream_t s) {
    const int64_t total = rows * (int64_t)n;
    if (total == 0) return RTS_OK;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(pack_candidates_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, cols, ld,
                       local_idx, n, ld_idx, row_ends, packed);
    return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
}

int launch_pack_pairs(const float* x, int64_t rows, int64_t cols, int64_t ld, const int32_t* local_idx,
                      int32_t kc, int64_t ld_idx, const int32_t* row_ends, int32_t rank, int32_t world,
                      int32_t* pairs, hipStream_t s) {
    const int64_t total = rows * (int64_t)kc;
    if (total == 0) return RTS_OK;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(pack_pairs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, cols, ld,
                       local_idx, kc, ld_idx, row_ends, rank, world, pairs);
    return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
}

int launch_merge_packed(const int32_t* gathered, bool row_major, int32_t world, int64_t rows,
                        int32_t n, int32_t k, int32_t* out_ids, int32_t* sat_word,
                        const RowsArgs* rows_args, hipStream_t s) {
    if (rows == 0) return RTS_OK;
    const Layout lay = row_major ? Layout{1, world} : Layout{rows, 1};
    const RowsArgs ra = rows_args ? *rows_args : RowsArgs{};
    if (dispatch_packed_wave((n + kWave - 1) / kWave, world, gathered, lay, rows, n, k, out_ids,
                             sat_word, ra, s))
        return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
    const int kpt = pick_kpt((int64_t)world * n);
    const int rc = dispatch_kpt<PackedLaunch>(kpt, gathered, lay, world, rows, n, k, out_ids,
                                              sat_word, ra, s);
    if (rc != RTS_OK) return rc;
    return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
}

int rescue_candidates(int32_t world, int32_t n, int32_t k) {
    const int32_t slots = (k - 1) / n;
    return world * n + (slots < world ? slots : world) * k;
}

int launch_rescue_push(const int32_t* local_packed, int32_t rank, int32_t world, int64_t rows,
                       int32_t n, int32_t k, const int32_t* sat_word, int32_t* recv, hipStream_t s) {
    if (rows == 0 || (k - 1) / n == 0) return RTS_OK;
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL(rescue_push_kernel, dim3((unsigned)blocks), dim3(256), 0, s, local_packed, rank,
                       world, rows, n, k, sat_word, recv);
    return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
}

int launch_merge_rescue(const int32_t* gathered, const int32_t* recv, int32_t world, int64_t rows,
                        int32_t n, int32_t k, const int32_t* sat_word, int32_t* out_ids,
                        const RowsArgs* rows_args, hipStream_t s) {
    if (rows == 0 || (k - 1) / n == 0) return RTS_OK;
    const int kpt = pick_kpt(rescue_candidates(world, n, k));
    const RowsArgs ra = rows_args ? *rows_args : RowsArgs{};
    const int rc = dispatch_kpt<RescueLaunch>(kpt, gathered, recv, world, rows, n, k, sat_word,
                                              out_ids, ra, s);
    if (rc != RTS_OK) return rc;
    return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
}

int launch_emit_rows(const int32_t* ids, int64_t rows, int32_t k, int32_t world, int32_t dcp_rank,
                     const int32_t* req_id, const int32_t* block_table, int64_t table_rows,
                     int32_t table_cols, int64_t ld_table, int32_t block_size, int64_t stride_rows,
                     int32_t* rows_out, int32_t out_cols, int32_t* valid_out, hipStream_t s) {
    if (rows == 0) return RTS_OK;
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL(emit_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ids, rows, k, world,
                       dcp_rank, req_id, block_table, table_rows, table_cols, ld_table, block_size,
                       stride_rows, rows_out, out_cols, valid_out);
    return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
}

int launch_merge_pairs(const int32_t* pairs, bool row_major, int32_t world, int64_t rows, int32_t kc,
                       int32_t k, int32_t* out_ids, hipStream_t s) {
    if (rows == 0) return RTS_OK;
    const Layout lay = row_major ? Layout{1, world} : Layout{rows, 1};
    // One wave per rank when a rank's candidates fit in 32 registers per lane.
    const int qk = (kc + kWave - 1) / kWave;
    if (qk <= 32 && world <= 16) {
        const dim3 g((unsigned)rows), b((unsigned)(kWave * world));
        if (qk <= 4)
            hipLaunchKernelGGL(merge_pairs_wave_kernel<4>, g, b, 0, s, pairs, lay, world, rows, kc, k,
                               out_ids);
        else if (qk <= 8)
            hipLaunchKernelGGL(merge_pairs_wave_kernel<8>, g, b, 0, s, pairs, lay, world, rows, kc, k,
                               out_ids);
        else if (qk <= 16)
            hipLaunchKernelGGL(merge_pairs_wave_kernel<16>, g, b, 0, s, pairs, lay, world, rows, kc, k,
                               out_ids);
        else
            hipLaunchKernelGGL(merge_pairs_wave_kernel<32>, g, b, 0, s, pairs, lay, world, rows, kc, k,
                               out_ids);
        return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
    }
    const int kpt = pick_kpt((int64_t)world * kc);
    const int rc = dispatch_kpt<PairsLaunch>(kpt, pairs, lay, world, rows, kc, k, out_ids, s);
    if (rc != RTS_OK) return rc;
    return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
}

}  // namespace rts
