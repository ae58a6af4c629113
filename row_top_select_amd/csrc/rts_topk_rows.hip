// Per-row exact top-K over fp32 / bf16 logits with causal row ends, for gfx950.
//
// What is computed (vLLM PR 57206 "Use DeepSelect for eligible sparse-indexer
// prefill chunks", Purpose and Test Plan; order of the kernels page of
// vllm.models.kimi_k3.nvidia.ops.dcp_topk_merge, module docstring and
// DCPTopkSelectKernel): for row i with e = clamp(row_end_i, 0, cols), the ids
// of the k best non-NaN entries of x[i, 0:e] under (score desc, -0 below +0,
// id asc), in that order, then -1.
//
// How (one HBM pass, no workgroup barrier while streaming):
//   * A wave owns a contiguous piece of a row and reads it in ascending column
//     order, 256 elements per chunk (16 B per lane for fp32, 8 B for bf16),
//     a group of chunks in flight while the previous group is filtered.
//   * It keeps a threshold tau: the score key of the k-th best composite seen
//     so far.  A later element can only enter the top-k if its key is > tau (a
//     tie has a larger id and loses), so the filter is one float compare per
//     element against the float whose key is tau + 1; NaN fails every compare.
//   * Survivors are appended to a wave-private LDS stage (ballot + lane prefix
//     count).  When the stage cannot take another 64 survivors, a wave-level radix
//     select finds the exact k-th composite among the staged entries and keeps
//     only the top k.  Its digit window is relative to [min, max] of the keys
//     still in play, so concentrated score distributions do not pile into one
//     bin.
//   * At the end the surviving k entries are bitonic-sorted in registers.
//     Waves of one workgroup share tau through LDS (another wave's tau admits
//     ties, so it is used non-strictly) and merge their sorted lists pairwise
//     with the elementwise max of a descending and an ascending list (which is
//     bitonic and holds the top half) plus a bitonic merge.  With several
//     workgroups per row each writes its sorted list to the workspace and a
//     second kernel merges them the same way.
// The result is exact for any distribution; adversarial orders only cost more
// compactions, never more HBM traffic.
#include "rts_device.hpp"
#include "rts_internal.h"
#include "../../include/row_top_select.h"

namespace rts {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
struct RowTraits;
template <>
struct RowTraits<false> {
    using elem = float;
    using vec = u32x4;  // 4 elements
};
template <>
struct RowTraits<true> {
    using elem = uint16_t;
    using vec = u32x2;  // 4 elements
};

constexpr int kVec = 4;             // elements per lane per chunk
constexpr int kChunk = kWave * kVec;  // elements per chunk
constexpr int kGroup = 4;           // chunks per group (one group in flight)

template <bool BF16>
__device__ __forceinline__ uint32_t load_bits(const typename RowTraits<BF16>::elem* p) {
    if constexpr (BF16) {
        return (uint32_t)(*p) << 16;
    } else {
        return __float_as_uint(*p);
    }
}

template <bool BF16>
__device__ __forceinline__ void unpack(typename RowTraits<BF16>::vec v, uint32_t (&bits)[kVec]) {
    if constexpr (BF16) {
        bits[0] = v[0] << 16;
        bits[1] = v[0] & 0xFFFF0000u;
        bits[2] = v[1] << 16;
        bits[3] = v[1] & 0xFFFF0000u;
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) bits[q] = v[q];
    }
}

// One level of the wave radix select: bins of [mn, mx] of the composites in
// [lo_edge, hi_edge] (all nonzero ones on the first level).  Returns true when
// done, with *T set; otherwise narrows [lo_edge, hi_edge] and need.
template <int NV, bool FIRST>
__device__ __forceinline__ bool wave_radix_level(const uint64_t (&v)[NV], uint64_t& lo_edge,
                                                 uint64_t& hi_edge, int& need, uint64_t* T,
                                                 uint32_t* hist, bool force_end) {
    const int lane = lane_id();
    uint64_t mn = ~0ull, mx = 0;
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const bool in = FIRST ? v[r] != 0ull : (v[r] >= lo_edge && v[r] <= hi_edge);
        mn = in ? umin64(mn, v[r]) : mn;
        mx = in ? umax64(mx, v[r]) : mx;
    }
    mn = wave_min64(mn);
    mx = wave_max64(mx);
    if (mn == mx) {
        *T = mn;
        return true;
    }
    const uint64_t d = mx - mn;
    const int bl = 64 - __clzll((long long)d);
    const int s = bl > 8 ? bl - 8 : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[lane * 4 + j] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const bool in = FIRST ? v[r] != 0ull : (v[r] >= lo_edge && v[r] <= hi_edge);
        if (in)
            __hip_atomic_fetch_add(&hist[(uint32_t)((v[r] - mn) >> s)], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
    wave_lds_sync();
    // Lane l owns bins 255-4l .. 252-4l, scanned from the top.
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = hist[255 - 4 * lane - j];
    const uint32_t tot = c[0] + c[1] + c[2] + c[3];
    uint32_t run = wave_incl_scan32(tot) - tot;
    int fj = -1;
    uint32_t above = 0, cb = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (fj < 0 && run < (uint32_t)need && run + c[j] >= (uint32_t)need) {
            fj = j;
            above = run;
            cb = c[j];
        }
        run += c[j];
    }
    wave_lds_sync();
    const uint64_t fm = __ballot(fj >= 0);
    if (fm == 0ull || force_end) {  // only if the count invariant were broken
        *T = mn;
        return true;
    }
    const int fl = __ffsll((long long)fm) - 1;
    const int bj = __builtin_amdgcn_readlane(fj, fl);
    above = __builtin_amdgcn_readlane(above, fl);
    cb = __builtin_amdgcn_readlane(cb, fl);
    const uint32_t bin = 255u - 4u * (uint32_t)fl - (uint32_t)bj;
    need -= (int)above;
    const uint64_t blo = mn + ((uint64_t)bin << s);
    if ((int)cb == need) {
        *T = blo;
        return true;
    }
    lo_edge = blo;
    // The top bin ends at mx (blo + 2^s - 1 could wrap past 2^64 there).
    hi_edge = bin == (uint32_t)(d >> s) ? mx : blo + ((1ull << s) - 1ull);
    return false;
}

// Exact k-th largest composite among v[] (0 = empty); requires k <= number of
// nonzero entries.  Returns T such that exactly k nonzero entries are >= T
// when composites are distinct.  hist: 256 wave-private LDS counters.  Each
// level narrows the range by at least 2^7, so 10 levels always finish; the
// cap only bounds the loop if the count invariant were ever broken.
template <int NV>
__device__ __forceinline__ uint64_t wave_radix_kth(const uint64_t (&v)[NV], int k, uint32_t* hist) {
    uint64_t lo_edge = 1, hi_edge = ~0ull, T = 0;
    int need = k;
    if (wave_radix_level<NV, true>(v, lo_edge, hi_edge, need, &T, hist, false)) return T;
    for (int level = 1;; ++level)
        if (wave_radix_level<NV, false>(v, lo_edge, hi_edge, need, &T, hist, level >= 12)) return T;
}

template <int E, int ES, bool BF16, int P>
__global__ __launch_bounds__(kWave* P) __attribute__((amdgpu_waves_per_eu(E <= 8 ? 4 : 2)))
void topk_rows_stream_kernel(
    const void* __restrict__ xv, int64_t cols, int64_t ld, const int32_t* __restrict__ row_ends,
    int32_t k, int32_t* __restrict__ out, int64_t ld_out, uint64_t* __restrict__ part,
    int32_t groups) {
    using T = typename RowTraits<BF16>::elem;
    using V = typename RowTraits<BF16>::vec;
    constexpr int LP = kWave * E;
    constexpr int SCAP = kWave * ES;            // room for new survivors
    constexpr int SBUF = SCAP > LP ? SCAP : LP;  // also carries the selected list into L
    static_assert(SCAP >= kChunk, "the stage must take a whole chunk");

    __shared__ uint64_t stage_all[P][SBUF];
    __shared__ uint32_t hist_all[P][256];
    __shared__ uint32_t thr_shared;

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row = blockIdx.x / groups;
    const int g = (int)(blockIdx.x - row * groups);
    uint64_t* stage = stage_all[wave];
    uint32_t* hist = hist_all[wave];

    int64_t e = row_ends ? (int64_t)row_ends[row] : cols;
    e = e < 0 ? 0 : (e > cols ? cols : e);

    if constexpr (P > 1) {
        if (threadIdx.x == 0) thr_shared = 0u;
        __syncthreads();
    }

    // This wave's piece [a, b) of the row.
    const int64_t pieces = (int64_t)groups * P;
    const int64_t piece = (int64_t)g * P + wave;
    int64_t per = (e + pieces - 1) / pieces;
    per = (per + kChunk - 1) / kChunk * kChunk;
    const int64_t a = piece * per < e ? piece * per : e;
    const int64_t b = a + per < e ? a + per : e;

    const T* rowp = reinterpret_cast<const T*>(xv) + row * ld;

    int cnt = 0;                     // staged entries (wave-uniform)
    int nl = 0;                      // entries in the register list L (wave-uniform)
    uint32_t thr_own = 0x007FFFFFu;  // key of -inf: every non-NaN value passes
    float f = float_of_key32(thr_own);
    // The current top list: up to k composites, E per lane, unsorted.
    uint64_t L[E];
#pragma unroll
    for (int r = 0; r < E; ++r) L[r] = 0;

    auto refresh = [&]() {
        uint32_t t = thr_own;
        if constexpr (P > 1) {
            const uint32_t s =
                __hip_atomic_load(&thr_shared, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            t = s > t ? s : t;
        }
        f = float_of_key32(t);
    };

    // Staged entries hold the raw score bits in the high word (the key transform
    // is applied once per entry when the stage is compacted).
    auto append = [&](uint64_t m, uint32_t bits, uint32_t col) {
        if ((m >> lane) & 1ull) stage[cnt + (int)mbcnt64(m)] = composite(bits, col);
        cnt += (int)__popcll(m);
    };

    // Elements one per lane (head and tail of the piece); needs 64 free slots.
    auto consider = [&](uint32_t bits, uint32_t col, bool valid) {
        const uint64_t m = __ballot(valid && __uint_as_float(bits) >= f);
        if (m) append(m, bits, col);
    };

    // Geometry: head [a, a1) up to the first aligned vector, body of whole
    // chunks, tail [t0, b).
    int64_t a1 = a, nch = 0, t0 = a;
    if (a < b) {
        constexpr int64_t vbytes = sizeof(V);
        const uintptr_t base = reinterpret_cast<uintptr_t>(rowp);
        const int64_t off = (int64_t)((base % vbytes) / sizeof(T));
        a1 = a + (kVec - (off + a) % kVec) % kVec;
        a1 = a1 < b ? a1 : b;
        nch = (b - a1) / kChunk;
        t0 = a1 + nch * kChunk;
    }
    const V* bp = reinterpret_cast<const V*>(rowp + a1) + lane;
    const int64_t ngroups = (nch + kGroup - 1) / kGroup;

    // Issue priority.  The SIMD issues the oldest ready wave first, so waves
    // that started later fall behind once compactions compete for issue slots.
    // A streaming wave takes priority 3..1 as it advances through its piece, so
    // the ones behind win; a wave that compacts drops to 0, so waves about to
    // issue loads keep the memory pipe full while it works.
    auto set_stream_prio = [](int64_t g_done, int64_t g_total) {
        const int64_t q = g_total > 0 ? (g_done * 3) / g_total : 0;
        if (q == 0) __builtin_amdgcn_s_setprio(3);
        else if (q == 1) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(1);
    };
    __builtin_amdgcn_s_setprio(3);

    // Head: fewer than kVec elements, the stage is empty.
    if (a1 > a) {
        const int64_t col = a + lane;
        const bool valid = col < a1;
        consider(valid ? load_bits<BF16>(rowp + col) : 0u, (uint32_t)col, valid);
    }

    V A[kGroup], B[kGroup];
    auto load_group = [&](V(&dst)[kGroup], int64_t gi) {
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            int64_t c = gi * kGroup + u;
            c = c < nch ? c : nch - 1;
            dst[u] = __builtin_nontemporal_load(bp + c * kWave);
        }
    };
    int64_t gi = 0;
    if (ngroups > 0) {
        load_group(A, 0);
        load_group(B, ngroups > 1 ? 1 : 0);
    }
    int ustart = 0;  // first chunk of the group still to process
    // A chunk interrupted by a full stage: its masks (taken against the older,
    // lower threshold: a superset) and values; finished right after the
    // compaction.  Re-filtering it strictly could drop a tie whose id is smaller
    // than that of an entry of the same chunk already in the list.
    bool pend = false;
    int pend_c = 0;
    uint32_t pbits[kVec] = {0, 0, 0, 0};
    uint64_t pm[kVec] = {0, 0, 0, 0};
    uint32_t pcol0 = 0;
    int64_t tpos = t0;
    int phase = ngroups > 0 ? 0 : 1;  // 0 body, 1 tail, 2 end

    // One chunk: returns false (after saving the rest as pending) if the stage
    // filled up inside it.
    auto chunk = [&](V vv, uint32_t col0, int u) -> bool {
        uint32_t bits[kVec];
        unpack<BF16>(vv, bits);
        uint64_t m[kVec];
#pragma unroll
        for (int c = 0; c < kVec; ++c) m[c] = __ballot(__uint_as_float(bits[c]) >= f);
        if ((m[0] | m[1] | m[2] | m[3]) == 0ull) return true;
#pragma unroll
        for (int c = 0; c < kVec; ++c) {
            if (m[c]) {
                if (cnt + kWave > SCAP) {
                    pend = true;
                    pend_c = c;
                    pcol0 = col0;
#pragma unroll
                    for (int q = 0; q < kVec; ++q) {
                        pbits[q] = bits[q];
                        pm[q] = m[q];
                    }
                    ustart = u + 1;
                    return false;
                }
                append(m[c], bits[c], col0 + (uint32_t)c);
            }
        }
        return true;
    };

    for (;;) {
        bool need = false;
        if (phase == 0) {
            while (true) {
                if (ustart == 0 && (gi + 1) * kGroup <= nch) {
#pragma unroll
                    for (int u = 0; u < kGroup; ++u) {
                        if (!need)
                            need = !chunk(A[u], (uint32_t)(a1 + (gi * kGroup + u) * kChunk + lane * kVec), u);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < kGroup; ++u) {
                        if (!need && u >= ustart && gi * kGroup + u < nch)
                            need = !chunk(A[u], (uint32_t)(a1 + (gi * kGroup + u) * kChunk + lane * kVec), u);
                    }
                }
                if (need) break;
                ustart = 0;
                ++gi;
                if (gi >= ngroups) {
                    phase = 1;
                    break;
                }
#pragma unroll
                for (int u = 0; u < kGroup; ++u) A[u] = B[u];
                load_group(B, gi + 1 < ngroups ? gi + 1 : gi);
                if constexpr (P > 1) refresh();
                if ((gi & 7) == 0) set_stream_prio(gi, ngroups);
            }
        }
        if (!need && phase == 1) {
            while (tpos < b) {
                if (cnt + kWave > SCAP) {
                    need = true;
                    break;
                }
                const int64_t col = tpos + lane;
                const bool valid = col < b;
                consider(valid ? load_bits<BF16>(rowp + col) : 0u, (uint32_t)col, valid);
                tpos += kWave;
            }
            if (!need) phase = 2;
        }
        if (!need && phase == 2 && cnt == 0) break;

        // Compaction (single call site): L <- exact top-k of L and the stage.
        __builtin_amdgcn_s_setprio(0);
        wave_lds_sync();
        uint64_t v[E + ES];
#pragma unroll
        for (int r = 0; r < E; ++r) v[r] = L[r];
#pragma unroll
        for (int r = 0; r < ES; ++r) {
            const int idx = r * kWave + lane;
            const uint64_t raw = idx < cnt ? stage[idx] : 0ull;
            v[E + r] = idx < cnt ? composite(key32_of_bits((uint32_t)(raw >> 32)), composite_id(raw)) : 0ull;
        }
        const uint64_t T0 = nl + cnt > k ? wave_radix_kth<E + ES>(v, k, hist) : 1ull;
        wave_lds_sync();
        int base = 0;
        uint64_t kth = ~0ull;
#pragma unroll
        for (int r = 0; r < E + ES; ++r) {
            const bool sel = v[r] != 0ull && v[r] >= T0;
            const uint64_t m = __ballot(sel);
            if (sel) stage[base + (int)mbcnt64(m)] = v[r];
            base += (int)__popcll(m);
            kth = sel ? umin64(kth, v[r]) : kth;
        }
        // Distinct composites leave at most k; never exceed the list.
        nl = base < LP ? base : LP;
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const int idx = lane * E + r;
            L[r] = idx < nl ? stage[idx] : 0ull;
        }
        wave_lds_sync();
        cnt = 0;
        if (nl >= k) {
            kth = wave_min64(kth);
            thr_own = (uint32_t)(kth >> 32) + 1u;
            if constexpr (P > 1) {
                if (lane == 0)
                    __hip_atomic_fetch_max(&thr_shared, (uint32_t)(kth >> 32), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        refresh();
        set_stream_prio(gi, ngroups);
        if (pend) {
            // The stage is empty now, so the rest of the chunk fits.
#pragma unroll
            for (int c = 0; c < kVec; ++c)
                if (c >= pend_c && pm[c]) append(pm[c], pbits[c], pcol0 + (uint32_t)c);
            pend = false;
        }
        if (phase == 2 && cnt == 0) break;
    }

    // The wave's top list, sorted descending, blocked (lane l: l*E .. l*E+E-1).
    wave_bitonic_sort<E, true>(L);

    // Workgroup: merge the waves' lists pairwise (stage memory is reused).
    if constexpr (P > 1) {
        for (int step = 1; step < P; step <<= 1) {
            __syncthreads();
            if ((wave & (2 * step - 1)) == step) {
#pragma unroll
                for (int r = 0; r < E; ++r) stage[lane * E + r] = L[r];
            }
            __syncthreads();
            if ((wave & (2 * step - 1)) == 0) {
                const uint64_t* src = stage_all[wave + step];
#pragma unroll
                for (int r = 0; r < E; ++r) L[r] = umax64(L[r], src[LP - 1 - (lane * E + r)]);
                wave_bitonic_merge<E, true>(L);
            }
        }
    }

    if (wave == 0) {
        if (groups == 1) {
            int32_t* o = out + row * ld_out;
#pragma unroll
            for (int r = 0; r < E; ++r) {
                const int i = lane * E + r;
                if (i < k) o[i] = L[r] ? (int32_t)composite_id(L[r]) : -1;
            }
        } else {
            uint64_t* p = part + ((int64_t)row * groups + g) * LP;
#pragma unroll
            for (int r = 0; r < E; ++r) p[lane * E + r] = L[r];
        }
    }
}

// Merges the `groups` sorted partial lists of each row (workspace) into ids.
template <int E, int P>
__global__ __launch_bounds__(kWave* P) void topk_rows_merge_parts_kernel(
    const uint64_t* __restrict__ part, int32_t groups, int32_t k, int32_t* __restrict__ out,
    int64_t ld_out) {
    constexpr int LP = kWave * E;
    __shared__ uint64_t xch[P][LP];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row = blockIdx.x;

    uint64_t L[E];
#pragma unroll
    for (int r = 0; r < E; ++r) L[r] = 0;
    for (int gi = wave; gi < groups; gi += P) {
        const uint64_t* src = part + ((int64_t)row * groups + gi) * LP;
#pragma unroll
        for (int r = 0; r < E; ++r) L[r] = umax64(L[r], src[LP - 1 - (lane * E + r)]);
        wave_bitonic_merge<E, true>(L);
    }
    for (int step = 1; step < P; step <<= 1) {
        __syncthreads();
        if ((wave & (2 * step - 1)) == step) {
#pragma unroll
            for (int r = 0; r < E; ++r) xch[wave][lane * E + r] = L[r];
        }
        __syncthreads();
        if ((wave & (2 * step - 1)) == 0) {
#pragma unroll
            for (int r = 0; r < E; ++r) L[r] = umax64(L[r], xch[wave + step][LP - 1 - (lane * E + r)]);
            wave_bitonic_merge<E, true>(L);
        }
    }
    if (wave == 0) {
        int32_t* o = out + row * ld_out;
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const int i = lane * E + r;
            if (i < k) o[i] = L[r] ? (int32_t)composite_id(L[r]) : -1;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

constexpr int kTargetWaves = 4096;  // 16 waves on each of 256 CUs

int list_e(int32_t k) {
    int e = 1;
    while (kWave * e < k) e <<= 1;
    return e;
}

// Stage entries per lane (new survivors between two compactions).
constexpr int stage_es(int e) { return e <= 4 ? e + 8 : (e <= 16 ? 16 : 8); }

template <int E, bool BF16, int P>
void launch_stream(const void* x, int64_t rows, int64_t cols, int64_t ld, const int32_t* re,
                   int32_t k, int32_t* out, int64_t ld_out, uint64_t* part, int groups,
                   hipStream_t s) {
    constexpr int ES = stage_es(E);
    hipLaunchKernelGGL((topk_rows_stream_kernel<E, ES, BF16, P>), dim3((unsigned)(rows * groups)),
                       dim3(kWave * P), 0, s, x, cols, ld, re, k, out, ld_out, part, groups);
}

template <int E, bool BF16>
void launch_stream_p(int p, const void* x, int64_t rows, int64_t cols, int64_t ld,
                     const int32_t* re, int32_t k, int32_t* out, int64_t ld_out, uint64_t* part,
                     int groups, hipStream_t s) {
    if (p == 4)
        launch_stream<E, BF16, 4>(x, rows, cols, ld, re, k, out, ld_out, part, groups, s);
    else if (p == 2)
        launch_stream<E, BF16, 2>(x, rows, cols, ld, re, k, out, ld_out, part, groups, s);
    else
        launch_stream<E, BF16, 1>(x, rows, cols, ld, re, k, out, ld_out, part, groups, s);
}

template <int E>
void launch_e(bool bf16, int p, const void* x, int64_t rows, int64_t cols, int64_t ld,
              const int32_t* re, int32_t k, int32_t* out, int64_t ld_out, uint64_t* part,
              int groups, hipStream_t s) {
    if (bf16)
        launch_stream_p<E, true>(p, x, rows, cols, ld, re, k, out, ld_out, part, groups, s);
    else
        launch_stream_p<E, false>(p, x, rows, cols, ld, re, k, out, ld_out, part, groups, s);
    if (groups > 1)
        hipLaunchKernelGGL((topk_rows_merge_parts_kernel<E, 4>), dim3((unsigned)rows),
                           dim3(kWave * 4), 0, s, part, groups, k, out, ld_out);
}

}  // namespace

TopkPlan plan_topk_rows(int dtype, int64_t rows, int64_t cols, int32_t k, bool allow_split) {
    (void)dtype;
    TopkPlan p{list_e(k), 1, 1, 0};
    const int64_t lp = (int64_t)kWave * p.e;
    // Keep pieces long enough that compactions stay a small part of the work.
    const int64_t min_piece = lp * 8 > 4096 ? lp * 8 : 4096;
    int64_t max_pieces = cols / min_piece;
    if (max_pieces < 1) max_pieces = 1;
    const int64_t want = rows > 0 ? (kTargetWaves + rows - 1) / rows : 1;
    const int64_t pieces = want < max_pieces ? want : max_pieces;
    if (pieces >= 4) {
        p.waves = 4;
        int64_t gr = (pieces + 3) / 4;
        if (!allow_split || gr < 2) gr = 1;
        if (gr > 256) gr = 256;
        p.groups = (int)gr;
    } else if (pieces >= 2) {
        p.waves = 2;
    }
    if (p.groups > 1) p.ws_bytes = (size_t)rows * p.groups * lp * sizeof(uint64_t);
    return p;
}

int launch_topk_rows(const void* logits, int dtype, int64_t rows, int64_t cols, int64_t ld,
                     const int32_t* row_ends, int32_t k, int32_t* out, int64_t ld_out,
                     const TopkPlan& plan, void* workspace, hipStream_t s) {
    if (rows == 0) return RTS_OK;
    const bool bf16 = dtype == RTS_BF16;
    uint64_t* part = reinterpret_cast<uint64_t*>(workspace);
    const int p = plan.waves, g = plan.groups;
    switch (plan.e) {
        case 1: launch_e<1>(bf16, p, logits, rows, cols, ld, row_ends, k, out, ld_out, part, g, s); break;
        case 2: launch_e<2>(bf16, p, logits, rows, cols, ld, row_ends, k, out, ld_out, part, g, s); break;
        case 4: launch_e<4>(bf16, p, logits, rows, cols, ld, row_ends, k, out, ld_out, part, g, s); break;
        case 8: launch_e<8>(bf16, p, logits, rows, cols, ld, row_ends, k, out, ld_out, part, g, s); break;
        case 16: launch_e<16>(bf16, p, logits, rows, cols, ld, row_ends, k, out, ld_out, part, g, s); break;
        case 32: launch_e<32>(bf16, p, logits, rows, cols, ld, row_ends, k, out, ld_out, part, g, s); break;
        default: return RTS_EUNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
}

}  // namespace rts
