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
// Short rows with k > 1024 take a second kernel (topk_rows_block_kernel) that
// holds a whole row in one workgroup's registers (described at the kernel).
#include <mutex>
#include <type_traits>

#include "rts_device.hpp"
#include "rts_internal.h"
#include "rts_levels.hpp"
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
// Chunks per load group: 4 KB per wave in flight either way (16 B per lane
// for fp32, 8 B for bf16).
template <bool BF16>
constexpr int kGroupOf = BF16 ? 8 : 4;

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

// ---------------------------------------------------------------------------
// Exact k-th composite of a wave-held set (the compaction's select).
//
// A window [w, w + span] of one 32-bit word is cut into 256 bins of width
// 2^s, counted in wave-private LDS (the wave's stage memory, whose entries
// are in registers by then; NS0 lane-striped copies for the first level,
// one copy after).  The bin where the count from the top
// reaches `need` becomes the next window (s drops by 8), first on the key
// word, then, when the k-th key is tied, on the low (id) word of the entries
// with that key.  Bins are sized from the known range, so no level needs a
// min/max pass, and a register whose entries all lie outside the window
// costs two compares.
// ---------------------------------------------------------------------------

// Counts the entries whose word x = word - w lies in [0, span] into bin
// x >> s, in NS lane-striped copies.  LO: the word is the low word, and only
// entries whose key equals key_eq count (a tie level).  Empty entries (0)
// never count: their key is 0, below every window.
template <int NV, bool LO, int NS>
__device__ __forceinline__ void radix_hist(const uint64_t (&v)[NV], uint32_t w, uint32_t span,
                                           uint32_t s, uint32_t key_eq, uint32_t* hist) {
    striped_clear<NS>(hist);
    wave_lds_sync();
    uint32_t* mine = striped_copy<NS>(hist);
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const uint32_t hi = (uint32_t)(v[r] >> 32);
        const uint32_t x = (LO ? (uint32_t)v[r] : hi) - w;
        const bool in = LO ? (hi == key_eq && x <= span) : x <= span;
        if (in) __hip_atomic_fetch_add(&mine[x >> s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
    wave_lds_sync();
}

// T such that exactly `need` nonzero entries of v[] are >= T (composites are
// distinct).  Requires at least `need` nonzero entries, all with key >= lb
// and low word in [id_lo, id_lo + id_span] (the piece's columns).
template <int NV, int NS0>
__device__ __forceinline__ uint64_t wave_kth(const uint64_t (&v)[NV], int need, uint32_t lb,
                                             uint32_t id_lo, uint32_t id_span, uint32_t* hist,
                                             bool coarse) {
    uint32_t mx = 0;
#pragma unroll
    for (int r = 0; r < NV; ++r) mx = mx > (uint32_t)(v[r] >> 32) ? mx : (uint32_t)(v[r] >> 32);
    mx = wave_max32(mx);
    // Key levels: s starts at most at 24 and drops by 8, so the fourth level
    // has s == 0 (bins of one key).
    // The window is [w, whi] (whi = w + span); every entry above it has
    // already been counted out of `need`.
    uint32_t w = lb, whi = mx, span = mx - lb;
    const int bl = span ? 32 - __clz((int)span) : 0;
    uint32_t s = bl > 8 ? (uint32_t)(bl - 8) : 0u;
#pragma unroll 1
    for (int level = 0; level < 4; ++level) {
        uint32_t bin, cb;
        bool ok;
        if (level == 0) {
            radix_hist<NV, false, NS0>(v, w, span, s, 0u, hist);
            ok = striped_find<NS0>(hist, need, bin, cb);
        } else {
            radix_hist<NV, false, 1>(v, w, span, s, 0u, hist);
            ok = striped_find<1>(hist, need, bin, cb);
        }
        if (!ok) return (uint64_t)w << 32;
        const uint32_t blo = w + (bin << s);
        if ((int)cb == need) return (uint64_t)blo << 32;
        w = blo;
        if (s == 0) break;  // the k-th key is tied
        // The chosen bin, clipped to the window (entries never exceed mx, so
        // the window stays below 2^32).
        const uint32_t top = whi - blo, width = (1u << s) - 1u;
        span = width < top ? width : top;
        whi = w + span;
        if (cb > (uint32_t)kWave || coarse) {
            // A crowded bin: narrow the window to the keys actually in it.
            // All equal (ties at the k-th key): straight to the tie levels,
            // instead of levels that would count every entry into one bin.
            // With coarse keys (bf16 widened: 2^16 apart; a row whose last
            // compaction ended tied) every bin takes this, as a bin of a few
            // such keys is usually one key.
            uint32_t bmn = 0xFFFFFFFFu, bmx = 0u;
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                const uint32_t kr = (uint32_t)(v[r] >> 32);
                const bool in = kr - w <= span;
                bmn = in && kr < bmn ? kr : bmn;
                bmx = in && kr > bmx ? kr : bmx;
            }
            bmn = wave_min32(bmn);
            bmx = wave_max32(bmx);
            w = bmn;
            if (bmn == bmx) break;
            whi = bmx;
            span = bmx - bmn;
            const int b2 = 32 - __clz((int)span);
            s = b2 > 8 ? (uint32_t)(b2 - 8) : 0u;
        } else {
            s = s > 8 ? s - 8 : 0u;
        }
    }
    // Tie levels on the low word among the entries with key w, over the
    // piece's columns only (the full 32-bit window would spend its first
    // levels with every tied entry in one bin).
    const uint32_t key = w;
    uint32_t wl = id_lo, spl = id_span;
    const int bll = spl ? 32 - __clz((int)spl) : 0;
    uint32_t sl = bll > 8 ? (uint32_t)(bll - 8) : 0u;
#pragma unroll 1
    for (int level = 0; level < 4; ++level) {
        radix_hist<NV, true, 1>(v, wl, spl, sl, key, hist);
        uint32_t bin, cb;
        if (!striped_find<1>(hist, need, bin, cb)) break;
        const uint32_t blo = wl + (bin << sl);
        if ((int)cb == need || sl == 0) return ((uint64_t)key << 32) | blo;
        const uint32_t top = id_lo + id_span - blo, width = (1u << sl) - 1u;
        spl = width < top ? width : top;
        wl = blo;
        sl = sl > 8 ? sl - 8 : 0u;
    }
    return ((uint64_t)key << 32) | wl;
}

template <int E, int ES, bool BF16, int P>
__global__ __launch_bounds__(kWave* P) __attribute__((amdgpu_waves_per_eu(E <= 8 ? 4 : 2)))
void topk_rows_stream_kernel(
    const void* __restrict__ xv, int64_t cols, int64_t ld, const int32_t* __restrict__ row_ends,
    int32_t k, int32_t* __restrict__ out, int64_t ld_out, uint64_t* __restrict__ part,
    int32_t groups) {
    using T = typename RowTraits<BF16>::elem;
    using V = typename RowTraits<BF16>::vec;
    constexpr int kGroup = kGroupOf<BF16>;
    constexpr int LP = kWave * E;
    constexpr int SCAP = kWave * ES;            // room for new survivors
    constexpr int SBUF = SCAP > LP ? SCAP : LP;  // also carries the selected list into L
    static_assert(SCAP >= kChunk, "the stage must take a whole chunk");

    // SBUF slots, then one slot per lane where lanes that fail the filter
    // write.  A compaction first moves the staged entries to registers, so
    // its histograms (NS lane-striped copies) reuse the stage memory.
    __shared__ __attribute__((aligned(16))) uint64_t stage_all[P][SBUF + kWave];
    __shared__ uint32_t thr_shared;
    // The first level of a compaction counts every entry over the whole
    // range in play, where a concentrated or heavy-tailed distribution puts
    // most entries into a few bins: 4 copies there; later levels see one
    // bin's entries, spread out, and use a single copy.
    constexpr int NS0 = stripes_fitting(2 * (SBUF + kWave)) < 4 ? stripes_fitting(2 * (SBUF + kWave)) : 4;

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row = blockIdx.x / groups;
    const int g = (int)(blockIdx.x - row * groups);
    uint64_t* stage = stage_all[wave];
    uint32_t* hist = reinterpret_cast<uint32_t*>(stage);

    int64_t e = row_ends ? (int64_t)row_ends[row] : cols;
    e = e < 0 ? 0 : (e > cols ? cols : e);

    if constexpr (P > 1) {
        if (threadIdx.x == 0) thr_shared = 0u;
        __syncthreads();
    }

    // This wave's piece [a, b) of the row (columns fit in 31 bits).
    const int64_t pieces = (int64_t)groups * P;
    const int64_t piece = (int64_t)g * P + wave;
    int64_t per = (e + pieces - 1) / pieces;
    per = (per + kChunk - 1) / kChunk * kChunk;
    const int a = (int)(piece * per < e ? piece * per : e);
    const int b = (int)(a + per < e ? a + per : e);

    const T* rowp = reinterpret_cast<const T*>(xv) + row * ld;

    int cnt = 0;                     // staged entries (wave-uniform)
    bool coarse = BF16;              // compactions narrow every boundary bin (see wave_kth)
    int nl = 0;                      // entries in the register list L (wave-uniform)
    uint32_t thr_own = 0x007FFFFFu;  // key of -inf: every non-NaN value passes
    float f = float_of_key32(thr_own);
    // The current top list: up to k composites, E per lane, in no order.
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

    // Staged entries hold the raw score bits in the high word and 2^32-1-col
    // in the low word; the key transform is applied when the stage is
    // compacted.
    auto put = [&](int slot, uint32_t bits, uint32_t idn) {
        uint32_t* p = reinterpret_cast<uint32_t*>(stage + slot);
        p[0] = idn;
        p[1] = bits;
    };

    // Elements one per lane (head and tail of the piece); needs 64 free slots.
    auto consider = [&](uint32_t bits, uint32_t col, bool valid) {
        const bool pass = valid && __uint_as_float(bits) >= f;
        const uint64_t m = __ballot(pass);
        if (m) {
            if (pass) put(cnt + (int)mbcnt64(m), bits, 0xFFFFFFFFu - col);
            cnt += (int)__popcll(m);
        }
    };

    // Geometry: head [a, a1) up to the first aligned vector, body of whole
    // chunks, tail [t0, b).
    int a1 = a, nch = 0, t0 = a;
    if (a < b) {
        constexpr int vbytes = sizeof(V);
        const uintptr_t base = reinterpret_cast<uintptr_t>(rowp);
        const int off = (int)((base % vbytes) / sizeof(T));
        a1 = a + (kVec - (off + a) % kVec) % kVec;
        a1 = a1 < b ? a1 : b;
        nch = (b - a1) / kChunk;
        t0 = a1 + nch * kChunk;
    }
    const V* cbase = reinterpret_cast<const V*>(rowp + a1);  // wave-uniform
    const int ngroups = (nch + kGroup - 1) / kGroup;
    // 2^32-1 minus this lane's first column in chunk 0.
    const uint32_t idn0 = 0xFFFFFFFFu - (uint32_t)(a1 + lane * kVec);

    // Issue priority.  The SIMD issues the oldest ready wave first, so waves
    // that started later fall behind once compactions compete for issue slots.
    // A streaming wave takes priority 3..1 as it advances through its piece, so
    // the ones behind win; a wave that compacts drops to 0, so waves about to
    // issue loads keep the memory pipe full while it works.
    const int g1 = ngroups / 3, g2 = (2 * ngroups) / 3;
    auto set_stream_prio = [&](int gdone) {
        if (gdone < g1) __builtin_amdgcn_s_setprio(3);
        else if (gdone < g2) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(1);
    };
    __builtin_amdgcn_s_setprio(3);

    // Head: fewer than kVec elements, the stage is empty.
    if (a1 > a) {
        const int col = a + lane;
        const bool valid = col < a1;
        consider(valid ? load_bits<BF16>(rowp + col) : 0u, (uint32_t)col, valid);
    }

    V A[kGroup], B[kGroup];
    // Loads group gi.  The refills are unconditional, so the order of
    // outstanding loads is the same on every path.  Buffer loads through a
    // resource made per group (base: the group's first chunk; size: the
    // piece's bytes left, at most a group): the lane's byte offset sits in a
    // VGPR set once, so a refill computes no vector address in the registers
    // the previous group's data occupies (which made it wait for the other
    // group's loads).  Chunks past the piece's end are out of range and read
    // as zeros without touching memory; they are never filtered.
    const int voff = lane * (int)sizeof(V);
    auto load_group = [&](V(&dst)[kGroup], int gi) {
        constexpr int kGroupBytes = kGroup * kChunk * (int)sizeof(T);
        const int left = nch - gi * kGroup;
        const int bytes = left <= 0 ? 0 : (left >= kGroup ? kGroupBytes : left * kChunk * (int)sizeof(T));
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<V*>(cbase + (int64_t)gi * kGroup * kWave), (short)0, bytes, 0x00020000);
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            constexpr int kChunkBytes = kChunk * (int)sizeof(T);
            if constexpr (BF16)
                dst[u] = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff + u * kChunkBytes, 0, 2);
            else
                dst[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + u * kChunkBytes, 0, 2);
        }
    };
    int gi = 0;
    if (ngroups > 0) {
        load_group(A, 0);
        load_group(B, 1);
    }
    // First chunk of group A still to filter.  A chunk whose survivors do not
    // fit in the stage is left whole and filtered again after the compaction
    // (against the raised threshold: its elements come after every listed
    // one, so a tie with the k-th listed key loses and the strict filter is
    // exact).
    int ustart = 0;
    int tpos = t0;
    int phase = ngroups > 0 ? 0 : 1;  // 0 body, 1 tail, 2 end

    // One chunk (lane l holds columns col0+4l .. col0+4l+3, idn = 2^32-1 -
    // (col0+4l)): stages every survivor, or nothing and returns false when
    // they do not all fit.  Lanes whose element fails write their own sink
    // slot past the stage instead, so a component costs no exec-mask changes.
    // Slots are addressed by LDS byte address (a wave-uniform running base
    // plus 8 * the lane's rank among the component's survivors), and the two
    // words of an entry are written from their own registers.
    const uint32_t stage_base = lds_addr(stage);
    const uint32_t sink = stage_base + (uint32_t)(SBUF + lane) * 8u;
    auto chunk = [&](V vv, uint32_t idn) -> bool {
        uint32_t bits[kVec];
        unpack<BF16>(vv, bits);
        bool pass[kVec];
        uint64_t m[kVec];
#pragma unroll
        for (int c = 0; c < kVec; ++c) {
            pass[c] = __uint_as_float(bits[c]) >= f;
            m[c] = __ballot(pass[c]);
        }
        if ((m[0] | m[1] | m[2] | m[3]) == 0ull) return true;
        // A chunk adds at most kChunk entries: count exactly only near full.
        if (cnt > SCAP - kChunk &&
            cnt + (int)(__popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3])) > SCAP)
            return false;
        // The running slot count stays in a VGPR and advances with v_bcnt (the
        // lane's slot comes from v_mbcnt on it), so an append costs no SALU
        // beyond the test of its mask.
        uint32_t off = (uint32_t)cnt;
        asm volatile("" : "+v"(off));
#pragma unroll
        for (int c = 0; c < kVec; ++c) {
            if (m[c]) {
                const uint32_t lo = (uint32_t)m[c], hi = (uint32_t)(m[c] >> 32);
                const uint32_t pos = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, off));
                const uint32_t a = select_by_mask(m[c], stage_base + pos * 8u, sink);
                lds_store2(a, idn - (uint32_t)c, bits[c]);
                uint32_t t;
                asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(t) : "s"(lo), "v"(off));
                asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(off) : "s"(hi), "v"(t));
            }
        }
        cnt = __builtin_amdgcn_readfirstlane((int)off);
        return true;
    };

    // Filters the chunks ustart.. of group gi held in buf; true if the stage
    // filled up (ustart then names the chunk to filter again).
    auto run_group = [&](V(&buf)[kGroup]) -> bool {
        const uint32_t idg = idn0 - (uint32_t)(gi * kGroup * kChunk);
        if (ustart == 0 && (gi + 1) * kGroup <= nch) {
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                if (!chunk(buf[u], idg - (uint32_t)(u * kChunk))) {
                    ustart = u;
                    return true;
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                if (u >= ustart && gi * kGroup + u < nch &&
                    !chunk(buf[u], idg - (uint32_t)(u * kChunk))) {
                    ustart = u;
                    return true;
                }
            }
        }
        return false;
    };
    // The buffers alternate: A holds group gi and B group gi + 1 at the top of
    // an iteration; each is refilled with the group after next as soon as it
    // is consumed, so two groups stay in flight without register copies.  The
    // body is straight-line (A half, then B half), so at the back edge B's
    // loads are always the younger ones.  half == 1 only on re-entry after a
    // compaction that interrupted the B half.
    int half = 0;

    for (;;) {
        bool need = false;
        if (phase == 0) {
            while (true) {
                if (half == 0) {
                    if (run_group(A)) {
                        need = true;
                        break;
                    }
                    load_group(A, gi + 2);
                    ustart = 0;
                    if (++gi >= ngroups) {
                        phase = 1;
                        break;
                    }
                    if constexpr (P > 1) refresh();
                    if ((gi & 7) == 0) set_stream_prio(gi);
                }
                half = 0;
                if (run_group(B)) {
                    half = 1;
                    need = true;
                    break;
                }
                load_group(B, gi + 2);
                ustart = 0;
                if (++gi >= ngroups) {
                    phase = 1;
                    break;
                }
                if constexpr (P > 1) refresh();
                if ((gi & 7) == 0) set_stream_prio(gi);
            }
        }
        if (!need && phase == 1) {
            while (tpos < b) {
                if (cnt + kWave > SCAP) {
                    need = true;
                    break;
                }
                const int col = tpos + lane;
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
            v[E + r] = idx < cnt ? ((uint64_t)key32_of_bits((uint32_t)(raw >> 32)) << 32) |
                                       (uint32_t)raw
                                 : 0ull;
        }
        // Every entry has key >= thr_own - 1: the list's entries are at or
        // above its k-th key, and the filter passes keys >= thr_own (-0 also
        // passes a +0 threshold, one key below).  Until the list first holds
        // k entries that bound is the key of -inf, far below the entries:
        // the window then starts at their smallest key, or concentrated
        // scores (all inside one binade) would share a few bins of the first
        // levels and serialise their histogram atomics.
        uint64_t T0 = 1ull;
        if (nl + cnt > k) {
            uint32_t lb = thr_own - 1u;
            if (nl < k) {
                uint32_t m1 = 0xFFFFFFFFu;  // min of key - 1: empty slots (key 0) wrap to the top
#pragma unroll
                for (int r = 0; r < E + ES; ++r) {
                    const uint32_t km1 = (uint32_t)(v[r] >> 32) - 1u;
                    m1 = km1 < m1 ? km1 : m1;
                }
                lb = wave_min32(m1) + 1u;
            }
            // low words of the piece's entries: 2^32-1-col for col in [a, b)
            wave_lds_sync();  // the stage's entries are in v[]: its memory holds the histograms
            T0 = wave_kth<E + ES, NS0>(v, k, lb, 0xFFFFFFFFu - (uint32_t)(b - 1), (uint32_t)(b - 1 - a), hist,
                                       coarse);
            // A k-th composite with a nonzero id word ended in the tie levels.
            coarse = BF16 || (uint32_t)T0 != 0u;
        }
        int base = 0;
        uint32_t kmin = 0xFFFFFFFFu;
#pragma unroll
        for (int r = 0; r < E + ES; ++r) {
            const bool sel = v[r] >= T0;  // T0 >= 1: empty slots never
            const uint64_t m = __ballot(sel);
            const int nsel = (int)__popcll(m);
            // Exactly k entries are selected; the bound only guards the
            // stage if that were ever not so.
            if (sel && base + nsel <= SBUF) {
                stage[base + (int)mbcnt64(m)] = v[r];
                const uint32_t key = (uint32_t)(v[r] >> 32);
                kmin = key < kmin ? key : kmin;
            }
            base += base + nsel <= SBUF ? nsel : 0;
        }
        // Distinct composites leave at most k; never exceed the list.
        nl = base < LP ? base : LP;
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const int idx = r * kWave + lane;
            L[r] = idx < nl ? stage[idx] : 0ull;
        }
        wave_lds_sync();
        cnt = 0;
        if (nl >= k) {
            const uint32_t kth = wave_min32(kmin);
            thr_own = kth + 1u;
            if constexpr (P > 1) {
                if (lane == 0)
                    __hip_atomic_fetch_max(&thr_shared, kth, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        refresh();
        set_stream_prio(gi);
        if (phase == 2) break;
        // Every load has landed by now (the compaction is long); waiting here
        // keeps the compiler's view of which buffer is younger exact at the
        // loop head, so the stream loop waits only for the buffer it reads.
        __builtin_amdgcn_s_waitcnt(0);
    }
    // One wave with a bf16 row of fewer than 2^16 columns sorts 32-bit words:
    // the key's top 16 bits (the rest follow the sign) over 0xFFFF - column,
    // the composite's order, at half the lane traffic and selects.
    if constexpr (BF16 && P == 1) {
        if (groups == 1 && cols <= 65536) {
            uint32_t L32[E];
#pragma unroll
            for (int r = 0; r < E; ++r)
                L32[r] = ((uint32_t)(L[r] >> 32) & 0xFFFF0000u) | ((uint32_t)L[r] & 0xFFFFu);
            wave_bitonic_sort<E, true>(L32);
            int lane_o = lane;
            asm volatile("" : "+v"(lane_o));
            int32_t* o = out + row * ld_out;
#pragma unroll
            for (int r = 0; r < E; ++r) {
                const int i = lane_o * E + r;
                if (i < k) o[i] = L32[r] ? (int32_t)(0xFFFFu - (L32[r] & 0xFFFFu)) : -1;
            }
            return;
        }
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
        // An opaque copy of the lane index: without it the compiler computes
        // the output positions at the start and holds them through the stream.
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        if (groups == 1) {
            int32_t* o = out + row * ld_out;
#pragma unroll
            for (int r = 0; r < E; ++r) {
                const int i = lane_o * E + r;
                if (i < k) o[i] = L[r] ? (int32_t)composite_id(L[r]) : -1;
            }
        } else {
            uint64_t* p = part + ((int64_t)row * groups + g) * LP;
#pragma unroll
            for (int r = 0; r < E; ++r) p[lane_o * E + r] = L[r];
        }
    }
}

// ---------------------------------------------------------------------------
// Short rows with a large k: one workgroup of NW waves holds the whole row in
// registers (KPT elements per thread, the column implied by the position), so
// a row costs one read and no compaction however many candidates survive.
//   1. the row as fp32 bits (bf16 widened), an empty slot (NaN, or at or past
//      the row end) a quiet NaN; valid count and score range;
//   2. a first radix level linear in the score (256 bins of [min, max]),
//      lane-striped LDS histogram copies;
//   3. one pass: keys above the boundary bin are selected (written once the
//      waves' offsets are known), the boundary bin's go to a per-wave LDS
//      list, where the later levels and the tie rule (ascending column) run;
//      a row whose list overflows runs them over its registers as keys;
//   4. the selected (exactly min(k, valid)) in LDS are put in order: fp32 rows
//      by bucket rank (each id written straight to its place), bf16 rows and
//      fp32 rows with crowded buckets by a bitonic network over the workgroup
//      (each wave sorts 64*E in registers, even waves descending, odd
//      ascending; the cross-wave steps exchange through LDS and each wave
//      finishes with an in-register merge).
// Element i of thread t: column 4 * (g * 64 * NW + t) + j for i = 4g + j, so
// each group of four is one 16-byte (fp32) or 8-byte (bf16) load and a wave's
// load covers 1 KB (512 B) of the row.
// ---------------------------------------------------------------------------
template <int NW>
struct BlockRowSmem {
    static constexpr bool kWave0Find = true;
    uint32_t hist[kLevelCopies][kLevelStride];
    uint32_t bins[256];
    uint32_t bc[4];
    uint32_t tied[kWave];
    uint32_t ntied;
    uint32_t nsel;
    uint32_t nlist[NW];
    uint32_t red[NW][4];
};

template <int NW, int KPT, int E, bool BF16>
__global__ __launch_bounds__(kWave* NW) void topk_rows_block_kernel(
    const void* __restrict__ xv, int64_t cols, int64_t ld, const int32_t* __restrict__ row_ends,
    int32_t k, int32_t* __restrict__ out, int64_t ld_out) {
    using T = typename RowTraits<BF16>::elem;
    using V = typename RowTraits<BF16>::vec;
    constexpr int NT = kWave * NW;
    constexpr int S = kWave * E;  // sort slots per wave
    constexpr int LS = S * NW;    // sort slots of the workgroup (>= k)
    static_assert(KPT % 4 == 0, "keys come in groups of four");
    __shared__ BlockRowSmem<NW> sm;
    constexpr int CAPL = 128;     // boundary-bin list entries per wave
    // A second sort exchange buffer for 8 waves (six cross-wave steps) of
    // 32-bit elements; with 64-bit ones, or 4 waves, the LDS would cost
    // workgroups per CU.
    constexpr bool kSortDoubleBuffer = NW >= 8 && BF16;
    // Sort elements: for bf16 one 32-bit word, the key's top 16 bits (the
    // rest follow the sign) over 0xFFFF - column (columns < 2^14 here), with
    // the order of the 64-bit composite; for fp32 the composite.  0: empty.
    using SK = std::conditional_t<BF16, uint32_t, uint64_t>;
    auto sort_key = [](uint32_t key, uint32_t col) -> SK {
        if constexpr (BF16)
            return (key & 0xFFFF0000u) | (0xFFFFu - col);
        else
            return composite(key, col);
    };
    auto sort_key_of = [&](uint64_t c) -> SK { return sort_key((uint32_t)(c >> 32), composite_id(c)); };
    __shared__ SK buf[LS];
    __shared__ SK buf2[kSortDoubleBuffer ? LS : 1];
    __shared__ uint64_t lst[NW][CAPL];
    const int t = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int64_t row = blockIdx.x;
    int64_t e = row_ends ? (int64_t)row_ends[row] : cols;
    e = e < 0 ? 0 : (e > cols ? cols : e);
    const T* rowp = reinterpret_cast<const T*>(xv) + row * ld;

    for (int q = t; q < kLevelCopies * kLevelStride; q += NT) (&sm.hist[0][0])[q] = 0u;
    if (t == 0) {
        sm.ntied = 0u;
        sm.nsel = 0u;
    }
    if (t < NW) sm.nlist[t] = 0u;

    // Column of key i, from the thread's base column 4t.  Each pass takes an
    // opaque copy of the base, so the compiler cannot keep KPT column values
    // live from pass to pass.
    auto col_base = [&]() -> uint32_t {
        uint32_t b = 4u * (uint32_t)t;
        asm volatile("" : "+v"(b));
        return b;
    };
    auto col_at = [](uint32_t base, int i) -> uint32_t {
        return base + (uint32_t)(4 * (i >> 2) * NT + (i & 3));
    };
    // Loads through a buffer resource over the row's valid bytes: a lane's
    // offset is one register and the group's offset a constant, and reads
    // past the row end return zero without touching memory.  Every group is
    // one vector load, all issued before any is used; the group cut by the
    // row end, or every group of a row not aligned to a vector, is read
    // element by element.
    const int ei = (int)e;  // e <= cols <= 64 * 8 * KPT
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(rowp), (short)0, ei * (int)sizeof(T), 0x00020000);
    const bool vec_ok = (reinterpret_cast<uintptr_t>(rowp) % sizeof(V)) == 0;
    // The row as fp32 bits (bf16 widened), every empty slot (past the row
    // end, or NaN) the quiet NaN kEmpty: ordered compares on it are false,
    // and a key is formed only where one is needed.
    constexpr uint32_t kEmpty = 0x7FC00000u;
    uint32_t fb[KPT];
    // The passes that need every key (the register levels, the selection
    // below) turn fb into keys in place first (0 for an empty slot).
    bool keyed = false;
    auto to_keys = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) fb[i] = fb[i] == kEmpty ? 0u : key32_of_bits(fb[i]);
        keyed = true;
    };
    {
        V raw[KPT / 4];
        const int voff = t * (int)sizeof(V);
#pragma unroll
        for (int g = 0; g < KPT / 4; ++g) {
            constexpr int kGroupStride = NT * (int)sizeof(V);
            if constexpr (BF16)
                raw[g] = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, g * kGroupStride, 2);
            else
                raw[g] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, g * kGroupStride, 2);
        }
        const int t4 = (int)col_base();
#pragma unroll
        for (int g = 0; g < KPT / 4; ++g) {
            const int c0 = g * NT * 4 + t4;
            uint32_t bits[4];
            unpack<BF16>(raw[g], bits);
            if (c0 < ei && (!vec_ok || c0 + 4 > ei)) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (BF16)
                        bits[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsrc, (c0 + j) * 2, 0, 0) << 16;
                    else
                        bits[j] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (c0 + j) * 4, 0, 0);
                }
            }
            if ((g + 1) * NT * 4 <= ei) {  // the whole group is inside the row end, for every lane
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    fb[4 * g + j] = __builtin_isnan(__uint_as_float(bits[j])) ? kEmpty : bits[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = c0 + j < ei && !__builtin_isnan(__uint_as_float(bits[j]));
                    fb[4 * g + j] = ok ? bits[j] : kEmpty;
                }
            }
        }
    }

    // Valid count and key range: per lane in floats (compare and select,
    // which passes over kEmpty), then as keys for the wave and workgroup
    // reductions (lane w < NW combines wave w's).  A lane's zero minimum
    // (maximum) counts as -0 (+0): a compare does not order the two zeros.
    uint32_t nv = 0, mn, mx;
    {
        float fmn = __builtin_inff(), fmx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const float f = __uint_as_float(fb[i]);
            nv += __builtin_isnan(f) ? 0u : 1u;
            fmn = f < fmn ? f : fmn;
            fmx = f > fmx ? f : fmx;
        }
        mn = fmn == 0.0f ? 0x7FFFFFFFu : key32_of_bits(__float_as_uint(fmn));  // key of -0
        mx = fmx == 0.0f ? 0x80000000u : key32_of_bits(__float_as_uint(fmx));  // key of +0
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
        const bool wl = lane < NW;
        nv = wave_sum32(wl ? sm.red[lane][0] : 0u);
        mn = wave_min32(wl ? sm.red[lane][1] : 0xFFFFFFFFu);
        mx = wave_max32(wl ? sm.red[lane][2] : 0u);
    }

    // Selected: key > thr_gt, or key == tie_key and column <= col_cut.
    uint32_t thr_gt = 0u, tie_key = 0u, col_cut = 0u;
    auto selected = [&](uint32_t kk, uint32_t c) {
        return kk != 0u && (kk > thr_gt || (kk == tie_key && c <= col_cut));
    };
    bool written = false;  // the k selected composites are in buf already
    if (nv > (uint32_t)k) {
        auto visit = [&](auto f) __attribute__((always_inline)) {
            const uint32_t cb = col_base();
#pragma unroll
            for (int i = 0; i < KPT; ++i) f(fb[i], col_at(cb, i));  // fb holds keys here
        };
        int need = k;
        uint32_t wlo = mn, whi = mx;
        bool done = false;
        // First level in score space: bins of the score range, linear in
        // the value.  bin(v) = min(255, (v - lo) * 256 / (hi - lo)) is
        // monotone in the key (rounding is monotone; +-0 share a bin), so the
        // keys of a bin form one key range.  Key-space bins of the full range
        // are a binade wide and would put a bell-shaped row into a handful of
        // bins.  Infinite or degenerate ranges skip this level.
        const float lo = float_of_key32(mn), hi = float_of_key32(mx);
        const float scale = 256.0f / (hi - lo);
        if (__builtin_isfinite(lo) && __builtin_isfinite(hi) && hi > lo && __builtin_isfinite(scale)) {
            // tb = (v - lo) * scale lies in [0, 256] for a value, NaN for an
            // empty slot, which counts into the padding word 256 (no level
            // reads it).
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const float tb = (__uint_as_float(fb[i]) - lo) * scale;
                const uint32_t tbi = (uint32_t)tb;
                const uint32_t vb = tb >= 0.0f ? (tbi < 255u ? tbi : 255u) : 256u;
                __hip_atomic_fetch_add(&sm.hist[lane & (kLevelCopies - 1)][vb], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            uint32_t bin, cbin;
            if (level_hist_find(sm, need, bin, cbin)) {
                // One pass over the keys: a key in a bin above the boundary bin
                // is selected (a bit of amask, written once the offsets are
                // known), a key in the boundary bin goes to the wave's list (at
                // most CAPL; slots from an LDS counter, as the list's order
                // does not matter), where the later levels and the tie rule
                // resolve it.  The boundary bin's key range comes along.
                // Counts stay per lane: no wave masks are held per key.
                uint32_t amask = 0u, na = 0u, lmn = 0xFFFFFFFFu, lmx = 0u;
                const uint32_t cbl = col_base();
                // The bins again from an opaque copy of the offset: otherwise
                // the compiler keeps every key's bin from the histogram pass
                // (a register per key).
                float lo2 = lo;
                asm volatile("" : "+v"(lo2));
                // The bin test as compares on tb: bin(v) > bin iff tb >= bin + 1
                // (never for the top bin), bin(v) == bin iff bin <= tb and not
                // above; both are false for an empty slot.
                const float t_in = (float)bin;
                const float t_above = bin < 255u ? (float)(bin + 1u) : __builtin_inff();
#pragma unroll
                for (int i = 0; i < KPT; ++i) {
                    const float tb = (__uint_as_float(fb[i]) - lo2) * scale;
                    const bool above = tb >= t_above;
                    amask |= above ? (1u << i) : 0u;
                    na += above ? 1u : 0u;
                    if (tb >= t_in && !above) {
                        const uint32_t kk = key32_of_bits(fb[i]);
                        const uint32_t pos = __hip_atomic_fetch_add(&sm.nlist[wave], 1u, __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_WORKGROUP);
                        if (pos < (uint32_t)CAPL) lst[wave][pos] = composite(kk, col_at(cbl, i));
                        lmn = kk < lmn ? kk : lmn;
                        lmx = kk > lmx ? kk : lmx;
                    }
                }
                const uint32_t na_incl = wave_incl_scan32(na);
                const uint32_t na_wave = (uint32_t)__builtin_amdgcn_readlane((int)na_incl, kWave - 1);
                lmn = wave_min32(lmn);
                lmx = wave_max32(lmx);
                if (lane == 0) {
                    sm.red[wave][0] = na_wave;
                    sm.red[wave][2] = lmn;
                    sm.red[wave][3] = lmx;
                }
                lds_barrier();
                // Lane w < NW takes wave w's figures; wave reductions combine
                // them (fewer registers than every wave's figures in each lane).
                const uint32_t nl = sm.nlist[wave];
                uint32_t aoff, atot, bmn, bmx;
                bool fits;
                {
                    const bool wl = lane < NW;
                    const uint32_t wa = wl ? sm.red[lane][0] : 0u;
                    const uint32_t incl = wave_incl_scan32(wa);
                    atot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
                    aoff = wave == 0 ? 0u : (uint32_t)__builtin_amdgcn_readlane((int)incl, wave - 1);
                    fits = wave_max32(wl ? sm.nlist[lane] : 0u) <= (uint32_t)CAPL;
                    bmn = wave_min32(wl ? sm.red[lane][2] : 0xFFFFFFFFu);
                    bmx = wave_max32(wl ? sm.red[lane][3] : 0u);
                }
                if ((int)cbin == need) thr_gt = bmn - 1u;  // the whole bin is taken: keys >= its smallest
                if (fits) {
                    // The list's levels on the keys' significant bits: a bf16
                    // key varies only in its top 16 (the rest follow the sign),
                    // so ties show at the first level there.  lthr / ltie /
                    // lcut: the selection rule in those units.
                    constexpr int KS = BF16 ? 16 : 0;
                    uint32_t lthr = (bmn >> KS) - 1u, ltie = 0u, lcut = 0u;  // whole bin taken
                    if ((int)cbin != need) {
                        const uint32_t mine = nl;  // this wave's list entries
                        auto visit_list = [&](auto f) __attribute__((always_inline)) {
                            for (uint32_t p = (uint32_t)lane; p < mine; p += kWave) {
                                const uint64_t c = lst[wave][p];
                                f((uint32_t)(c >> (32 + KS)), composite_id(c));
                            }
                        };
                        const uint32_t llo = bmn >> KS, lhi = bmx >> KS;
                        const uint32_t span = lhi - llo;
                        const int bl = span ? 32 - __clz((int)span) : 0;
                        const uint32_t sh = bl > 8 ? (uint32_t)(bl - 8) : 0u;
                        bool ties;
                        uint32_t ntie;
                        radix_levels(sm, visit_list, need, llo, span, sh, lhi, lthr, ties, ltie, ntie);
                        if (ties) lcut = tie_cut(sm, visit_list, ltie, ntie, need, (uint32_t)(cols - 1));
                    }
                    // The selected: keys above the boundary bin at this wave's
                    // offset, then the list's selected after all of those (any
                    // order: the sort below fixes it), then empty slots.
                    const uint32_t cbw = col_base();
                    uint32_t q = aoff + na_incl - na;  // this lane's first slot
#pragma unroll
                    for (int i = 0; i < KPT; ++i) {
                        const uint32_t a = (amask >> i) & 1u;
                        if (a) buf[q] = sort_key(key32_of_bits(fb[i]), col_at(cbw, i));
                        q += a;
                    }
                    for (uint32_t p = (uint32_t)lane; p < nl; p += kWave) {
                        const uint64_t c = lst[wave][p];
                        const uint32_t kk = (uint32_t)(c >> (32 + KS));
                        if (kk > lthr || (kk == ltie && composite_id(c) <= lcut)) {
                            const uint32_t q = __hip_atomic_fetch_add(&sm.nsel, 1u, __ATOMIC_RELAXED,
                                                                      __HIP_MEMORY_SCOPE_WORKGROUP);
                            buf[atot + q] = sort_key_of(c);
                        }
                    }
                    for (int p = k + t; p < LS; p += NT) buf[p] = 0;
                    written = true;
                    done = true;
                } else {
                    lds_barrier();  // sm.red is rewritten below
                    if ((int)cbin == need) {
                        done = true;
                    } else {
                        wlo = bmn;
                        whi = bmx;
                    }
                }
            }
        }
        if (!done) {
            to_keys();
            const uint32_t span = whi - wlo;
            const int bl = span ? 32 - __clz((int)span) : 0;
            const uint32_t sh = bl > 8 ? (uint32_t)(bl - 8) : 0u;
            bool ties;
            uint32_t ntie;
            radix_levels(sm, visit, need, wlo, span, sh, whi, thr_gt, ties, tie_key, ntie);
            if (ties) col_cut = tie_cut(sm, visit, tie_key, ntie, need, (uint32_t)(cols - 1));
        }
    }

    if (!written) {
        // The selected composites into LDS (any order), empty slots after them.
        if (!keyed) to_keys();
        uint32_t cnt = 0;
        uint32_t cb = col_base();
#pragma unroll
        for (int i = 0; i < KPT; ++i) cnt += (uint32_t)__popcll(__ballot(selected(fb[i], col_at(cb, i))));
        if (lane == 0) sm.red[wave][3] = cnt;
        lds_barrier();
        const uint32_t incl = wave_incl_scan32(lane < NW ? sm.red[lane][3] : 0u);
        uint32_t off = wave == 0 ? 0u : (uint32_t)__builtin_amdgcn_readlane((int)incl, wave - 1);
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
        cb = col_base();
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const uint32_t c = col_at(cb, i);
            const uint32_t kk = fb[i];
            const bool sel = selected(kk, c);
            const uint64_t m = __ballot(sel);
            const uint32_t pos = off + mbcnt64(m);
            if (sel && pos < (uint32_t)LS) {
                // The key through a copy in another register: a composite
                // built on the register itself would pin every key to the odd
                // half of an aligned register pair.
                uint32_t kc;
                asm volatile("v_mov_b32 %0, %1" : "=&v"(kc) : "v"(kk));
                buf[pos] = sort_key(kc, c);
            }
            off += (uint32_t)__popcll(m);
        }
        for (int p = (int)(total < (uint32_t)LS ? total : (uint32_t)LS) + t; p < LS; p += NT) buf[p] = 0;
    }
    lds_barrier();

    // fp32 rows with the k selected in buf: each goes straight to its place,
    // no sort network.  Buckets of the selected keys' range from the top
    // (2^bits of them, bits from the LDS the list used) order the keys
    // between buckets; a key's place in its bucket is the count of its
    // bucket-mates with a larger composite.  Buckets of more than 32 (ties,
    // crowded values) leave the row to the network below.
    bool ranked = false;
    if constexpr (!BF16) {
        if (written) {
            constexpr int NB = NW * CAPL * 2;  // buckets: the list's LDS as words
            constexpr int BPT = NB / NT;       // buckets per thread (4)
            static_assert(BPT * NT == NB && NB <= 65536, "bucket layout");
            constexpr int NBB = NB == 2048 ? 11 : NB == 1024 ? 10 : 12;
            static_assert((1 << NBB) == NB, "buckets are a power of two");
            uint32_t* bcount = reinterpret_cast<uint32_t*>(&lst[0][0]);
            uint16_t* bidx = reinterpret_cast<uint16_t*>(&sm.hist[0][0]);
            static_assert(sizeof(sm.hist) >= LS * sizeof(uint16_t), "index list fits the histogram");
            SK v[E];
            uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
            for (int r = 0; r < E; ++r) {
                v[r] = buf[t * E + r];
                const uint32_t kk = (uint32_t)(v[r] >> 32);
                if (t * E + r < k) {
                    kmn = kk < kmn ? kk : kmn;
                    kmx = kk > kmx ? kk : kmx;
                }
            }
            kmn = wave_min32(kmn);
            kmx = wave_max32(kmx);
            if (lane == 0) {
                sm.red[wave][0] = kmn;
                sm.red[wave][1] = kmx;
            }
            for (int q = t; q < NB; q += NT) bcount[q] = 0u;
            lds_barrier();
            kmn = wave_min32(lane < NW ? sm.red[lane][0] : 0xFFFFFFFFu);
            kmx = wave_max32(lane < NW ? sm.red[lane][1] : 0u);
            const uint32_t span = kmx - kmn;
            const int sbits = span ? 32 - __clz((int)span) : 0;
            const uint32_t bsh = sbits > NBB ? (uint32_t)(sbits - NBB) : 0u;
            uint32_t bk[E], slot[E];
#pragma unroll
            for (int r = 0; r < E; ++r) {
                bk[r] = (kmx - (uint32_t)(v[r] >> 32)) >> bsh;  // < NB
                slot[r] = 0u;
                if (t * E + r < k)
                    slot[r] = __hip_atomic_fetch_add(&bcount[bk[r]], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            lds_barrier();
            // Bucket starts: this thread's BPT buckets, a wave scan, the waves' totals.
            uint32_t c[BPT], tot = 0u, cmax = 0u;
#pragma unroll
            for (int j = 0; j < BPT; ++j) {
                c[j] = bcount[t * BPT + j];
                tot += c[j];
                cmax = c[j] > cmax ? c[j] : cmax;
            }
            const uint32_t incl = wave_incl_scan32(tot);
            cmax = wave_max32(cmax);
            if (lane == 0) {
                sm.red[wave][2] = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
                sm.red[wave][3] = cmax;
            }
            lds_barrier();
            const uint32_t wincl = wave_incl_scan32(lane < NW ? sm.red[lane][2] : 0u);
            const uint32_t woff = wave == 0 ? 0u : (uint32_t)__builtin_amdgcn_readlane((int)wincl, wave - 1);
            const uint32_t big = wave_max32(lane < NW ? sm.red[lane][3] : 0u);
            if (big <= 32u) {
                uint32_t st = woff + incl - tot;
#pragma unroll
                for (int j = 0; j < BPT; ++j) {
                    bcount[t * BPT + j] = st;  // each thread rewrites only its own buckets
                    st += c[j];
                }
                lds_barrier();
                uint32_t bst[E], ben[E];
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    bst[r] = bcount[bk[r]];
                    ben[r] = bk[r] + 1 < (uint32_t)NB ? bcount[bk[r] + 1] : (uint32_t)k;
                    if (t * E + r < k) bidx[bst[r] + slot[r]] = (uint16_t)(t * E + r);
                }
                lds_barrier();
                int32_t* o_row = out + row * ld_out;
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    if (t * E + r < k) {
                        uint32_t above = 0u;
                        for (uint32_t q = bst[r]; q < ben[r]; ++q) above += buf[bidx[q]] > v[r] ? 1u : 0u;
                        o_row[bst[r] + above] = (int32_t)composite_id(v[r]);
                    }
                }
                ranked = true;
            }
        }
    }

    if (!ranked) {
        // Descending sort of the LS slots; element i = wave * S + lane * E + r.
        SK v[E];
    #pragma unroll
        for (int r = 0; r < E; ++r) v[r] = buf[wave * S + lane * E + r];
        wave_bitonic_sort_dir<E>(v, (wave & 1) == 0);
        // Cross-wave steps exchange through LDS.  With two exchange buffers
        // used in turn, a step's write cannot meet the previous step's reads
        // (those end before that step's barrier), so a step takes one barrier.
        int xi = 0;
    #pragma unroll
        for (int K = 2 * S; K <= LS; K *= 2) {
            const bool desc = ((wave * S) & K) == 0;
    #pragma unroll
            for (int J = K / 2; J >= S; J /= 2) {
                SK* xb = (kSortDoubleBuffer && (xi & 1)) ? buf2 : buf;
                ++xi;
                if (!kSortDoubleBuffer) lds_barrier();
    #pragma unroll
                for (int r = 0; r < E; ++r) xb[wave * S + lane * E + r] = v[r];
                lds_barrier();
                const int pw = wave ^ (J / S);
                const bool keep_max = (wave < pw) == desc;
    #pragma unroll
                for (int r = 0; r < E; ++r) {
                    const SK o = xb[pw * S + lane * E + r];
                    v[r] = keep_max ? (v[r] < o ? o : v[r]) : (v[r] < o ? v[r] : o);
                }
            }
            wave_bitonic_merge_dir<E>(v, desc);
        }
        int32_t* o_row = out + row * ld_out;
    #pragma unroll
        for (int r = 0; r < E; ++r) {
            const int i = wave * S + lane * E + r;
            if (i < k) {
                if constexpr (BF16)
                    o_row[i] = v[r] ? (int32_t)(0xFFFFu - (v[r] & 0xFFFFu)) : -1;
                else
                    o_row[i] = v[r] ? (int32_t)composite_id(v[r]) : -1;
            }
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

// Whole rows in one workgroup (topk_rows_block_kernel): 32 keys per thread,
// 4 waves for rows of up to 8192 columns, 8 up to 16384.
constexpr int kBlockKeys = 32;
constexpr int64_t kBlockMaxCols = (int64_t)kWave * 8 * kBlockKeys;

TopkPlan plan_topk_rows(int dtype, int64_t rows, int64_t cols, int32_t k, bool allow_split) {
    (void)dtype;
    TopkPlan p{list_e(k), 1, 1, 0, 0};
    // Short rows and k > 1024: the streaming kernel's list of 2048 per wave
    // holds 64 registers per lane (two waves per SIMD) and compacts after
    // every 512 survivors; a whole row in a workgroup's registers is read
    // once and selected without compactions (measured on 6710 x 16384 rows:
    // faster for k = 2048, slower for k <= 1024).  Enough rows to fill the GPU.
    if (k > 1024 && cols <= kBlockMaxCols && rows >= 256) {
        p.block_kpt = kBlockKeys;
        p.waves = cols <= kBlockMaxCols / 2 ? 4 : 8;
        return p;
    }
    const int64_t lp = (int64_t)kWave * p.e;
    const int64_t want = rows > 0 ? (kTargetWaves + rows - 1) / rows : 1;
    // Pieces long enough that compactions stay a small part of the work: the
    // waves of one workgroup share their threshold through LDS, so their
    // pieces may be shorter than those of separate workgroups, whose lists
    // also go through the workspace and a merge kernel.
    const int64_t wg_piece = lp * 4 > 2048 ? lp * 4 : 2048;
    const int64_t grp_piece = lp * 8 > 6400 ? lp * 8 : 6400;
    const int64_t per_wg = want < cols / wg_piece ? want : cols / wg_piece;
    p.waves = per_wg >= 4 ? 4 : per_wg >= 2 ? 2 : 1;
    if (p.waves == 4 && allow_split) {
        const int64_t by_len = cols / (4 * grp_piece);
        int64_t gr = want / 4 < by_len ? want / 4 : by_len;
        if (gr > 256) gr = 256;
        if (gr >= 2) p.groups = (int)gr;
    }
    // Partial lists stay within kMaxSplitBytes (fewer groups, or none).
    const int64_t list_bytes = lp * (int64_t)sizeof(uint64_t);
    while (p.groups > 1 && rows * p.groups * list_bytes > (int64_t)kMaxSplitBytes) --p.groups;
    if (p.groups > 1) p.ws_bytes = (size_t)rows * p.groups * lp * sizeof(uint64_t);
    return p;
}

// ---------------------------------------------------------------------------
// Scratch of topk_rows_noalloc: the split rows' partial lists live in this
// file-scope device array instead of a caller workspace.  Each device holds
// its own copy at its own address, taken with hipGetSymbolAddress on the
// first call on that device (with the device current) and kept; the array's
// host-side name is never passed to a kernel.  Every list a launch reads was
// written in full by the same launch, so nothing needs clearing; calls that
// overlap on one device share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint64_t scratch[kMaxSplitBytes / sizeof(uint64_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int scratch_of_current_device(void** ptr, size_t* bytes) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return RTS_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return RTS_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return RTS_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = sizeof(scratch);
    return RTS_OK;
}

namespace {

template <int NW, int E, bool BF16>
void launch_block(const void* x, int64_t rows, int64_t cols, int64_t ld, const int32_t* re, int32_t k,
                  int32_t* out, int64_t ld_out, hipStream_t s) {
    hipLaunchKernelGGL((topk_rows_block_kernel<NW, kBlockKeys, E, BF16>), dim3((unsigned)rows),
                       dim3(kWave * NW), 0, s, x, cols, ld, re, k, out, ld_out);
}

// E: sort slots per lane, 64 * NW * E >= k.
template <int NW, bool BF16>
int launch_block_e(const void* x, int64_t rows, int64_t cols, int64_t ld, const int32_t* re, int32_t k,
                   int32_t* out, int64_t ld_out, hipStream_t s) {
    constexpr int S1 = kWave * NW;  // k in (1024, 2048]
    if (k <= 4 * S1 && NW == 8) launch_block<NW, 4, BF16>(x, rows, cols, ld, re, k, out, ld_out, s);
    else if (k <= 8 * S1) launch_block<NW, 8, BF16>(x, rows, cols, ld, re, k, out, ld_out, s);
    else return RTS_EUNSUPPORTED;
    return RTS_OK;
}

int launch_block_rows(bool bf16, int waves, const void* x, int64_t rows, int64_t cols, int64_t ld,
                      const int32_t* re, int32_t k, int32_t* out, int64_t ld_out, hipStream_t s) {
    if (waves == 4)
        return bf16 ? launch_block_e<4, true>(x, rows, cols, ld, re, k, out, ld_out, s)
                    : launch_block_e<4, false>(x, rows, cols, ld, re, k, out, ld_out, s);
    if (waves == 8)
        return bf16 ? launch_block_e<8, true>(x, rows, cols, ld, re, k, out, ld_out, s)
                    : launch_block_e<8, false>(x, rows, cols, ld, re, k, out, ld_out, s);
    return RTS_EUNSUPPORTED;
}

}  // namespace

int launch_topk_rows(const void* logits, int dtype, int64_t rows, int64_t cols, int64_t ld,
                     const int32_t* row_ends, int32_t k, int32_t* out, int64_t ld_out,
                     const TopkPlan& plan, void* workspace, hipStream_t s) {
    if (rows == 0) return RTS_OK;
    const bool bf16 = dtype == RTS_BF16;
    if (plan.block_kpt > 0) {
        const int rc = launch_block_rows(bf16, plan.waves, logits, rows, cols, ld, row_ends, k, out,
                                         ld_out, s);
        if (rc != RTS_OK) return rc;
        return hipGetLastError() == hipSuccess ? RTS_OK : RTS_EHIP;
    }
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
