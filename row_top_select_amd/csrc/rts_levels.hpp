// Workgroup radix-select levels over 32-bit keys held or visited by every
// thread of a workgroup, shared by the pair select and the short-row top-k
// (gfx950, wave64).
//
// A visitor hands out this thread's entries: visit(f) calls f(key, id) for
// each, key 0 meaning empty.  A level counts the keys of a window
// [wlo, wlo + span] into 256 bins of width 2^sh (atomics into lane-striped LDS
// copies), then wave 0 finds the bin where the count from the top reaches
// `need`.  The levels end with either a plain threshold (the selected keys are
// those > thr_gt) or ties at one key, of which the `need` smallest ids are
// selected.  The workgroup's shared memory type Smem provides
// hist[kLevelCopies][kLevelStride], bins[256], bc[4], tied[64] and ntied.
#pragma once

#include <type_traits>

#include "rts_device.hpp"

namespace rts {

constexpr int kLevelCopies = 8;
constexpr int kLevelStride = 257;

// Workgroup barrier that orders LDS traffic only (a plain __syncthreads also
// waits for every outstanding vector-memory access of the wave).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Counts key - wlo, when it lies in [0, span], into bin (key - wlo) >> sh.
template <typename Smem>
__device__ __forceinline__ void level_hist_add(Smem& sm, uint32_t key, uint32_t wlo,
                                              uint32_t span, uint32_t sh) {
    const uint32_t x = key - wlo;
    if (x <= span)
        __hip_atomic_fetch_add(&sm.hist[lane_id() & (kLevelCopies - 1)][x >> sh], 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Smem types that set kWave0Find = true take level_hist_find's two-barrier
// form (wave 0 alone sums the copies); the others the four-barrier form
// (every thread sums a few bins), which holds fewer registers in wave 0.
template <typename S, typename = void>
struct Wave0Find : std::false_type {};
template <typename S>
struct Wave0Find<S, std::void_t<decltype(S::kWave0Find)>> : std::integral_constant<bool, S::kWave0Find> {};

// All threads, after their level_hist_add calls: sums (and clears, for the
// next level) the copies, then wave 0 finds the bin where the count from the
// top reaches need.  Returns (uniform) ok, the bin and its count, and lowers
// need by the count above the bin.
template <typename Smem>
__device__ __forceinline__ bool level_hist_find(Smem& sm, int& need, uint32_t& bin, uint32_t& cb) {
    const int lane = lane_id();
    lds_barrier();
    if constexpr (Wave0Find<Smem>::value) {
        // Two barriers: the result words are next written by wave 0 after
        // the following level's first barrier, which every wave reaches only
        // once it has read them.
        if (threadIdx.x < (unsigned)kWave) {
            // One bin at a time: the caller's keys are live in registers here.
#pragma unroll 1
            for (int q = 0; q < 4; ++q) {
                const int b = lane + q * kWave;
                uint32_t t = 0;
#pragma unroll
                for (int c = 0; c < kLevelCopies; ++c) {
                    t += sm.hist[c][b];
                    sm.hist[c][b] = 0u;
                }
                sm.bins[b] = t;
            }
            wave_lds_sync();
        }
    } else {
        for (int b = threadIdx.x; b < 256; b += blockDim.x) {  // the block may have < 256 threads
            uint32_t t = 0;
#pragma unroll
            for (int c = 0; c < kLevelCopies; ++c) {
                t += sm.hist[c][b];
                sm.hist[c][b] = 0u;
            }
            sm.bins[b] = t;
        }
        lds_barrier();
    }
    if (threadIdx.x < (unsigned)kWave) {
        int nd = need;
        uint32_t b, c;
        const bool ok = radix_find(sm.bins, nd, b, c);
        if (lane == 0) {
            sm.bc[0] = ok ? 1u : 0u;
            sm.bc[1] = b;
            sm.bc[2] = c;
            sm.bc[3] = (uint32_t)nd;
        }
    }
    lds_barrier();
    const bool ok = sm.bc[0] != 0u;
    bin = sm.bc[1];
    cb = sm.bc[2];
    if (ok) need = (int)sm.bc[3];
    if constexpr (!Wave0Find<Smem>::value) lds_barrier();  // sm.bc is rewritten by the next level
    return ok;
}

// Radix levels over the keys that `visit` hands out (visit(f) calls
// f(key, id) for each of this thread's entries), starting from the window
// [wlo, wlo + span] in bins of 2^sh: ends with either a plain threshold (the
// k selected are the keys > thr_gt) or ties at tie_key, ntie of them, of which
// the `need` lowest ids are selected.
template <typename Smem, typename Visit>
__device__ __forceinline__ void radix_levels(Smem& sm, Visit visit, int& need, uint32_t wlo,
                                            uint32_t span, uint32_t sh, uint32_t mx, uint32_t& thr_gt,
                                            bool& ties, uint32_t& tie_key, uint32_t& ntie) {
    ties = false;
    tie_key = 0u;
    ntie = 0u;
    thr_gt = wlo - 1u;
#pragma unroll 1
    for (int level = 0; level < 4; ++level) {  // a 32-bit key needs four at most
        visit([&](uint32_t key, uint32_t) __attribute__((always_inline)) { level_hist_add(sm, key, wlo, span, sh); });
        uint32_t bin, cb;
        if (!level_hist_find(sm, need, bin, cb)) {
            thr_gt = wlo - 1u;
            return;
        }
        const uint32_t blo = wlo + (bin << sh);
        if ((int)cb == need) {
            thr_gt = blo - 1u;
            return;
        }
        if (sh == 0) {
            thr_gt = blo;
            tie_key = blo;
            ties = true;
            ntie = cb;
            return;
        }
        wlo = blo;
        const uint32_t top = mx - blo, width1 = (1u << sh) - 1u;
        span = width1 < top ? width1 : top;
        sh = sh > 8 ? sh - 8 : 0u;
    }
}

// The largest id taken among the ntie entries with key == tie_key, when the
// `need` lowest ids are taken (ids at most id_hi < 2^31): a wave sort for up
// to 64, else levels over id_hi - id.
template <typename Smem, typename Visit>
__device__ __forceinline__ uint32_t tie_cut(Smem& sm, Visit visit, uint32_t tie_key,
                                                 uint32_t ntie, int need,
                                                 uint32_t id_hi = 0x7FFFFFFFu) {
    const int lane = lane_id();
    if (ntie <= (uint32_t)kWave) {
        visit([&](uint32_t key, uint32_t id) __attribute__((always_inline)) {
            if (key == tie_key) {
                const uint32_t s = __hip_atomic_fetch_add(&sm.ntied, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_WORKGROUP);
                if (s < (uint32_t)kWave) sm.tied[s] = id;
            }
        });
        lds_barrier();
        if (threadIdx.x < (unsigned)kWave) {
            uint64_t sv[1] = {lane < (int)ntie ? (uint64_t)sm.tied[lane] : ~0ull};
            wave_bitonic_sort<1, false>(sv);
            const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)sv[0], need - 1);
            if (lane == 0) {
                sm.bc[0] = c;
                sm.ntied = 0u;
            }
        }
        lds_barrier();
        const uint32_t cut = sm.bc[0];
        lds_barrier();
        return cut;
    }
    uint32_t gw = 0u, gspan = id_hi;
    const int gbl = gspan ? 32 - __clz((int)gspan) : 0;
    uint32_t gs = gbl > 8 ? (uint32_t)(gbl - 8) : 0u;
#pragma unroll 1
    for (int gl = 0; gl < 4; ++gl) {
        visit([&](uint32_t key, uint32_t id) __attribute__((always_inline)) {
            if (key == tie_key) level_hist_add(sm, id_hi - id, gw, gspan, gs);
        });
        uint32_t gbin, gcb;
        if (!level_hist_find(sm, need, gbin, gcb)) break;
        gw += gbin << gs;
        if ((int)gcb == need || gs == 0) break;
        const uint32_t top = id_hi - gw, width = (1u << gs) - 1u;
        gspan = width < top ? width : top;
        gs = gs > 8 ? gs - 8 : 0u;
    }
    return id_hi - gw;
}

}  // namespace rts
