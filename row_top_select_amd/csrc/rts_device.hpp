// Device building blocks shared by the row top-K and merge kernels (gfx950,
// wave64).  Keys are 64-bit composites that order candidates under
// (score desc, id asc) as plain unsigned integers:
//
//   composite = (key32(score) << 32) | (0xFFFFFFFF - id),  0 = empty slot
//
// key32 is the order-preserving map of an IEEE binary32 bit pattern (the
// 32-bit form of the bf16 key of the kernels page, section "_ord16": flip a
// negative value, set the sign bit of a non-negative one), so -0 sorts just
// below +0 and every non-NaN value has key32 >= key32(-inf) = 0x007FFFFF > 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rts {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t key32_of_bits(uint32_t u) {
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Inverse of key32_of_bits: the float whose key is k.
__device__ __forceinline__ float float_of_key32(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ bool f32_bits_is_nan(uint32_t u) {
    return (u & 0x7FFFFFFFu) > 0x7F800000u;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t id) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

__device__ __forceinline__ uint32_t composite_id(uint64_t c) {
    return 0xFFFFFFFFu - (uint32_t)c;
}

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int mask) {
    int lo = __shfl_xor((int)(uint32_t)v, mask, kWave);
    int hi = __shfl_xor((int)(uint32_t)(v >> 32), mask, kWave);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
    uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a < b ? b : a; }

// Orders LDS traffic of one wave (lanes exchanging data through LDS without a
// workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Bitonic network over 64*N values held "blocked" by one wave: lane l holds
// elements l*N .. l*N+N-1 in v[0..N-1].  Partners closer than N are in the
// same lane; farther partners are exchanged with a lane xor.
// ---------------------------------------------------------------------------
template <int N, bool DESC>
__device__ __forceinline__ void bitonic_stage(uint64_t (&v)[N], int lane, int k, int j) {
    if (j < N) {
#pragma unroll
        for (int r = 0; r < N; ++r) {
            if ((r & j) == 0) {
                const int i = lane * N + r;
                const bool up = ((i & k) == 0) != DESC;
                const uint64_t a = v[r], b = v[r | j];
                const bool sw = up ? (a > b) : (a < b);
                v[r] = sw ? b : a;
                v[r | j] = sw ? a : b;
            }
        }
    } else {
        const int lj = j / N;
        const bool lower = (lane & lj) == 0;
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const uint64_t o = shfl_xor64(v[r], lj);
            const int i = lane * N + r;
            const bool up = ((i & k) == 0) != DESC;
            v[r] = (lower == up) ? umin64(v[r], o) : umax64(v[r], o);
        }
    }
}

// Full sort: ascending (DESC=false) or descending.
template <int N, bool DESC>
__device__ __forceinline__ void wave_bitonic_sort(uint64_t (&v)[N]) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 2; k <= kWave * N; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) bitonic_stage<N, DESC>(v, lane, k, j);
    }
}

// Sorts a bitonic sequence (e.g. the elementwise max of a descending and an
// ascending sorted sequence).
template <int N, bool DESC>
__device__ __forceinline__ void wave_bitonic_merge(uint64_t (&v)[N]) {
    const int lane = lane_id();
#pragma unroll
    for (int j = (kWave * N) >> 1; j > 0; j >>= 1) bitonic_stage<N, DESC>(v, lane, kWave * N, j);
}

// ---------------------------------------------------------------------------
// Wave reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_sum32(uint32_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v += (uint32_t)__shfl_xor((int)v, d, kWave);
    return v;
}

__device__ __forceinline__ uint32_t wave_or32(uint32_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v |= (uint32_t)__shfl_xor((int)v, d, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_and64(uint64_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v &= shfl_xor64(v, d);
    return v;
}

__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v |= shfl_xor64(v, d);
    return v;
}

__device__ __forceinline__ uint64_t wave_min64(uint64_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v = umin64(v, shfl_xor64(v, d));
    return v;
}

// Inclusive prefix sum over one wave.
__device__ __forceinline__ uint32_t wave_incl_scan32(uint32_t v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        uint32_t t = (uint32_t)__shfl_up((int)v, d, kWave);
        if (lane >= d) v += t;
    }
    return v;
}

}  // namespace rts
