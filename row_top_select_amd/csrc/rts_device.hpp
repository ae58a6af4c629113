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

// ---------------------------------------------------------------------------
// Lane exchange and reductions.  DPP (row/quad permutes, row broadcasts) and
// ds_swizzle stay out of LDS memory; only a lane xor of 32 uses ds_bpermute.
// DPP control codes of the GFX9 encoding.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowShl4 = 0x104;  // lane i <- lane i+4 (same row of 16)
constexpr int kDppRowShr1 = 0x111;  // lane i <- lane i-1
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowRor8 = 0x128;  // lane i <- lane (i+8) mod 16
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> rows 2 and 3

template <int CTRL, int ROW_MASK = 0xF, bool BOUND = false>
__device__ __forceinline__ uint32_t dpp32(uint32_t old, uint32_t src) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, ROW_MASK, 0xF, BOUND);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp64(uint64_t old, uint64_t src) {
    const uint32_t lo = dpp32<CTRL, ROW_MASK>((uint32_t)old, (uint32_t)src);
    const uint32_t hi = dpp32<CTRL, ROW_MASK>((uint32_t)(old >> 32), (uint32_t)(src >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// v of lane (lane ^ lj), for lj a power of two below 64.
__device__ __forceinline__ uint32_t lane_xor32(uint32_t v, int lj) {
    switch (lj) {
        case 1: return dpp32<kDppQuadXor1>(v, v);
        case 2: return dpp32<kDppQuadXor2>(v, v);
        // ds_swizzle bit mode: lane' = ((lane & 0x1F) | 0) ^ xor within 32 lanes.
        case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);
        case 8: return dpp32<kDppRowRor8>(v, v);
        case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
        default: return (uint32_t)__shfl_xor((int)v, lj, kWave);
    }
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int mask) {
    const uint32_t lo = lane_xor32((uint32_t)v, mask);
    const uint32_t hi = lane_xor32((uint32_t)(v >> 32), mask);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
    uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Lane-wise select by a wave mask: if_set where the lane's bit of m is set.
// One v_cndmask; written out so the compiler cannot turn it into a branch.
__device__ __forceinline__ uint32_t select_by_mask(uint64_t m, uint32_t if_set, uint32_t if_clear) {
    uint32_t r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(m));
    return r;
}

// LDS byte address of a pointer into __shared__ memory, and a two-word store
// at such an address (the words come from any two registers).
typedef __attribute__((address_space(3))) uint32_t lds_u32;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_store2(uint32_t addr, uint32_t lo, uint32_t hi) {
    lds_u32* q = (lds_u32*)(uintptr_t)addr;
    q[0] = lo;
    q[1] = hi;
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
// same lane; farther partners are exchanged with a lane xor.  Which lanes sort
// a pair descending, or keep the larger partner, is a fixed pattern of lane
// bits per stage, so a compare-exchange is one compare, one scalar xor of
// wave masks and a select per word.  Elements are 32-bit keys or 64-bit
// composites (uint32_t or uint64_t arrays).
// ---------------------------------------------------------------------------

// Lanes whose index has bit x set (x a power of two); none for x >= 64.
__device__ __forceinline__ constexpr uint64_t lanes_with_bit(int x) {
    return x == 1    ? 0xAAAAAAAAAAAAAAAAull
           : x == 2  ? 0xCCCCCCCCCCCCCCCCull
           : x == 4  ? 0xF0F0F0F0F0F0F0F0ull
           : x == 8  ? 0xFF00FF00FF00FF00ull
           : x == 16 ? 0xFFFF0000FFFF0000ull
           : x == 32 ? 0xFFFFFFFF00000000ull
                     : 0ull;
}

__device__ __forceinline__ uint64_t select64_by_mask(uint64_t m, uint64_t if_set, uint64_t if_clear) {
    const uint32_t lo = select_by_mask(m, (uint32_t)if_set, (uint32_t)if_clear);
    const uint32_t hi = select_by_mask(m, (uint32_t)(if_set >> 32), (uint32_t)(if_clear >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Lane exchange and select for either element width of the networks below
// (32-bit keys, or 64-bit composites).
__device__ __forceinline__ uint32_t lane_xor_k(uint32_t v, int lj) { return lane_xor32(v, lj); }
__device__ __forceinline__ uint64_t lane_xor_k(uint64_t v, int lj) { return shfl_xor64(v, lj); }
__device__ __forceinline__ uint32_t select_k(uint64_t m, uint32_t if_set, uint32_t if_clear) {
    return select_by_mask(m, if_set, if_clear);
}
__device__ __forceinline__ uint64_t select_k(uint64_t m, uint64_t if_set, uint64_t if_clear) {
    return select64_by_mask(m, if_set, if_clear);
}

// flip = ~0: the whole network sorts descending (a wave-uniform value, so
// the direction may also be chosen at run time).
template <int N, int K, int J, typename U>
__device__ __forceinline__ void bitonic_stage_flip(U (&v)[N], uint64_t flip) {
    // Element i = l*N + r lies in an ascending run iff (i & K) == 0 (the
    // reverse when flipped).  For K >= N that is bit K/N of the lane.
    if constexpr (J < N) {
#pragma unroll
        for (int r = 0; r < N; ++r) {
            if ((r & J) == 0) {
                const uint64_t desc =
                    (K < N ? (((r & K) != 0) ? ~0ull : 0ull) : lanes_with_bit(K / N)) ^ flip;
                const U a = v[r], b = v[r | J];
                // Ascending: swap if a > b; descending: if a < b (equal: either).
                const uint64_t sw = __ballot(a > b) ^ desc;
                v[r] = select_k(sw, b, a);
                v[r | J] = select_k(sw, a, b);
            }
        }
    } else {
        constexpr int LJ = J / N;
        const uint64_t desc = lanes_with_bit(K / N) ^ flip;
        // The lower partner keeps the smaller value in an ascending run.
        const uint64_t keep_max = lanes_with_bit(LJ) ^ desc;
#pragma unroll
        for (int r = 0; r < N; ++r) {
            const U o = lane_xor_k(v[r], LJ);
            const uint64_t take = __ballot(v[r] > o) ^ keep_max;
            v[r] = select_k(take, o, v[r]);
        }
    }
}

// Stages J, J/2, .., 1 of the merge step of size K.
template <int N, int K, int J, typename U>
__device__ __forceinline__ void bitonic_steps(U (&v)[N], uint64_t flip) {
    if constexpr (J >= 1) {
        bitonic_stage_flip<N, K, J>(v, flip);
        bitonic_steps<N, K, J / 2>(v, flip);
    }
}

template <int N, int K, typename U>
__device__ __forceinline__ void bitonic_sort_from(U (&v)[N], uint64_t flip) {
    if constexpr (K <= kWave * N) {
        bitonic_steps<N, K, K / 2>(v, flip);
        bitonic_sort_from<N, K * 2>(v, flip);
    }
}

// Full sort: ascending (DESC=false) or descending.  Every stage is its own
// instantiation, so k and j are constants without relying on loop unrolling.
template <int N, bool DESC, typename U>
__device__ __forceinline__ void wave_bitonic_sort(U (&v)[N]) {
    bitonic_sort_from<N, 2>(v, DESC ? ~0ull : 0ull);
}

// Sorts a bitonic sequence (e.g. the elementwise max of a descending and an
// ascending sorted sequence).
template <int N, bool DESC, typename U>
__device__ __forceinline__ void wave_bitonic_merge(U (&v)[N]) {
    bitonic_steps<N, kWave * N, kWave * N / 2>(v, DESC ? ~0ull : 0ull);
}

// The same, with the direction a wave-uniform run-time value (read from the
// first lane, so the masks derived from it stay scalar).
__device__ __forceinline__ uint64_t uniform_flip(bool desc) {
    const uint32_t f = (uint32_t)__builtin_amdgcn_readfirstlane(desc ? -1 : 0);
    return ((uint64_t)f << 32) | f;
}
template <int N, typename U>
__device__ __forceinline__ void wave_bitonic_sort_dir(U (&v)[N], bool desc) {
    bitonic_sort_from<N, 2>(v, uniform_flip(desc));
}
template <int N, typename U>
__device__ __forceinline__ void wave_bitonic_merge_dir(U (&v)[N], bool desc) {
    bitonic_steps<N, kWave * N, kWave * N / 2>(v, uniform_flip(desc));
}

// ---------------------------------------------------------------------------
// Wave reductions (result uniform, read from lane 63) and inclusive scan.
// Steps: quad xor 1 and 2, half-row and row mirrors (each row of 16 then holds
// its total), row 15 -> rows 1/3, lane 31 -> rows 2/3.
// ---------------------------------------------------------------------------
template <typename Op>
__device__ __forceinline__ uint64_t wave_reduce64(uint64_t v, Op op) {
    v = op(v, dpp64<kDppQuadXor1>(v, v));
    v = op(v, dpp64<kDppQuadXor2>(v, v));
    v = op(v, dpp64<kDppRowHalfMirror>(v, v));
    v = op(v, dpp64<kDppRowMirror>(v, v));
    v = op(v, dpp64<kDppRowBcast15, 0xA>(v, v));
    v = op(v, dpp64<kDppRowBcast31, 0xC>(v, v));
    return readlane64(v, kWave - 1);
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce32(uint32_t v, Op op) {
    v = op(v, dpp32<kDppQuadXor1>(v, v));
    v = op(v, dpp32<kDppQuadXor2>(v, v));
    v = op(v, dpp32<kDppRowHalfMirror>(v, v));
    v = op(v, dpp32<kDppRowMirror>(v, v));
    v = op(v, dpp32<kDppRowBcast15, 0xA>(v, v));
    v = op(v, dpp32<kDppRowBcast31, 0xC>(v, v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_sum32(uint32_t v) {
    return wave_reduce32(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_or32(uint32_t v) {
    return wave_reduce32(v, [](uint32_t a, uint32_t b) { return a | b; });
}
__device__ __forceinline__ uint32_t wave_max32(uint32_t v) {
    return wave_reduce32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min32(uint32_t v) {
    return wave_reduce32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint64_t wave_min64(uint64_t v) {
    return wave_reduce64(v, [](uint64_t a, uint64_t b) { return umin64(a, b); });
}
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
    return wave_reduce64(v, [](uint64_t a, uint64_t b) { return umax64(a, b); });
}

// Inclusive prefix sum over the wave (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan32(uint32_t v) {
    v += dpp32<kDppRowShr1, 0xF, true>(0u, v);
    v += dpp32<kDppRowShr2, 0xF, true>(0u, v);
    v += dpp32<kDppRowShr4, 0xF, true>(0u, v);
    v += dpp32<kDppRowShr8, 0xF, true>(0u, v);
    v += dpp32<kDppRowBcast15, 0xA>(0u, v);
    v += dpp32<kDppRowBcast31, 0xC>(0u, v);
    return v;
}

// ---------------------------------------------------------------------------
// Radix-select step over 256 wave-private LDS bins (bin b counts the entries of
// its digit).
// ---------------------------------------------------------------------------
// Scans the bins from the top: finds the bin where the running count reaches
// need, lowers need by the count above it and returns the bin and its count
// (uniform).  False only if the counts were inconsistent.  c[j] is the count
// of bin 255 - 4 * lane - j (lane l owns bins 255-4l .. 252-4l).
__device__ __forceinline__ bool radix_find_counts(const uint32_t (&c)[4], int& need, uint32_t& bin,
                                                  uint32_t& cb) {
    const uint32_t tot = c[0] + c[1] + c[2] + c[3];
    uint32_t run = wave_incl_scan32(tot) - tot;
    int fj = -1;
    uint32_t above = 0, cl = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (fj < 0 && run < (uint32_t)need && run + c[j] >= (uint32_t)need) {
            fj = j;
            above = run;
            cl = c[j];
        }
        run += c[j];
    }
    wave_lds_sync();  // the next level clears the bins
    const uint64_t fm = __ballot(fj >= 0);
    if (fm == 0ull) return false;
    const int fl = __ffsll((long long)fm) - 1;
    bin = 255u - 4u * (uint32_t)fl - (uint32_t)__builtin_amdgcn_readlane(fj, fl);
    need -= (int)__builtin_amdgcn_readlane(above, fl);
    cb = __builtin_amdgcn_readlane(cl, fl);
    return true;
}

// radix_find over one 256-bin table.
__device__ __forceinline__ bool radix_find(const uint32_t* hist, int& need, uint32_t& bin,
                                           uint32_t& cb) {
    const int lane = lane_id();
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = hist[255 - 4 * lane - j];
    return radix_find_counts(c, need, bin, cb);
}

// ---------------------------------------------------------------------------
// Wave-private 256-bin histogram in NS lane-striped copies: lane l counts
// into copy l % NS, so lanes that share a bin mostly hit different
// addresses.  Copies are kStripeStride words apart (16-byte aligned, each
// copy's banks shifted by 4).
// ---------------------------------------------------------------------------
constexpr int kStripes = 4;
constexpr int kStripeStride = 260;
constexpr int kStripedWords = kStripes * kStripeStride;

// Stripe count that fits `words` words of LDS: a power of two, at most 8.
constexpr int stripes_fitting(int words) {
    return words >= 8 * kStripeStride ? 8 : words >= 4 * kStripeStride ? 4 : words >= 2 * kStripeStride ? 2 : 1;
}

// Each store covers one whole copy (64 lanes x 16 B).
template <int NS = kStripes>
__device__ __forceinline__ void striped_clear(uint32_t* hist) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const int lane = lane_id();
#pragma unroll
    for (int c = 0; c < NS; ++c)
        *reinterpret_cast<u32x4_t*>(hist + c * kStripeStride + 4 * lane) = u32x4_t{0u, 0u, 0u, 0u};
}

// This lane's copy.
template <int NS = kStripes>
__device__ __forceinline__ uint32_t* striped_copy(uint32_t* hist) {
    return hist + (lane_id() & (NS - 1)) * kStripeStride;
}

template <int NS = kStripes>
__device__ __forceinline__ void striped_add(uint32_t* hist, uint32_t bin) {
    __hip_atomic_fetch_add(&striped_copy<NS>(hist)[bin], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// radix_find over the sum of the striped copies.
template <int NS = kStripes>
__device__ __forceinline__ bool striped_find(const uint32_t* hist, int& need, uint32_t& bin,
                                             uint32_t& cb) {
    const int lane = lane_id();
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    // bins 252-4l .. 255-4l: one 16-byte read per copy, the copies summed
    // one after the other (a real loop: the callers hold many registers)
    u32x4_t acc = *reinterpret_cast<const u32x4_t*>(hist + 252 - 4 * lane);
#pragma unroll 1
    for (int s = 1; s < NS; ++s)
        acc += *reinterpret_cast<const u32x4_t*>(hist + s * kStripeStride + 252 - 4 * lane);
    const uint32_t c[4] = {acc[3], acc[2], acc[1], acc[0]};
    return radix_find_counts(c, need, bin, cb);
}

}  // namespace rts
