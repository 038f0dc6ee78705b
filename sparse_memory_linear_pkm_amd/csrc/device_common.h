// device_common.h -- small gfx950 device helpers shared by the SDM kernels.
// (Kernel-side only; nothing here is used by the CPU oracle.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Buffer resource word 3 for raw (untyped) buffer access on gfx9 parts.
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kBufferRsrcWord3);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h)
{
    return __uint_as_float((uint32_t)h << 16);
}

// Total order used by every selection: score descending, then index
// ascending.  key = (monotone bits of score) << 32 | ~index, so a larger key
// is a better candidate.  -0.0 is folded into +0.0 first so that the order
// agrees with IEEE comparison (where the two are equal).  Finite scores map
// to keys > 0; key 0 means "no candidate".
__device__ __forceinline__ uint64_t score_key(float s, uint32_t idx)
{
    s = s + 0.0f;
    uint32_t u = __float_as_uint(s);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(~idx);
}

__device__ __forceinline__ float key_score(uint64_t key)
{
    uint32_t u = (uint32_t)(key >> 32);
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) { return ~(uint32_t)key; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m)
{
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    lo = (uint32_t)__shfl_xor((int)lo, m, kWave);
    hi = (uint32_t)__shfl_xor((int)hi, m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l)
{
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        uint64_t y = shfl_xor_u64(x, m);
        x = y > x ? y : x;
    }
    return x;
}

__device__ __forceinline__ int wave_sum_i32(int x)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

__device__ __forceinline__ float wave_sum_f32(float x)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// Exclusive prefix sum across the wave.
__device__ __forceinline__ int wave_excl_prefix_i32(int x)
{
    const int lane = lane_id();
    int incl = x;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        int y = __shfl_up(incl, m, kWave);
        if (lane >= m) incl += y;
    }
    return incl - x;
}

// Bitonic sort of one key per lane, descending across lanes 0..63.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key)
{
    const int lane = lane_id();
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t other = shfl_xor_u64(key, j);
            const bool lower = (lane & j) == 0;
            const bool desc_block = (lane & k) == 0;
            const bool keep_max = (lower == desc_block);
            const uint64_t mx = key > other ? key : other;
            const uint64_t mn = key > other ? other : key;
            key = keep_max ? mx : mn;
        }
    }
    return key;
}

// Exact top-n (n <= 64) of `len` candidates, one wave.  get(p) returns the key
// of candidate p (p in [0, len)); keys are unique and > 0.  On return lane j
// (j < n) holds the j-th best key, sorted descending; other lanes hold 0.
// lds_scratch: 64 uint64 of per-wave LDS.
//
// Method: the n-th largest of the 64 per-lane maxima is a lower bound tau
// with at least n candidates >= tau; the candidates >= tau are compacted and
// sorted when they fit in one wave, otherwise the n best are extracted one by
// one (exact in both cases).
template <class Get>
__device__ __forceinline__ uint64_t wave_topn(int len, int n, Get get, uint64_t *lds_scratch)
{
    const int lane = lane_id();
    uint64_t lmax = 0;
    for (int p = lane; p < len; p += kWave) {
        uint64_t k = get(p);
        lmax = k > lmax ? k : lmax;
    }
    const uint64_t sorted_max = wave_sort_desc(lmax);
    const uint64_t tau = readlane_u64(sorted_max, n - 1);
    int cnt = 0;
    for (int p = lane; p < len; p += kWave) cnt += get(p) >= tau ? 1 : 0;
    const int total = wave_sum_i32(cnt);
    uint64_t result = 0;
    if (total <= kWave) {
        int pos = wave_excl_prefix_i32(cnt);
        for (int p = lane; p < len; p += kWave) {
            uint64_t k = get(p);
            if (k >= tau) lds_scratch[pos++] = k;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint64_t mine = lane < total ? lds_scratch[lane] : 0;
        __builtin_amdgcn_wave_barrier();
        result = wave_sort_desc(mine);
        if (lane >= n) result = 0;
    } else {
        uint64_t prev = ~0ull;
        for (int j = 0; j < n; ++j) {
            uint64_t best = 0;
            for (int p = lane; p < len; p += kWave) {
                uint64_t k = get(p);
                if (k < prev && k > best) best = k;
            }
            best = wave_max_u64(best);
            if (lane == j) result = best;
            prev = best;
        }
    }
    return result;
}

}  // namespace sdm
