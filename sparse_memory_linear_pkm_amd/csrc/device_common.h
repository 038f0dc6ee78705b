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
// ascending.  score_bits maps a float to an unsigned integer in the same
// order (-0.0 is folded into +0.0 first, so that equal floats map to equal
// bits), and key = score_bits << 32 | ~index, so a larger key is a better
// candidate.  Finite scores have score_bits > 0, so key 0 means "no
// candidate".
__device__ __forceinline__ uint32_t score_bits(float s)
{
    s = s + 0.0f;
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t score_key(float s, uint32_t idx)
{
    return ((uint64_t)score_bits(s) << 32) | (uint64_t)(~idx);
}

__device__ __forceinline__ float key_score(uint64_t key)
{
    uint32_t u = (uint32_t)(key >> 32);
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) { return ~(uint32_t)key; }

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l)
{
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int mbcnt64(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Orders LDS accesses among the lanes of one wave (a write by one lane, then
// a read of it by another).  The LDS executes one wave's instructions in
// issue order, so only the compiler must be kept from reordering; a memory
// fence here would also make the compiler wait for outstanding loads that
// target LDS directly (buffer_load ... lds), which never alias these arrays.
__device__ __forceinline__ void wave_lds_sync()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Lane exchanges on the VALU (no LDS crossbar): x[lane ^ J] for J = 1..32.
// DPP quad_perm for 1 and 2, row_shl:4 / row_shr:4 for 4, row_ror:8 for 8,
// and the gfx950 v_permlane16_swap / v_permlane32_swap for 16 and 32.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x)
{
    static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32, "xor distance");
    // mov_dpp has no "old" operand to initialise; every lane that is selected
    // below reads a valid source lane
    const int xi = (int)x;
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    } else if constexpr (J == 4) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x104, 0xF, 0xF, true);  // row_shl:4
        const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x114, 0xF, 0xF, true);  // row_shr:4
        return (lane_id() & 4) ? dn : up;
    } else if constexpr (J == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x128, 0xF, 0xF, true);  // row_ror:8
    } else if constexpr (J == 16) {
        const auto s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane_id() & 16) ? s[0] : s[1];
    } else {
        const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane_id() & 32) ? s[0] : s[1];
    }
}

template <int J>
__device__ __forceinline__ uint64_t lane_xor(uint64_t x)
{
    const uint32_t lo = lane_xor<J>((uint32_t)x), hi = lane_xor<J>((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Butterfly sum across the wave.  Every lane ends with the same value, and
// the order of additions is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum_f32(float x)
{
    x += __uint_as_float(lane_xor<1>(__float_as_uint(x)));
    x += __uint_as_float(lane_xor<2>(__float_as_uint(x)));
    x += __uint_as_float(lane_xor<4>(__float_as_uint(x)));
    x += __uint_as_float(lane_xor<8>(__float_as_uint(x)));
    x += __uint_as_float(lane_xor<16>(__float_as_uint(x)));
    x += __uint_as_float(lane_xor<32>(__float_as_uint(x)));
    return x;
}

template <class T>
__device__ __forceinline__ T wave_max(T x)
{
    T y;
    y = lane_xor<1>(x);  x = y > x ? y : x;
    y = lane_xor<2>(x);  x = y > x ? y : x;
    y = lane_xor<4>(x);  x = y > x ? y : x;
    y = lane_xor<8>(x);  x = y > x ? y : x;
    y = lane_xor<16>(x); x = y > x ? y : x;
    y = lane_xor<32>(x); x = y > x ? y : x;
    return x;
}

// Descending bitonic sort across the 64 lanes of NR independent values per
// lane (NR sorts interleaved, so their dependency chains overlap).  One
// compare-exchange stage: block size K, partner distance J.
template <int K, int J, int NR, class T>
__device__ __forceinline__ void bitonic_stage(T (&x)[NR])
{
    if constexpr (J >= 1) {
        const int lane = lane_id();
        const bool keep_max = ((lane & J) == 0) == ((lane & K) == 0);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const T other = lane_xor<J>(x[r]);
            // equal values: taking either is the same
            const bool take = (other > x[r]) == keep_max;
            x[r] = take ? other : x[r];
        }
        bitonic_stage<K, J / 2, NR>(x);
    }
}

template <int K, int WIDTH, int NR, class T>
__device__ __forceinline__ void bitonic_from(T (&x)[NR])
{
    if constexpr (K <= WIDTH) {
        bitonic_stage<K, K / 2, NR>(x);
        bitonic_from<K * 2, WIDTH, NR>(x);
    }
}

// Sorts lanes [0, WIDTH) of each of the NR values descending (WIDTH = 32
// also sorts lanes 32..63 among themselves, ascending; callers that use it
// keep every candidate in lanes 0..31).
template <int NR, int WIDTH = kWave, class T>
__device__ __forceinline__ void wave_sort_desc(T (&x)[NR])
{
    static_assert(WIDTH == 32 || WIDTH == 64, "sort width");
    bitonic_from<2, WIDTH, NR>(x);
}

// Exact top-n (1 <= n <= 64, n <= len) of `len` candidates for each of NR
// independent rows, one wave.  get(r, p) returns the key of candidate p of
// row r (p in [0, len)); the keys of a row are distinct and > 0.  On return
// lane j < n of res[r] holds the j-th best key of row r (descending); the
// other lanes hold 0.  scratch: NR * 64 uint64 of this wave's LDS.
//
// len <= 64: the candidates are sorted directly (one per lane).  Otherwise,
// per row: tau = the n-th largest per-lane maximum score (compared on the
// score bits only) bounds the answer from below, since at least n candidates
// (one per lane above it) reach it; the candidates whose score reaches tau
// are compacted with ballots and sorted as 64-bit keys (over 32 lanes when
// every row has at most 32 of them).  When more than 64 reach tau (ties, or
// n close to 64), that row is instead extracted one best key at a time,
// which is exact as well.
//
// idx_bits > 0 declares that every key's low word is ~i for an index
// i < 2^idx_bits; the survivors of a row are then sorted as 32-bit keys
// ((score bits - tau + 1) << idx_bits | (2^idx_bits - 1 - i)), the same
// order exactly, whenever every row's score bits above tau fit in the
// remaining high bits (else as 64-bit keys).
template <int NR, class Get>
__device__ __forceinline__ void wave_topn(int len, int n, Get get, uint64_t *scratch,
                                          uint64_t (&res)[NR], int idx_bits = 0)
{
    const int lane = lane_id();
    if (len <= kWave) {
        uint64_t c[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) c[r] = lane < len ? get(r, lane) : 0ull;
        if (len <= 32)
            wave_sort_desc<NR, 32>(c);
        else
            wave_sort_desc<NR, 64>(c);
#pragma unroll
        for (int r = 0; r < NR; ++r) res[r] = lane < n ? c[r] : 0ull;
        return;
    }
    // the candidates are read kBatch per lane at a time (clamped positions,
    // masked values), so that their LDS reads are in flight together
    constexpr int kBatch = 8;
    uint32_t m[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) m[r] = 0;
    for (int p0 = 0; p0 < len; p0 += kBatch * kWave) {
        uint32_t hv[kBatch][NR];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int p = p0 + b * kWave + lane;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint32_t hi = (uint32_t)(get(r, p < len ? p : len - 1) >> 32);
                hv[b][r] = p < len ? hi : 0u;
            }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
#pragma unroll
            for (int r = 0; r < NR; ++r) m[r] = hv[b][r] > m[r] ? hv[b][r] : m[r];
    }
    wave_sort_desc<NR>(m);
    uint32_t tau[NR];
    int total[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        tau[r] = (uint32_t)__builtin_amdgcn_readlane((int)m[r], n - 1);
        total[r] = 0;
    }
    const int iters = (len + kWave - 1) / kWave;
    for (int i0 = 0; i0 < iters; i0 += kBatch) {
        uint64_t kv[kBatch][NR];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int p = lane + (i0 + b) * kWave;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint64_t k = get(r, p < len ? p : len - 1);
                kv[b][r] = p < len ? k : 0ull;
            }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (i0 + b < iters) {   // uniform
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const uint64_t k = kv[b][r];
                    const bool f = (uint32_t)(k >> 32) >= tau[r];   // tau > 0, so k != 0
                    const uint64_t ball = __ballot(f);
                    const int pos = total[r] + mbcnt64(ball);
                    if (f && pos < kWave) scratch[r * kWave + pos] = k;
                    total[r] += __popcll(ball);
                }
            }
        }
    }
    wave_lds_sync();
    uint64_t c[NR];
    int most = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        c[r] = lane < total[r] ? scratch[r * kWave + lane] : 0ull;
        most = total[r] > most ? total[r] : most;
    }
    __builtin_amdgcn_wave_barrier();
    // 32-bit keys when every row's score range above tau fits
    bool narrow = idx_bits > 0;
    uint32_t span[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const uint32_t top = (uint32_t)__builtin_amdgcn_readlane((int)m[r], 0);   // the row's best score bits
        span[r] = top - tau[r] + 1u;
        narrow = narrow && (uint64_t)span[r] < (1ull << (32 - idx_bits));
    }
    if (narrow) {
        const uint32_t imask = (1u << idx_bits) - 1u;
        uint32_t c32[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint32_t hi = (uint32_t)(c[r] >> 32), i = ~(uint32_t)c[r];
            c32[r] = c[r] ? ((hi - tau[r] + 1u) << idx_bits) | (imask - i) : 0u;
        }
        if (most <= 32 && n <= 32)
            wave_sort_desc<NR, 32>(c32);
        else
            wave_sort_desc<NR, 64>(c32);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint32_t hi = (c32[r] >> idx_bits) + tau[r] - 1u, i = imask - (c32[r] & imask);
            c[r] = c32[r] ? ((uint64_t)hi << 32) | (uint32_t)~i : 0ull;
        }
    } else if (most <= 32 && n <= 32) {
        wave_sort_desc<NR, 32>(c);
    } else {
        wave_sort_desc<NR, 64>(c);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        res[r] = lane < n ? c[r] : 0ull;
        if (total[r] > kWave) {
            uint64_t prev = ~0ull, out = 0;
            for (int j = 0; j < n; ++j) {
                uint64_t best = 0;
                for (int p = lane; p < len; p += kWave) {
                    const uint64_t k = get(r, p);
                    best = (k < prev && k > best) ? k : best;
                }
                best = wave_max(best);
                out = lane == j ? best : out;
                prev = best;
            }
            res[r] = out;
        }
    }
}

}  // namespace sdm
