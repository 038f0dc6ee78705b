// scan_lanes.h -- the per-row arithmetic of the sparse gated delta rule in
// the lane layout shared by the prefill scan (sdm_scan_lanes.hip) and the
// decode step (sdm_decode.hip), so that both compute every value with the
// same operations in the same order.
//
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 steps 2-3 (Eq. 4):
//     p = sum_j w_j M[s_j];  M[s_j] = a M[s_j] + b w_j (v - a p);
//     o = sum_j r_j M[s'_j]  (after the write).
// Layout: an aligned group of Q lanes (Q a power of two >= W, R) holds one
// 16-byte column chunk of one token's rows, lane j of the group row j of the
// write list and row j of the read list (lanes past W or R hold zero rows
// with zero weight, which add exactly +0 to the sums).
#pragma once

#include "device_common.h"

namespace sdm {

// x + x[DPP-selected lane] on each component
template <int C>
__device__ __forceinline__ f32x4 add_dpp(f32x4 x)
{
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        r[e] = x[e] + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[e]), C, 0xF, 0xF, true));
    return r;
}

// Sum over the aligned group of Q lanes that holds this lane, left in every
// lane of the group.  Each stage adds two partial sums that cover disjoint
// halves of the stage's lane block, and both partners of a pair add the
// same two values, so every lane of the group ends with the same bits.
template <int Q>
__device__ __forceinline__ f32x4 group_sum(f32x4 x)
{
    static_assert(Q == 1 || Q == 2 || Q == 4 || Q == 8 || Q == 16 || Q == 32 || Q == 64, "group size");
    if constexpr (Q >= 2) x = add_dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (Q >= 4) x = add_dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (Q >= 8) x = add_dpp<0x141>(x);   // row_half_mirror: lane ^ 7 within 8
    if constexpr (Q >= 16) x = add_dpp<0x140>(x);  // row_mirror: lane ^ 15 within 16
    if constexpr (Q >= 32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[e]), __float_as_uint(x[e]), false, false);
            x[e] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
        }
    }
    if constexpr (Q >= 64) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[e]), __float_as_uint(x[e]), false, false);
            x[e] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
        }
    }
    return x;
}

__device__ __forceinline__ f32x4 mul4(float s, f32x4 x) { return (f32x4){s * x.x, s * x.y, s * x.z, s * x.w}; }

// p (or o): the weighted sum of the group's rows
template <int Q>
__device__ __forceinline__ f32x4 weighted_rows(float w, f32x4 x)
{
    return group_sum<Q>(mul4(w, x));
}

// Bitwise OR over the aligned group of Q lanes that holds this lane, left in
// every lane of the group.
template <int Q>
__device__ __forceinline__ uint32_t group_or(uint32_t x)
{
    if constexpr (Q >= 2) x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);
    if constexpr (Q >= 4) x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);
    if constexpr (Q >= 8) x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, true);
    if constexpr (Q >= 16) x |= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, true);
    if constexpr (Q >= 32) {
        const auto s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        x = s[0] | s[1];
    }
    if constexpr (Q >= 64) {
        const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        x = s[0] | s[1];
    }
    return x;
}

// The new value of a written row x with weight w: a x + bw (v - a p), where
// bw = b * w (one fp32 product, formed by the caller).
__device__ __forceinline__ f32x4 written_row(f32x4 x, float a, float bw, f32x4 v, f32x4 p)
{
    const f32x4 u = (f32x4){__builtin_fmaf(-a, p.x, v.x), __builtin_fmaf(-a, p.y, v.y),
                            __builtin_fmaf(-a, p.z, v.z), __builtin_fmaf(-a, p.w, v.w)};
    return (f32x4){__builtin_fmaf(a, x.x, bw * u.x), __builtin_fmaf(a, x.y, bw * u.y),
                   __builtin_fmaf(a, x.z, bw * u.z), __builtin_fmaf(a, x.w, bw * u.w)};
}

// One 4-column chunk of v as fp32 (8 bytes of bf16 or 16 bytes of fp32).
__device__ __forceinline__ f32x4 v_chunk(uint2 raw)
{
    return (f32x4){__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                   __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 v_chunk(f32x4 raw) { return raw; }

}  // namespace sdm
