// scan_step.h -- one token of the sparse gated delta rule on one 32-column
// slice of one (sequence, head) memory, by one wave.
//
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 step 2 (Gated Delta Write, Eq. 4) and step 3 (Sparse Read);
// "Sparse Delta Memory: Scaling Linear RNN States to 1M Tokens via
// Sparsity", Methodology item 2:
//     p = sum_j w_j M[s_j]                      (rows before the write)
//     M[s_j] = a M[s_j] + b w_j (v - a p)       (all j at once)
//     o = sum_j r_j M[s'_j]                     (rows after the write)
// Columns are independent, so a memory of width d_v is processed as d_v/32
// independent 32-column slices.
//
// Lane layout: lane l covers columns 4*(l & 7) .. +3 of the slice and rows
// (l >> 3) + 8*k of the slot list (k = 0..7, W and R <= 64), so one 128-byte
// row segment is one coalesced 8-lane access and every load or store is
// 16 bytes per lane.  The sum over rows is a reduction over lanes that share
// (l & 7).
#pragma once

#include "device_common.h"

namespace sdm {

__device__ __forceinline__ f32x4 fma4(float s, f32x4 x, f32x4 acc)
{
    acc.x = __builtin_fmaf(s, x.x, acc.x);
    acc.y = __builtin_fmaf(s, x.y, acc.y);
    acc.z = __builtin_fmaf(s, x.z, acc.z);
    acc.w = __builtin_fmaf(s, x.w, acc.w);
    return acc;
}

__device__ __forceinline__ f32x4 shfl_xor4(f32x4 x, int m)
{
    f32x4 y;
    y.x = __shfl_xor(x.x, m, kWave);
    y.y = __shfl_xor(x.y, m, kWave);
    y.z = __shfl_xor(x.z, m, kWave);
    y.w = __shfl_xor(x.w, m, kWave);
    return y;
}

// x[l] + x[l ^ 8] + x[l ^ 16] + x[l ^ 24] + ... : the sum over the 8 lanes
// that share (l & 7), left in every one of them.  Lane exchanges run on the
// VALU: DPP row_ror:8 pairs l with l ^ 8 inside each 16-lane row, and the
// gfx950 permlane16/32 swaps pair l with l ^ 16 and l ^ 32.
__device__ __forceinline__ float rowgroup_sum1(float x)
{
    constexpr int kRowRor8 = 0x128;
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowRor8, 0xf, 0xf, false));
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// Sum over the 8 row groups (lanes with equal lane & 7).
__device__ __forceinline__ f32x4 rowgroup_sum(f32x4 x)
{
    f32x4 r;
    r.x = rowgroup_sum1(x.x);
    r.y = rowgroup_sum1(x.y);
    r.z = rowgroup_sum1(x.z);
    r.w = rowgroup_sum1(x.w);
    return r;
}

template <bool BF16>
__device__ __forceinline__ f32x4 load_v4(const void *vrow, int col)
{
    if constexpr (BF16) {
        const uint2 raw = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(vrow) + col);
        f32x4 r;
        r.x = __uint_as_float(raw.x << 16);
        r.y = __uint_as_float(raw.x & 0xffff0000u);
        r.z = __uint_as_float(raw.y << 16);
        r.w = __uint_as_float(raw.y & 0xffff0000u);
        return r;
    } else {
        return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(vrow) + col);
    }
}

__device__ __forceinline__ f32x4 mload(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
}

__device__ __forceinline__ void mstore(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, f32x4 x)
{
    __builtin_amdgcn_raw_buffer_store_b128(x, rs, byte_off, 0, 0);
}

// One token, one slice.  Mrs covers the (b, h) memory [N, d_v]; col is the
// first of this lane's four columns (slice*32 + 4*(lane & 7)).
// wi/ww (W entries) and ri/rw (R entries) may live in global memory or LDS.
template <bool BF16>
__device__ __forceinline__ void scan_token_slice(__amdgpu_buffer_rsrc_t Mrs, int d_v, int col,
                                                 const int32_t *wi, const float *ww, int W,
                                                 const int32_t *ri, const float *rw, int R,
                                                 const void *vrow, float at, float bt, float *orow)
{
    const int lane = lane_id();
    const int rsub = lane >> 3;
    f32x4 m[8];
    float wj[8];
    uint32_t off[8];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int j = rsub + 8 * k;
        if (8 * k < W && j < W) {
            off[k] = ((uint32_t)wi[j] * (uint32_t)d_v + (uint32_t)col) * 4u;
            wj[k] = ww[j];
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int j = rsub + 8 * k;
        if (8 * k < W && j < W) {
            m[k] = mload(Mrs, off[k]);
            acc = fma4(wj[k], m[k], acc);
        }
    }
    const f32x4 p = rowgroup_sum(acc);
    const f32x4 vv = load_v4<BF16>(vrow, col);
    f32x4 u;
    u.x = __builtin_fmaf(-at, p.x, vv.x);
    u.y = __builtin_fmaf(-at, p.y, vv.y);
    u.z = __builtin_fmaf(-at, p.z, vv.z);
    u.w = __builtin_fmaf(-at, p.w, vv.w);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int j = rsub + 8 * k;
        if (8 * k < W && j < W) {
            const float bw = bt * wj[k];
            f32x4 nm;
            nm.x = __builtin_fmaf(at, m[k].x, bw * u.x);
            nm.y = __builtin_fmaf(at, m[k].y, bw * u.y);
            nm.z = __builtin_fmaf(at, m[k].z, bw * u.z);
            nm.w = __builtin_fmaf(at, m[k].w, bw * u.w);
            mstore(Mrs, off[k], nm);
        }
    }
    // The read must see this token's writes: same-wave stores are ordered
    // before later loads of the same addresses.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int j = rsub + 8 * k;
        if (8 * k < R && j < R) {
            const uint32_t o2 = ((uint32_t)ri[j] * (uint32_t)d_v + (uint32_t)col) * 4u;
            acc = fma4(rw[j], mload(Mrs, o2), acc);
        }
    }
    const f32x4 o = rowgroup_sum(acc);
    if (rsub == 0) *reinterpret_cast<f32x4 *>(orow + col) = o;
}

}  // namespace sdm
