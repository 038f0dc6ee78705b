// pkm_address.h -- product-key addressing building blocks (device side).
//
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 2 (Product-Key Memories) and Sec. 3.1 step 1 (Sparse Key Selection):
// the key is split in two halves, each half is scored against its own set of
// n_sub sub-keys, the N = n_sub^2 slot scores are the outer sum of the two
// half-score vectors and only the top-k' of each half enter the merge.
// Sec. 4 (SDM Configuration): the selected scores are softmax-normalised.
//
// Used by the prefill addressing kernel and by the fused decode kernel, so
// both select bit-identical slots from identical scores.
#pragma once

#include "device_common.h"

namespace sdm {

constexpr int kTileRows = 16;  // token rows scored together (MFMA M dimension)

// fp32 half scores S[r][u] = <x_r[c*half : (c+1)*half], C[h][c][u]> for the
// rows r < nrows of one tile, written to LDS (row stride n_sub).  bf16 inputs
// use the gfx950 MFMA v_mfma_f32_16x16x32_bf16 with fp32 accumulation (rows
// >= nrows enter the MFMA as zero vectors and are not stored); every output
// element depends only on its own row, so a row's scores do not depend on
// which other rows share the tile.  All threads of the block take part; the caller
// synchronises before reading S.
//   x: base of the tile's first row; consecutive tile rows are row_stride
//      elements apart.
template <bool BF16>
__device__ __forceinline__ void score_half_tile(const void *x, int64_t row_stride, int nrows,
                                                const void *Cc /* [n_sub, half] of (h, c) */,
                                                int c, int half, int n_sub, float *S)
{
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    if constexpr (BF16) {
        const int lane = lane_id();
        const int wave = tid / kWave;
        const int nwaves = nthreads / kWave;
        const int r = lane & 15;          // A row / B column handled by this lane
        const int kg = lane >> 4;         // which 8-wide k group of the 32
        const uint16_t *xr = static_cast<const uint16_t *>(x) + (int64_t)r * row_stride + c * half;
        const uint16_t *C16 = static_cast<const uint16_t *>(Cc);
        const int nk = half / 32;
        for (int st = wave; st * 16 < n_sub; st += nwaves) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int u = st * 16 + r;    // sub-key (B column) of this lane
            const uint16_t *cr = C16 + (int64_t)u * half;
            for (int kk = 0; kk < nk; ++kk) {
                bf16x8 av = (bf16x8){}, bv = (bf16x8){};
                if (r < nrows) av = *reinterpret_cast<const bf16x8 *>(xr + kk * 32 + kg * 8);
                if (u < n_sub) bv = *reinterpret_cast<const bf16x8 *>(cr + kk * 32 + kg * 8);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
            }
            // D[i][j]: lane holds column j = lane & 15 (sub-key), rows 4*(lane>>4) + e
            if (u < n_sub) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 4 * kg + e;
                    if (row < nrows) S[row * n_sub + u] = acc[e];
                }
            }
        }
    } else {
        const float *xf = static_cast<const float *>(x);
        const float *Cf = static_cast<const float *>(Cc);
        for (int e = tid; e < nrows * n_sub; e += nthreads) {
            const int row = e / n_sub, u = e - row * n_sub;
            const float *xr = xf + (int64_t)row * row_stride + c * half;
            const float *cr = Cf + (int64_t)u * half;
            float acc = 0.f;
            for (int d = 0; d < half; ++d) acc = __builtin_fmaf(xr[d], cr[d], acc);
            S[e] = acc;
        }
    }
}

// Top-k' of one row of half scores (n_sub values in LDS) by one wave.
// Lane j < k' receives the key of the j-th best sub-key.
__device__ __forceinline__ uint64_t half_topk(const float *Srow, int n_sub, int kp, uint64_t *scratch)
{
    return wave_topn(n_sub, kp,
                     [&](int p) { return score_key(Srow[p], (uint32_t)p); }, scratch);
}

// Merge of two per-half lists (keys in lane j < kp, sorted) into the top-n
// slots, then softmax weights.  lists: per-wave LDS of 2*64 uint64.
// Lane j < n ends with (slot_j, weight_j).
__device__ __forceinline__ void merge_softmax(uint64_t k0, uint64_t k1, int kp, int n_sub, int n,
                                              uint64_t *lists, uint64_t *scratch, int &slot,
                                              float &weight)
{
    const int lane = lane_id();
    lists[lane] = k0;
    lists[kWave + lane] = k1;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t *l0 = lists, *l1 = lists + kWave;
    auto get = [&](int p) {
        const int ia = p / kp, ib = p - ia * kp;
        const uint64_t ka = l0[ia], kb = l1[ib];
        const float s = key_score(ka) + key_score(kb);
        const uint32_t idx = key_index(ka) * (uint32_t)n_sub + key_index(kb);
        return score_key(s, idx);
    };
    const uint64_t best = wave_topn(kp * kp, n, get, scratch);
    const float s = key_score(best);
    const float smax = __shfl(s, 0, kWave);
    const float e = lane < n ? expf(s - smax) : 0.f;
    const float z = wave_sum_f32(e);
    weight = e / z;
    slot = (int)key_index(best);
    __builtin_amdgcn_wave_barrier();
}

}  // namespace sdm
