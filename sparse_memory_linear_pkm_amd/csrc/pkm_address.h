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
// both select bit-identical slots and weights from identical scores.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace sdm {

constexpr int kTileRows = 16;     // token rows scored together (MFMA M dimension)

// B-operand fragments of one 16-sub-key tile of a [n_sub][half] bf16
// codebook for one k-step of v_mfma_f32_16x16x32_bf16 (the caller's C
// already offset to the k-step's first element): lane (r, kg) = (lane & 15,
// lane >> 4) needs elements kg*8 .. +8 of sub-key tile*16 + r.  Loaded in
// that lane order, the 4 consecutive lanes of every quad would read 4
// different sub-key rows (128 bytes apart for d_k = 128), which the load path
// serves one row at a time (measured: scoring alone 2.4x slower than with
// contiguous loads); instead lane l loads piece l & 3 of row l >> 2 (each
// quad reads 64 contiguous bytes) and ds_bpermute hands lane (r, kg) its
// piece from lane 4r + kg.  The operands, and so the scores, are unchanged.
// (Whole contiguous rows per load, with two exchanges and a select per
// register, measured slower: the exchanges cost more than the loads saved.)
// Sub-keys past n_sub (unless FULL) load a valid neighbour and are zeroed.
template <bool FULL>
__device__ __forceinline__ i32x4 codebook_tile_load(const uint16_t *C, int half, int n_sub, int tile)
{
    const int lane = lane_id();
    const int u = tile * 16 + (lane >> 2);
    const int e = (lane & 3) * 8;
    if constexpr (FULL) {
        return *reinterpret_cast<const i32x4 *>(C + (int64_t)u * half + e);
    } else {
        const i32x4 v = *reinterpret_cast<const i32x4 *>(C + (int64_t)min(u, n_sub - 1) * half + e);
        return u < n_sub ? v : (i32x4){0, 0, 0, 0};
    }
}

__device__ __forceinline__ bf16x8 codebook_tile_frag(i32x4 raw)
{
    const int lane = lane_id();
    const int src = (4 * (lane & 15) + (lane >> 4)) << 2;
    i32x4 g;
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = __builtin_amdgcn_ds_bpermute(src, raw[e]);
    return __builtin_bit_cast(bf16x8, g);
}

// fp32 half scores S[r][u] = <x_r[c*half : (c+1)*half], C[h][c][u]> for the
// first `srows` rows of one 16-row tile, written to LDS (row stride n_sub) as
// their order-preserving bits (score_bits), the form every comparison uses.
// Rows >= nrows are scored as zero vectors (so stored rows past the real ones
// hold zeros).  bf16 inputs use the gfx950 MFMA v_mfma_f32_16x16x32_bf16 with
// fp32 accumulation; every output element depends only on its own row, so a
// row's scores do not depend on which other rows share the tile.  All threads
// of the block take part; the caller synchronises before reading S.
//   x: base of the tile's first row; consecutive tile rows are row_stride
//      elements apart.
//   NB: sub-key tiles whose codebook loads a wave issues together (a
//      latency-bound caller with few waves wants many in flight; the result
//      does not depend on NB).
//   sst: row stride of S in elements (0: n_sub).
//   RAW: store the raw fp32 bits instead of score_bits (for callers that
//        compare the stored scores as floats).
//   FULL: n_sub is a multiple of 16 * NB, so every sub-key tile a wave takes
//        is whole and no lane needs the bounds check.
template <bool BF16, int NB = 1, int NK = 0, bool RAW = false, bool FULL = false>
__device__ __forceinline__ void score_half_tile(const void *x, int64_t row_stride, int nrows,
                                                int srows,
                                                const void *Cc /* [n_sub, half] of (h, c) */,
                                                int c, int half, int n_sub, uint32_t *S, int sst = 0)
{
    if (sst == 0) sst = n_sub;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    if constexpr (BF16) {
        const int lane = lane_id();
        const int wave = tid / kWave;
        const int nwaves = nthreads / kWave;
        const int r = lane & 15;          // A row / B column handled by this lane
        const int kg = lane >> 4;         // which 8-wide k group of the 32
        // rows past nrows and sub-keys past n_sub load a valid neighbour and
        // are zeroed (no branches around the loads)
        const uint16_t *xr = static_cast<const uint16_t *>(x) + (int64_t)max(min(r, nrows - 1), 0) * row_stride + c * half;
        const bool rlive = r < nrows;
        const uint16_t *C16 = static_cast<const uint16_t *>(Cc);
        // k-steps of 32: a compile-time count when NK > 0 (d_k = 64 * NK), else half / 32 (<= 8)
        constexpr int KMAX = NK > 0 ? NK : 8;
        const int nk = NK > 0 ? NK : half / 32;
        const bf16x8 zero = (bf16x8){};
        bf16x8 av[KMAX];
#pragma unroll
        for (int kk = 0; kk < KMAX; ++kk) {
            av[kk] = zero;
            if (NK > 0 || kk < nk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(xr + kk * 32 + kg * 8);
                av[kk] = rlive ? a : zero;
            }
        }
        // codebook fragments: contiguous loads and a lane exchange
        // (codebook_tile_load / codebook_tile_frag)
        for (int st0 = wave * NB; st0 * 16 < n_sub; st0 += nwaves * NB) {
            f32x4 acc[NB];
#pragma unroll
            for (int t = 0; t < NB; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
            // with a compile-time k-step count every load of the round is
            // issued before the first exchange (one memory round trip per
            // round instead of one per k-step); the MFMAs still accumulate
            // the k-steps in order, so the scores are unchanged
            constexpr int KL = NK > 0 ? NK : 1;   // k-steps loaded together
#pragma unroll
            for (int kk0 = 0; kk0 < KMAX; kk0 += KL) {
                if (NK > 0 || kk0 < nk) {
                    i32x4 raw[KL][NB];
#pragma unroll
                    for (int j = 0; j < KL; ++j)
#pragma unroll
                        for (int t = 0; t < NB; ++t)
                            raw[j][t] = codebook_tile_load<FULL>(C16 + (kk0 + j) * 32, half, n_sub, st0 + t);
#pragma unroll
                    for (int j = 0; j < KL; ++j) {
                        // every exchange of the k-step before its first MFMA
                        bf16x8 bv[NB];
#pragma unroll
                        for (int t = 0; t < NB; ++t) bv[t] = codebook_tile_frag(raw[j][t]);
#pragma unroll
                        for (int t = 0; t < NB; ++t)
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[kk0 + j], bv[t], acc[t], 0, 0, 0);
                    }
                }
            }
            // D[i][j]: lane holds column j = lane & 15 (sub-key), rows 4*(lane>>4) + e
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                const int u = (st0 + t) * 16 + r;
                if (FULL || u < n_sub) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 4 * kg + e;
                        if (row < srows) S[row * sst + u] = RAW ? __float_as_uint(acc[t][e]) : score_bits(acc[t][e]);
                    }
                }
            }
        }
    } else {
        const float *xf = static_cast<const float *>(x);
        const float *Cf = static_cast<const float *>(Cc);
        for (int e = tid; e < srows * n_sub; e += nthreads) {
            const int row = e / n_sub, u = e - row * n_sub;
            float acc = 0.f;
            if (row < nrows) {
                const float *xr = xf + (int64_t)row * row_stride + c * half;
                const float *cr = Cf + (int64_t)u * half;
                for (int d = 0; d < half; ++d) acc = __builtin_fmaf(xr[d], cr[d], acc);
            }
            S[row * sst + u] = RAW ? __float_as_uint(acc) : score_bits(acc);
        }
    }
}

// An entry of a selected half list: the raw fp32 score bits and the sub-key.
struct HalfEntry {
    uint32_t score;
    uint32_t index;
};

// Copy of a staircase into LDS by all threads of the block (the caller
// synchronises before use).
__device__ __forceinline__ void load_staircase(const Staircase &st, uint16_t *stair)
{
    for (int e = threadIdx.x; e < st.count; e += blockDim.x) stair[e] = st.e[e];
}

// Top-k' of NR rows of half scores, one wave.  Row r's n_sub score bits are
// at S + rows[r] * n_sub; lane j < k' of keys[r] receives the j-th best
// (score desc, sub-key asc).
// sst: row stride of S in elements (0: n_sub).  RAW: S holds raw fp32 bits
// (converted to score_bits on the fly).
template <int NR, bool RAW = false>
__device__ __forceinline__ void half_topk(const uint32_t *S, const int (&rows)[NR], int n_sub, int kp,
                                          uint64_t *scratch, uint64_t (&keys)[NR], int sst = 0)
{
    if (sst == 0) sst = n_sub;
    int ib = 1;   // bits of a sub-key index
    while ((1 << ib) < n_sub) ++ib;
    wave_topn<NR>(n_sub, kp,
                  [&](int r, int p) {
                      const uint32_t v = S[rows[r] * sst + p];
                      return ((uint64_t)(RAW ? score_bits(__uint_as_float(v)) : v) << 32) | (uint32_t)~p;
                  },
                  scratch, keys, ib);
}

// Merge of the two half lists of NR rows into the top-n slots and their
// softmax weights, one wave.  L0[r], L1[r]: the k' entries of row r's half 0
// and half 1 lists, best first.  The slot of pair (a, b) is
// L0[a].index * n_sub + L1[b].index and its score the fp32 sum of the two
// half scores.
//
// The top n are taken over the staircase first.  The result is exact when
// the n-th score found is strictly above every pair just outside the
// staircase, (a, floor(n / (a + 1))) for each a, which bound all pairs
// outside it; otherwise (a tie at the border) that row is redone over all
// k'^2 pairs.  Lane j < n ends with slot[r] and wt[r] of the j-th best.
template <int NR>
__device__ __forceinline__ void merge_softmax(const HalfEntry *const (&L0)[NR],
                                              const HalfEntry *const (&L1)[NR], int kp, int n_sub,
                                              int n, const uint16_t *stair, int nstair,
                                              uint64_t *scratch, int (&slot)[NR], float (&wt)[NR])
{
    const int lane = lane_id();
    auto pair_key = [&](int r, int a, int b) {
        const HalfEntry e0 = L0[r][a], e1 = L1[r][b];
        const float s = __uint_as_float(e0.score) + __uint_as_float(e1.score);
        return score_key(s, e0.index * (uint32_t)n_sub + e1.index);
    };
    uint64_t best[NR];
    wave_topn<NR>(nstair, n,
                  [&](int r, int p) {
                      const uint32_t ab = stair[p];
                      return pair_key(r, (int)(ab >> 8), (int)(ab & 0xff));
                  },
                  scratch, best);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        uint32_t fb = 0;
        const int b0 = n / (lane + 1);
        if (lane < kp && b0 < kp) {
            const float s = __uint_as_float(L0[r][lane].score) + __uint_as_float(L1[r][b0].score);
            fb = score_bits(s);
        }
        fb = wave_max(fb);
        const uint32_t nth = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(best[r] >> 32), n - 1);
        if (!(nth > fb)) {
            uint64_t one[1];
            wave_topn<1>(kp * kp, n,
                         [&](int, int p) {
                             const int a = p / kp;
                             return pair_key(r, a, p - a * kp);
                         },
                         scratch, one);
            best[r] = one[0];
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float s = key_score(best[r]);
        const float smax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(s), 0));
        const float e = lane < n ? __expf(s - smax) : 0.f;
        const float z = wave_sum_f32(e);
        wt[r] = __fdividef(e, z);
        slot[r] = (int)key_index(best[r]);
    }
}

}  // namespace sdm
