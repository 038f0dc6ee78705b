// pkm_score_topk.hip -- prefill PKM addressing over all token-heads.
//
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 2 (Product-Key Memories), Sec. 3.1 step 1 (Sparse Key Selection) and
// Sec. 4 (softmax-normalised read and write activations).
//
// One workgroup (4 waves) takes 16 consecutive token positions of one head
// and one kind (write: k against C_w, read: q against C_r):
//   1. for each half c: the [16 x d_k/2] x [d_k/2 x n_sub] score tile on bf16
//      MFMA (fp32 accumulation) into LDS;
//   2. each wave takes 4 of the 16 rows, one per 16-lane group: exact top-k'
//      of the half (pkm_select16.h); with 1024 or more sub-keys per half the
//      half is scored and selected in parts of 512 and the exact part lists
//      merged, which keeps the tile at 512 sub-keys and four workgroups on a
//      CU;
//   3. each wave: exact top-n of the outer-sum candidates of its 4 rows
//      (staircase-pruned, with an exact fallback), softmax, store slots and
//      weights.
// Rows whose fast selection cannot vouch for its order (tied key prefixes,
// more than 64 survivors, a tie at the staircase border) are redone by the
// one-row routines of pkm_address.h.  The N slot scores are never
// materialised.
//
// Work placement: consecutive workgroup ids are spread over the 8 XCDs, so
// the id is decoded such that the workgroups of one (head, kind) -- which
// all read the same codebook -- land on the same XCD and share its L2.
#include "kernels.h"
#include "pkm_address.h"
#include "pkm_select16.h"

namespace sdm {

constexpr int kAddrWaves = 4;
constexpr int kXcds = 8;

struct AddrLds {
    // byte offsets into dynamic LDS
    size_t S, L, buf, scratch, stair, total;
    int sst;   // row stride of S in elements
};

// The two half lists are kept in registers while the score tile is in use
// and written to LDS only for the merge, into the tile's space (free by
// then), so a workgroup's LDS is the tile, the survivor buffers, the one-row
// routines' scratch and the staircase: 39 KB for n_sub = 512 (four
// workgroups per CU), 71 KB for n_sub = 1024 (two).
__host__ __device__ inline AddrLds addr_lds_layout(int n_sub, int kp)
{
    AddrLds o;
    // rows padded with zeros to a multiple of 64 candidates, plus 4 elements
    // so that consecutive rows start in different LDS banks
    o.sst = ((n_sub + 63) / 64) * 64 + 4;
    const size_t tile = sizeof(uint32_t) * kTileRows * (size_t)o.sst;       // uint32 [16][sst]
    const size_t lists = sizeof(HalfEntry) * 2 * kTileRows * (size_t)kp;   // HalfEntry [2][16][kp]
    o.S = 0;
    o.L = 0;                                                      // aliases the tile (merge only)
    o.buf = ((tile > lists ? tile : lists) + 15) / 16 * 16;       // uint32 [16][64] survivors
    o.scratch = o.buf + sizeof(uint32_t) * kTileRows * 64;        // uint64 [4][64] (one-row routines)
    o.stair = o.scratch + sizeof(uint64_t) * kAddrWaves * kWave;
    o.total = o.stair + sizeof(uint16_t) * kMaxStair;
    return o;
}

// Codebook loads a wave issues together in the scoring (sub-key tiles).
constexpr int kScoreNB = 4;
// Sub-keys per part of a half in the split form.
constexpr int kSplit = 512;

// NK: compile-time k-steps of the scoring tile (d_k = 64 * NK), 0 = any d_k.
// FULL: n_sub is a multiple of 16 * kScoreNB (no bounds checks in the scoring).
// PARTS != 1: each half scored and selected in parts of kSplit sub-keys
// (n_sub a multiple of kSplit, at least two parts, k' <= 32), so that the
// tile, and the workgroup's LDS, is that of n_sub = kSplit; PARTS = 2 fixes
// two parts (n_sub = 1024) at compile time, 0 takes n_sub / kSplit.
template <bool BF16, int NK, bool FULL, int PARTS>
__global__ void __launch_bounds__(256, PARTS != 1 ? 4 : 1) pkm_score_topk_kernel(AddressArgs args, int ntiles)
{
    constexpr bool SPLIT = PARTS != 1;
    extern __shared__ __align__(16) unsigned char smem[];
    // id -> (kind, h, tile): groups of (head, kind) pairs are pinned to one XCD.
    const int npairs = 2 * args.H;
    const int64_t id = blockIdx.x;
    const int xcd = (int)(id % kXcds);
    const int64_t k_in = id / kXcds;            // index among this XCD's workgroups
    // pairs xcd, xcd + 8, ... belong to this XCD; when npairs is not a multiple
    // of 8 the last round is shared by all XCDs (still correct, less local).
    const int full_rounds = npairs / kXcds;
    const int64_t per_xcd = (int64_t)full_rounds * ntiles;
    int pair;
    int64_t tile;
    if (k_in < per_xcd) {
        pair = (int)(k_in / ntiles) * kXcds + xcd;
        tile = k_in % ntiles;
    } else {
        const int64_t rest = (id - per_xcd * kXcds);  // over the remaining pairs, plain order
        pair = full_rounds * kXcds + (int)(rest / ntiles);
        tile = rest % ntiles;
    }
    const int kind = pair & 1;
    const int h = pair >> 1;
    const AddressKind &K = args.kind[kind];
    const int64_t bt0 = tile * kTileRows;
    const int nrows = (int)min<int64_t>(kTileRows, args.BT - bt0);
    const int n_sub = args.n_sub, kp = args.k_prime, half = args.d_k / 2, n = K.n_out;
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & (kGroupLanes - 1);

    const AddrLds lay = addr_lds_layout(SPLIT ? kSplit : n_sub, kp);
    const int sst = lay.sst;
    uint32_t *S = reinterpret_cast<uint32_t *>(smem + lay.S);
    HalfEntry *L = reinterpret_cast<HalfEntry *>(smem + lay.L);
    uint32_t *buf = reinterpret_cast<uint32_t *>(smem + lay.buf);
    uint64_t *wscr = reinterpret_cast<uint64_t *>(smem + lay.scratch) + wave * kWave;
    uint16_t *stair = reinterpret_cast<uint16_t *>(smem + lay.stair);

    const size_t esz = BF16 ? 2 : 4;
    const unsigned char *xb = static_cast<const unsigned char *>(K.x) +
                              ((bt0 * args.H + h) * (int64_t)args.d_k) * esz;
    const unsigned char *Cb = static_cast<const unsigned char *>(K.C) +
                              ((int64_t)h * 2 * n_sub * half) * esz;
    const int64_t row_stride = (int64_t)args.H * args.d_k;

    load_staircase(K.stair, stair);   // ordered before use by the barriers below
    const int nstair = K.stair.count;
    // the padding of every score row past n_sub holds -inf (below every real
    // score; the scoring never writes it)
    {
        const int tcols = SPLIT ? kSplit : n_sub;   // sub-keys in the tile
        const int padw = sst - tcols;
        for (int e = threadIdx.x; e < kTileRows * padw; e += blockDim.x)
            S[(e / padw) * sst + tcols + e % padw] = 0xFF800000u;
    }

    // rows of this wave: wave + 4 g for lane group g
    const int row_g = wave + kAddrWaves * g;
    const RowBuf rb{buf + wave * kAddrWaves * 64};

    // the half lists of this lane's row, entries 4 c16 .. 4 c16 + 3
    HalfEntry hl[2][4];
    // SPLIT: each half's sub-keys in parts of kSplit, one part in the tile at
    // a time; each part's list is exact, and merge_sorted16 folds it into the
    // best k' so far (the same list, in the same order, as one selection over
    // the whole half)
    const int nparts = PARTS > 0 ? PARTS : n_sub / kSplit;
    const int ncols = SPLIT ? kSplit : n_sub;   // sub-keys per part
    // one part of half c: score it, select it, fold it into hl[c]
    auto do_part = [&](const int c, const int pt) __attribute__((always_inline)) {
        // (the split form loads two sub-key tiles per round instead of four:
        // fewer registers, so that four of its workgroups fit a CU)
        score_half_tile<BF16, SPLIT ? 2 : kScoreNB, NK, true, FULL>(
            xb, row_stride, nrows, kTileRows, Cb + ((int64_t)c * n_sub + (int64_t)pt * ncols) * half * esz, c,
            half, ncols, S, sst);
        __syncthreads();
        HalfEntry pl[4];
        uint32_t pn;   // entries of this part's list (the row's)
        // a later part lists only candidates at or above the k'-th score
        // so far: the earlier parts alone have k' at or above it, and on
        // equal scores their lower sub-keys come first
        uint32_t floor_bits = 0u;
        if (pt > 0) {
            const uint32_t sc[4] = {hl[c][0].score, hl[c][1].score, hl[c][2].score, hl[c][3].score};
            floor_bits = score_bits(__uint_as_float(rank_value(sc, kp - 1)));
        }
        const bool bad = half_topk16(S, sst, row_g, ncols, kp, rb, pl, pn, pt > 0, floor_bits);
        // rows the fast path could not vouch for: the exact one-row
        // routine, its list handed to the row's lane group through the
        // wave's scratch
        const uint64_t bb = __ballot(bad);
        for (int gg = 0; gg < kAddrWaves; ++gg) {
            if ((bb >> (16 * gg)) & 0xFFFFull) {
                const int rows1[1] = {wave + kAddrWaves * gg};
                uint64_t keys[1];
                half_topk<1, true>(S, rows1, ncols, kp, wscr, keys, sst);
                wave_lds_sync();
                if (lane < kp)
                    wscr[lane] = ((uint64_t)key_index(keys[0]) << 32) | __float_as_uint(key_score(keys[0]));
                wave_lds_sync();
                if (g == gg) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 4 * c16 + r;
                        const uint64_t e = wscr[j < kp ? j : 0];
                        pl[r].score = (uint32_t)e;
                        pl[r].index = (uint32_t)(e >> 32);
                    }
                    pn = (uint32_t)kp;
                }
                wave_lds_sync();
            }
        }
        __syncthreads();   // the tile is free: every wave has finished reading it
        if (pt == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) hl[c][r] = pl[r];
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) pl[r].index += (uint32_t)(pt * ncols);
            HalfEntry m[4];
            merge_sorted16(hl[c], pl, kp, (int)pn, m);
#pragma unroll
            for (int r = 0; r < 4; ++r) hl[c][r] = m[r];
        }
    };
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        if constexpr (PARTS > 0) {
#pragma unroll
            for (int pt = 0; pt < PARTS; ++pt) do_part(c, pt);
        } else {
            for (int pt = 0; pt < nparts; ++pt) do_part(c, pt);
        }
    }
    // both lists into LDS for the merge (each wave reads only its own rows)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 4 * c16 + r;
            if (j < kp) L[(c * kTileRows + row_g) * kp + j] = hl[c][r];
        }
    wave_lds_sync();

    int slot[4];
    float wt[4];
    const bool bad = merge16(L + row_g * kp, L + (kTileRows + row_g) * kp, kp, n_sub, n, stair, nstair, rb, slot, wt);
    if (!bad && row_g < nrows) {
        const int64_t gr = (bt0 + row_g) * args.H + h;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 4 * c16 + r;
            if (j < n) {
                K.idx[gr * n + j] = slot[r];
                K.wt[gr * n + j] = wt[r];
            }
        }
    }
    const uint64_t bb = __ballot(bad);
    for (int gg = 0; gg < kAddrWaves; ++gg) {
        if ((bb >> (16 * gg)) & 0xFFFFull) {
            const int r1 = wave + kAddrWaves * gg;
            const HalfEntry *L0[1] = {L + r1 * kp}, *L1[1] = {L + (kTileRows + r1) * kp};
            int s1[1];
            float w1[1];
            merge_softmax<1>(L0, L1, kp, n_sub, n, stair, nstair, wscr, s1, w1);
            if (r1 < nrows && lane < n) {
                const int64_t gr = (bt0 + r1) * args.H + h;
                K.idx[gr * n + lane] = s1[0];
                K.wt[gr * n + lane] = w1[0];
            }
            wave_lds_sync();
        }
    }
}

size_t address_smem_bytes(int n_sub, int k_prime) { return addr_lds_layout(n_sub, k_prime).total; }

// LDS a workgroup requests when it must leave room on its CU for a
// concurrent kernel: more than half of the CU's 160 KB, so that a CU holds
// at most one addressing workgroup, and 76 KB left for the other kernel (the
// prefill scan's workgroups need 24-64 KB).
constexpr size_t kOnePerCuLds = 84 * 1024;

hipError_t launch_pkm_address(const AddressArgs &args, bool bf16, hipStream_t stream, bool one_per_cu)
{
    if (args.BT <= 0) return hipSuccess;
    const int64_t ntiles = (args.BT + kTileRows - 1) / kTileRows;
    const int64_t grid = ntiles * 2 * args.H;
    if (ntiles > INT32_MAX || grid > UINT32_MAX) return hipErrorInvalidValue;
    // halves of 1024 or more sub-keys selected in parts of 512 (LDS 40 KB
    // instead of 72 KB or more: four workgroups per CU instead of two or one).  Not in the
    // one-per-CU launch: there the occupancy is fixed and the split form's
    // extra selection work only makes it longer (measured: the long-context
    // step's overlapped addressing 232 -> 345 ms and its scan 1-2% slower).
    const bool split = !one_per_cu && bf16 && args.d_k == 128 && args.n_sub >= 2 * kSplit &&
                       args.n_sub % kSplit == 0 && args.k_prime <= 32;
    size_t smem = address_smem_bytes(split ? kSplit : args.n_sub, args.k_prime);
    if (one_per_cu && smem < kOnePerCuLds) smem = kOnePerCuLds;   // the extra LDS is never touched
    auto launch = [&](auto kern) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), smem, stream, args, (int)ntiles);
        return hipSuccess;
    };
    hipError_t e;
    const bool full = args.n_sub % (16 * kScoreNB) == 0;
    if (!bf16)
        e = launch(pkm_score_topk_kernel<false, 0, false, 1>);
    else if (split && args.n_sub == 2 * kSplit)
        e = launch(pkm_score_topk_kernel<true, 2, true, 2>);
    else if (split)
        e = launch(pkm_score_topk_kernel<true, 2, true, 0>);
    else if (args.d_k == 128)
        e = full ? launch(pkm_score_topk_kernel<true, 2, true, 1>) : launch(pkm_score_topk_kernel<true, 2, false, 1>);
    else
        e = full ? launch(pkm_score_topk_kernel<true, 0, true, 1>) : launch(pkm_score_topk_kernel<true, 0, false, 1>);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace sdm
