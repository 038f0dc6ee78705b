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
//   2. each wave takes 4 of the 16 rows together: exact top-k' of the half;
//   3. each wave: exact top-n of the outer-sum candidates of its 4 rows
//      (staircase-pruned, with an exact fallback), softmax, store slots and
//      weights.
// The N slot scores are never materialised.
//
// Work placement: consecutive workgroup ids are spread over the 8 XCDs, so
// the id is decoded such that the workgroups of one (head, kind) -- which
// all read the same codebook -- land on the same XCD and share its L2.
#include "kernels.h"
#include "pkm_address.h"

namespace sdm {

constexpr int kAddrWaves = 4;
constexpr int kRowsPerWave = kTileRows / kAddrWaves;
constexpr int kXcds = 8;

struct AddrLds {
    // byte offsets into dynamic LDS
    size_t S, L, scratch, stair, total;
};

__host__ __device__ inline AddrLds addr_lds_layout(int n_sub, int kp)
{
    AddrLds o;
    o.S = 0;                                                   // float [16][n_sub]
    o.L = o.S + sizeof(float) * kTileRows * (size_t)n_sub;     // HalfEntry [2][16][kp]
    o.scratch = o.L + sizeof(HalfEntry) * 2 * kTileRows * (size_t)kp;  // u64 [4][4][64]
    o.stair = o.scratch + sizeof(uint64_t) * kAddrWaves * kRowsPerWave * kWave;
    o.total = o.stair + sizeof(uint16_t) * kMaxStair;
    return o;
}

// NK: compile-time k-steps of the scoring tile (d_k = 64 * NK), 0 = any d_k
template <bool BF16, int NK>
__global__ void __launch_bounds__(256) pkm_score_topk_kernel(AddressArgs args, int ntiles)
{
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

    const AddrLds lay = addr_lds_layout(n_sub, kp);
    uint32_t *S = reinterpret_cast<uint32_t *>(smem + lay.S);
    HalfEntry *L = reinterpret_cast<HalfEntry *>(smem + lay.L);
    uint64_t *wscr = reinterpret_cast<uint64_t *>(smem + lay.scratch) + wave * kRowsPerWave * kWave;
    uint16_t *stair = reinterpret_cast<uint16_t *>(smem + lay.stair);

    const size_t esz = BF16 ? 2 : 4;
    const unsigned char *xb = static_cast<const unsigned char *>(K.x) +
                              ((bt0 * args.H + h) * (int64_t)args.d_k) * esz;
    const unsigned char *Cb = static_cast<const unsigned char *>(K.C) +
                              ((int64_t)h * 2 * n_sub * half) * esz;
    const int64_t row_stride = (int64_t)args.H * args.d_k;

    load_staircase(K.stair, stair);   // ordered before use by the barriers below
    const int nstair = K.stair.count;

    int rows[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) rows[i] = wave + i * kAddrWaves;

#pragma unroll
    for (int c = 0; c < 2; ++c) {
        score_half_tile<BF16, 1, NK>(xb, row_stride, nrows, kTileRows,
                              Cb + (int64_t)c * n_sub * half * esz, c, half, n_sub, S);
        __syncthreads();
        uint64_t keys[kRowsPerWave];
        half_topk<kRowsPerWave>(S, rows, n_sub, kp, wscr, keys);
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            if (lane < kp) {
                HalfEntry e;
                e.score = __float_as_uint(key_score(keys[i]));
                e.index = key_index(keys[i]);
                L[(c * kTileRows + rows[i]) * kp + lane] = e;
            }
        }
        __syncthreads();
    }

    const HalfEntry *L0[kRowsPerWave], *L1[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
        L0[i] = L + rows[i] * kp;
        L1[i] = L + (kTileRows + rows[i]) * kp;
    }
    int slot[kRowsPerWave];
    float wt[kRowsPerWave];
    merge_softmax<kRowsPerWave>(L0, L1, kp, n_sub, n, stair, nstair, wscr, slot, wt);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
        if (rows[i] < nrows && lane < n) {
            const int64_t g = (bt0 + rows[i]) * args.H + h;
            K.idx[g * n + lane] = slot[i];
            K.wt[g * n + lane] = wt[i];
        }
    }
}

size_t address_smem_bytes(int n_sub, int k_prime) { return addr_lds_layout(n_sub, k_prime).total; }

hipError_t launch_pkm_address(const AddressArgs &args, bool bf16, hipStream_t stream)
{
    if (args.BT <= 0) return hipSuccess;
    const int64_t ntiles = (args.BT + kTileRows - 1) / kTileRows;
    const int64_t grid = ntiles * 2 * args.H;
    if (ntiles > INT32_MAX || grid > UINT32_MAX) return hipErrorInvalidValue;
    const size_t smem = address_smem_bytes(args.n_sub, args.k_prime);
    auto launch = [&](auto kern) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), smem, stream, args, (int)ntiles);
        return hipSuccess;
    };
    hipError_t e;
    if (!bf16)
        e = launch(pkm_score_topk_kernel<false, 0>);
    else if (args.d_k == 128)
        e = launch(pkm_score_topk_kernel<true, 2>);
    else
        e = launch(pkm_score_topk_kernel<true, 0>);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace sdm
