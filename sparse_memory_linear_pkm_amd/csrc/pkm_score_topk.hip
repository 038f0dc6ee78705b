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
//   2. one wave per row: exact top-k' of the half (score desc, index asc);
//   3. one wave per row: exact top-n of the k'^2 outer-sum candidates,
//      softmax, store slots and weights.
// The N slot scores are never materialised.
#include "kernels.h"
#include "pkm_address.h"

namespace sdm {

template <bool BF16>
__global__ void __launch_bounds__(256) pkm_score_topk_kernel(AddressArgs args)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int kind = blockIdx.z;
    const AddressKind &K = args.kind[kind];
    const int h = blockIdx.y;
    const int64_t bt0 = (int64_t)blockIdx.x * kTileRows;
    const int nrows = (int)min<int64_t>(kTileRows, args.BT - bt0);
    const int n_sub = args.n_sub, kp = args.k_prime, half = args.d_k / 2;
    constexpr int nwaves = 4;  // blockDim.x == 256
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();

    float *S = reinterpret_cast<float *>(smem);                                   // [16][n_sub]
    uint64_t *scratch = reinterpret_cast<uint64_t *>(smem + sizeof(float) * kTileRows * n_sub);
    uint64_t *wscr = scratch + wave * (3 * kWave);                                 // per wave

    const size_t esz = BF16 ? 2 : 4;
    const unsigned char *xb = static_cast<const unsigned char *>(K.x) +
                              ((bt0 * args.H + h) * (int64_t)args.d_k) * esz;
    const unsigned char *Cb = static_cast<const unsigned char *>(K.C) +
                              ((int64_t)h * 2 * n_sub * half) * esz;
    const int64_t row_stride = (int64_t)args.H * args.d_k;

    // per-wave rows: r = wave, wave + nwaves, ...  (kTileRows / nwaves of them)
    constexpr int kMaxRowsPerWave = kTileRows / nwaves;
    uint64_t lists[2][kMaxRowsPerWave];

#pragma unroll
    for (int c = 0; c < 2; ++c) {
        score_half_tile<BF16>(xb, row_stride, nrows, Cb + (int64_t)c * n_sub * half * esz, c, half,
                              n_sub, S);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kMaxRowsPerWave; ++i) {
            const int r = wave + i * nwaves;
            uint64_t key = 0;
            if (r < nrows) key = half_topk(S + r * n_sub, n_sub, kp, wscr);
            lists[c][i] = key;
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < kMaxRowsPerWave; ++i) {
        const int r = wave + i * nwaves;
        if (r >= nrows) continue;
        int slot;
        float wt;
        merge_softmax(lists[0][i], lists[1][i], kp, n_sub, K.n_out, wscr + kWave, wscr, slot, wt);
        const int64_t g = (bt0 + r) * args.H + h;
        if (lane < K.n_out) {
            K.idx[g * K.n_out + lane] = slot;
            K.wt[g * K.n_out + lane] = wt;
        }
    }
}

size_t address_smem_bytes(int n_sub)
{
    return sizeof(float) * kTileRows * (size_t)n_sub + sizeof(uint64_t) * 3 * kWave * 4;
}

hipError_t launch_pkm_address(const AddressArgs &args, bool bf16, hipStream_t stream)
{
    if (args.BT <= 0) return hipSuccess;
    dim3 grid((unsigned)((args.BT + kTileRows - 1) / kTileRows), (unsigned)args.H, 2);
    const size_t smem = address_smem_bytes(args.n_sub);
    if (bf16) {
        hipError_t e = hipFuncSetAttribute((const void *)pkm_score_topk_kernel<true>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(pkm_score_topk_kernel<true>, grid, dim3(256), smem, stream, args);
    } else {
        hipError_t e = hipFuncSetAttribute((const void *)pkm_score_topk_kernel<false>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(pkm_score_topk_kernel<false>, grid, dim3(256), smem, stream, args);
    }
    return hipGetLastError();
}

}  // namespace sdm
