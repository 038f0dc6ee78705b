// sdm_decode.hip -- one new token for each of B sequences: PKM addressing and
// one step of the sparse gated delta rule fused in a single launch.
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 steps 1-3 for a single token.
//
// One workgroup (4 waves) per (b, h):
//   A. the four half-score vectors (write/read x half 0/1) on bf16 MFMA, with
//      the same tile code as the prefill addressing (so the scores, and hence
//      the selected slots, are bit-identical to a prefill of the same token);
//   B. wave w selects the top-k' of list w;
//   C. waves 0 and 1 merge and softmax the write and read lists;
//   D. one wave per 32-column slice applies the write and the read.
#include "kernels.h"
#include "pkm_address.h"
#include "scan_step.h"

namespace sdm {

template <bool BF16>
__global__ void __launch_bounds__(256) sdm_decode_kernel(DecodeArgs A)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int bh = blockIdx.x;
    const int bb = bh / A.H, h = bh - bb * A.H;
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int n_sub = A.n_sub, half = A.d_k / 2, kp = A.k_prime;
    const size_t esz = BF16 ? 2 : 4;

    float *S = reinterpret_cast<float *>(smem);                          // [4][n_sub]
    uint64_t *lists = reinterpret_cast<uint64_t *>(S + 4 * n_sub);       // [4][64]
    uint64_t *wscr = lists + 4 * kWave + wave * (3 * kWave);             // per wave
    int32_t *fidx = reinterpret_cast<int32_t *>(lists + 4 * kWave + 4 * 3 * kWave);  // [2][64]
    float *fwt = reinterpret_cast<float *>(fidx + 2 * kWave);                          // [2][64]

    // A. scores (row 0 of a 16-row tile is this token; the others are zero)
#pragma unroll
    for (int kind = 0; kind < 2; ++kind) {
        const void *x = kind ? A.q : A.k;
        const void *C = kind ? A.C_r : A.C_w;
        const unsigned char *xb = static_cast<const unsigned char *>(x) + (size_t)bh * A.d_k * esz;
        const unsigned char *Cb = static_cast<const unsigned char *>(C) +
                                  (size_t)h * 2 * n_sub * half * esz;
        for (int c = 0; c < 2; ++c)
            score_half_tile<BF16>(xb, A.d_k, 1, Cb + (size_t)c * n_sub * half * esz, c, half, n_sub,
                                  S + (kind * 2 + c) * n_sub);
    }
    __syncthreads();
    // B. per-half top-k'
    lists[wave * kWave + lane] = half_topk(S + wave * n_sub, n_sub, kp, wscr);
    __syncthreads();
    // C. merge + softmax
    if (wave < 2) {
        const int kind = wave;
        const int n = kind ? A.R : A.W;
        int slot;
        float wt;
        merge_softmax(lists[(kind * 2) * kWave + lane], lists[(kind * 2 + 1) * kWave + lane], kp,
                      n_sub, n, wscr + kWave, wscr, slot, wt);
        fidx[kind * kWave + lane] = slot;
        fwt[kind * kWave + lane] = wt;
        int32_t *out = kind ? A.ridx_out : A.widx_out;
        if (out && lane < n) out[(size_t)bh * n + lane] = slot;
    }
    __syncthreads();
    // D. the write and the read, one wave per 32-column slice
    const __amdgpu_buffer_rsrc_t Mrs =
        make_rsrc(A.M + (size_t)bh * A.N * A.d_v, (uint32_t)((uint64_t)A.N * A.d_v * 4u));
    const unsigned char *vrow = static_cast<const unsigned char *>(A.v) + (size_t)bh * A.d_v * esz;
    const float at = A.a[bh], bt = A.b[bh];
    for (int slice = wave; slice * 32 < A.d_v; slice += 4) {
        const int col = slice * 32 + 4 * (lane & 7);
        scan_token_slice<BF16>(Mrs, A.d_v, col, fidx, fwt, A.W, fidx + kWave, fwt + kWave, A.R,
                               vrow, at, bt, A.o + (size_t)bh * A.d_v);
    }
}

size_t decode_smem_bytes(int n_sub)
{
    return sizeof(float) * 4 * (size_t)n_sub + sizeof(uint64_t) * (4 * kWave + 12 * kWave) +
           sizeof(int32_t) * 2 * kWave + sizeof(float) * 2 * kWave;
}

hipError_t launch_decode(const DecodeArgs &A, bool bf16, hipStream_t stream)
{
    const int64_t blocks = (int64_t)A.B * A.H;
    if (blocks == 0) return hipSuccess;
    const size_t smem = decode_smem_bytes(A.n_sub);
    if (bf16) {
        hipError_t e = hipFuncSetAttribute((const void *)sdm_decode_kernel<true>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(sdm_decode_kernel<true>, dim3((unsigned)blocks), dim3(256), smem, stream, A);
    } else {
        hipError_t e = hipFuncSetAttribute((const void *)sdm_decode_kernel<false>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(sdm_decode_kernel<false>, dim3((unsigned)blocks), dim3(256), smem, stream, A);
    }
    return hipGetLastError();
}

}  // namespace sdm
