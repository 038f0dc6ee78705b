// sdm_state_init.hip -- copy the learned initial memory M0 [H,N,d_v] into
// every sequence's state M [B,H,N,d_v].
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 "Learned Initial State" (M0 is a parameter shared by all
// sequences, used as each sequence's starting memory).
//
// Each 16-byte chunk of M0 is read once and written B times, so the traffic is
// (1 + B) x |M0| instead of 2B x |M0| for B separate copies.
#include "kernels.h"
#include "device_common.h"

namespace sdm {

// per_seq is a multiple of 4 and both pointers are 16-byte aligned (checked
// by the caller).
__global__ void __launch_bounds__(256) sdm_state_init_kernel(InitArgs A)
{
    const int64_t n4 = A.per_seq / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(A.M0);
    f32x4 *dst = reinterpret_cast<f32x4 *>(A.M);
    // copies in a block-rotated order (copy (k + blockIdx.x) mod B k-th), so
    // that the stores in flight at any moment spread over all B copies (the
    // copies of one chunk are a large power-of-two stride apart and would
    // otherwise tend to hit the same HBM channel together)
    const uint32_t nb = (uint32_t)A.B;   // B < 2^31 (checked by the caller)
    const uint32_t b0 = blockIdx.x % nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const f32x4 x = __builtin_nontemporal_load(src + i);
        uint32_t b = b0;
        for (uint32_t k = 0; k < nb; ++k) {
            __builtin_nontemporal_store(x, dst + (int64_t)b * n4 + i);
            b = b + 1u == nb ? 0u : b + 1u;
        }
    }
}

hipError_t launch_state_init(const InitArgs &A, hipStream_t stream)
{
    if (A.B == 0 || A.per_seq == 0) return hipSuccess;
    const int64_t n4 = A.per_seq / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;   // one 16-byte chunk per thread, then a grid-stride loop
    hipLaunchKernelGGL(sdm_state_init_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, A);
    return hipGetLastError();
}

}  // namespace sdm
