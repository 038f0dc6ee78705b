// sdm_scan.hip -- prefill scan: the sequence-serial sparse gated delta rule
// over T tokens for every (sequence, head), in place on the HBM-resident
// memory.  "Sparse Delta Memory: Scaling the State of Linear RNNs through
// Sparsity", Sec. 3.1 steps 2-3 (Eq. 4).
//
// Work unit: one wave per (b, h, 32-column slice).  Columns never interact,
// so the d_v/32 slices of one memory are independent recurrences over the
// same slot lists; each wave walks its tokens in order.
#include "kernels.h"
#include "scan_step.h"

namespace sdm {

template <bool BF16>
__global__ void __launch_bounds__(64) sdm_scan_serial_kernel(ScanArgs A)
{
    const int nslice = A.d_v / 32;
    const int unit = blockIdx.x;
    const int slice = unit % nslice;
    const int ch = unit / nslice;
    const int bb = ch / A.H, h = ch - bb * A.H;
    const int lane = lane_id();
    const int col = slice * 32 + 4 * (lane & 7);
    const size_t esz = BF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t Mrs =
        make_rsrc(A.M + (size_t)ch * A.N * A.d_v, (uint32_t)((uint64_t)A.N * A.d_v * 4u));
    for (int64_t t = 0; t < A.T; ++t) {
        const int64_t row = (bb * A.T + t) * A.H + h;
        scan_token_slice<BF16>(Mrs, A.d_v, col, A.widx + row * A.W, A.wwt + row * A.W, A.W,
                               A.ridx + row * A.R, A.rwt + row * A.R, A.R,
                               static_cast<const unsigned char *>(A.v) + row * A.d_v * esz,
                               A.a[row], A.b[row], A.o + row * A.d_v);
    }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the pipelined scan: forwarding codes [B,T,H,W+R] (uint16) and
// per-token hazard flags [B,T,H] (uint32).  The serial kernel needs none.
size_t scan_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int)
{
    if (scan_pipe_depth(W, R) == 0) return 0;
    const size_t rows = (size_t)(B * T * H);
    return align256(rows * (size_t)(W + R) * 2) + align256(rows * 4);
}

hipError_t launch_scan(const ScanArgs &A, bool bf16, void *ws, size_t, hipStream_t stream)
{
    const int64_t units = A.B * A.H * (A.d_v / 32);
    if (units == 0 || A.T == 0) return hipSuccess;
    const int D = scan_pipe_depth(A.W, A.R);
    if (D > 0) {
        const size_t rows = (size_t)(A.B * A.T * A.H);
        uint16_t *codes = static_cast<uint16_t *>(ws);
        uint32_t *flags = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(ws) +
                                                       align256(rows * (size_t)(A.W + A.R) * 2));
        HazardArgs hz{A.widx, A.ridx, codes, flags, A.B, A.T, A.H, A.W, A.R, D - 1};
        hipError_t e = launch_scan_hazard(hz, stream);
        if (e != hipSuccess) return e;
        return launch_scan_pipe(A, bf16, codes, flags, stream);
    }
    if (bf16)
        hipLaunchKernelGGL(sdm_scan_serial_kernel<true>, dim3((unsigned)units), dim3(64), 0, stream, A);
    else
        hipLaunchKernelGGL(sdm_scan_serial_kernel<false>, dim3((unsigned)units), dim3(64), 0, stream, A);
    return hipGetLastError();
}

}  // namespace sdm
