// scan_hazard.hip -- forwarding codes for the pipelined scan.
//
// The pipelined scan gathers the rows of token u while the D-1 tokens before
// it have not yet written theirs, so any of u's slots written by one of those
// tokens (and, for u's read slots, by u itself) must take the freshly written
// value instead of the gathered one.  This pass finds, for every token u and
// every list position p (write positions 0..W-1, read positions W..W+R-1):
//     the smallest delta (1 <= delta <= window for write positions,
//     0 <= delta <= window for read positions) such that token u-delta wrote
//     the slot, and the position j' of the slot in that token's write list.
// code = delta * 64 + j'  (0xFFFF: none), and flag[u] = 1 if any code is present.
// Slots are compared exactly (integers), so the codes are exact.
#include "kernels.h"
#include "device_common.h"

namespace sdm {

constexpr int kHzBlock = 16;     // tokens per workgroup
constexpr int kHzMaxWin = 15;    // largest supported window

__global__ void __launch_bounds__(64) scan_hazard_kernel(HazardArgs A)
{
    __shared__ int32_t wl[(kHzBlock + kHzMaxWin) * 64];
    const int lane = lane_id();
    const int nblk = (int)((A.T + kHzBlock - 1) / kHzBlock);
    const int64_t ch = blockIdx.x / nblk;
    const int64_t t0 = (int64_t)(blockIdx.x % nblk) * kHzBlock;
    const int bb = (int)(ch / A.H), h = (int)(ch % A.H);
    const int W = A.W, R = A.R, win = A.window;
    const int64_t tlo = t0 - win > 0 ? t0 - win : 0;
    const int64_t thi = t0 + kHzBlock < A.T ? t0 + kHzBlock : A.T;
    // write lists of tokens [tlo, thi) into LDS, row i <-> token tlo + i
    for (int64_t t = tlo; t < thi; ++t) {
        const int64_t row = ((int64_t)bb * A.T + t) * A.H + h;
        if (lane < W) wl[(t - tlo) * 64 + lane] = A.widx[row * W + lane];
    }
    __syncthreads();
    const int P = W + R;
    for (int64_t t = t0; t < thi; ++t) {
        const int64_t row = ((int64_t)bb * A.T + t) * A.H + h;
        bool any = false;
        for (int p = lane; p < P; p += kWave) {
            const int32_t slot = p < W ? wl[(t - tlo) * 64 + p] : A.ridx[row * R + (p - W)];
            uint32_t code = 0xFFFFu;
            const int dmin = p < W ? 1 : 0;
            for (int d = dmin; d <= win && code == 0xFFFFu; ++d) {
                const int64_t ts = t - d;
                if (ts < 0) break;
                const int32_t *lst = wl + (ts - tlo) * 64;
                for (int j = 0; j < W; ++j)
                    if (lst[j] == slot) {
                        code = (uint32_t)(d * 64 + j);
                        break;
                    }
            }
            A.codes[row * P + p] = (uint16_t)code;
            any |= code != 0xFFFFu;
        }
        const bool f = __ballot(any) != 0;
        if (lane == 0) A.flags[row] = f ? 1 : 0;
    }
}

hipError_t launch_scan_hazard(const HazardArgs &A, hipStream_t stream)
{
    if (A.window > kHzMaxWin || A.W > 64) return hipErrorInvalidValue;
    const int64_t nblk = (A.T + kHzBlock - 1) / kHzBlock;
    const int64_t grid = A.B * A.H * nblk;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(scan_hazard_kernel, dim3((unsigned)grid), dim3(64), 0, stream, A);
    return hipGetLastError();
}

}  // namespace sdm
