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
//
// One workgroup per (b, h, block of 32 tokens); one thread per (token,
// position).  The write lists of the block and of the `window` tokens before
// it sit in LDS; each thread scans the window from the farthest token to the
// nearest, so the last match it records is the latest writer, with no
// data-dependent loop exits.
#include "kernels.h"
#include "device_common.h"

namespace sdm {

constexpr int kHzBlock = 32;     // tokens per workgroup
constexpr int kHzMaxWin = 15;    // largest supported window
constexpr int kHzThreads = 256;

__global__ void __launch_bounds__(kHzThreads) scan_hazard_kernel(HazardArgs A)
{
    __shared__ int32_t wl[(kHzBlock + kHzMaxWin) * 64];   // write lists, row stride 64
    __shared__ uint32_t anyhz[kHzBlock];
    const int tid = threadIdx.x;
    const int nblk = (int)((A.T + kHzBlock - 1) / kHzBlock);
    const int64_t ch = blockIdx.x / nblk;
    const int64_t t0 = (int64_t)(blockIdx.x % nblk) * kHzBlock;
    const int bb = (int)(ch / A.H), h = (int)(ch % A.H);
    const int W = A.W, R = A.R, P = W + R, win = A.window;
    const int64_t tlo = t0 - win > 0 ? t0 - win : 0;
    const int64_t thi = t0 + kHzBlock < A.T ? t0 + kHzBlock : A.T;
    const int nrows = (int)(thi - tlo);
    for (int e = tid; e < nrows * W; e += kHzThreads) {
        const int r = e / W, j = e - r * W;
        const int64_t row = ((int64_t)bb * A.T + tlo + r) * A.H + h;
        wl[r * 64 + j] = A.widx[row * W + j];
    }
    if (tid < kHzBlock) anyhz[tid] = 0;
    __syncthreads();
    const int ntok = (int)(thi - t0);
    for (int e = tid; e < ntok * P; e += kHzThreads) {
        const int tl = e / P, p = e - tl * P;
        const int64_t t = t0 + tl;
        const int64_t row = ((int64_t)bb * A.T + t) * A.H + h;
        const int32_t slot = p < W ? wl[(t - tlo) * 64 + p] : A.ridx[row * R + (p - W)];
        const int dmin = p < W ? 1 : 0;
        int dmax = win;
        if (t - dmax < 0) dmax = (int)t;
        uint32_t code = 0xFFFFu;
        for (int d = dmax; d >= dmin; --d) {
            const int32_t *lst = wl + (t - d - tlo) * 64;
            int jm = -1;
            for (int j = 0; j < W; ++j) jm = lst[j] == slot ? j : jm;
            code = jm >= 0 ? (uint32_t)(d * 64 + jm) : code;
        }
        A.codes[row * P + p] = (uint16_t)code;
        if (code != 0xFFFFu) atomicOr(&anyhz[tl], 1u);
    }
    __syncthreads();
    if (tid < ntok) {
        const int64_t row = ((int64_t)bb * A.T + t0 + tid) * A.H + h;
        A.flags[row] = anyhz[tid];
    }
}

hipError_t launch_scan_hazard(const HazardArgs &A, hipStream_t stream)
{
    if (A.window > kHzMaxWin || A.W > 64) return hipErrorInvalidValue;
    const int64_t nblk = (A.T + kHzBlock - 1) / kHzBlock;
    const int64_t grid = A.B * A.H * nblk;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(scan_hazard_kernel, dim3((unsigned)grid), dim3(kHzThreads), 0, stream, A);
    return hipGetLastError();
}

}  // namespace sdm
