// scan_prep.hip -- preparation pass of the lane-parallel scan
// (sdm_scan_lanes.hip): forwarding codes, and the per-token inputs repacked
// into contiguous per-(sequence, head) streams in the order the scan reads
// them.
//
// Forwarding codes.  The scan gathers the rows of token u while the tokens
// just before it have not yet written theirs, so any of u's slots written by
// one of the `window` tokens before it (and, for u's read slots, by u itself)
// must take the freshly written value instead of the gathered one.  For every
// token u and list position j this pass finds:
//     the smallest delta (1 <= delta <= window for write positions,
//     0 <= delta <= window for read positions) such that token u - delta
//     wrote the slot, and the position j' of the slot in that token's write
//     list: code = delta * 64 + j' (window <= 511, so code < 0x7FFF; 0x7FFF
//     for write positions, 0xFFFF for read positions: none);
// and, for write positions, whether a later token up to the end of the scan
// step D - 1 steps after u's (tokens up to K*floor(u/K) + D*K - 1) writes the
// same slot, so this write need not be stored (the later one is; rows read in
// between are forwarded).  Stores of one row are then at least D steps apart,
// which orders them even when different waves issue them.  Slots are
// compared exactly (integers), so the codes are exact.
//
// Streams (chain = b * H + h, one chain contiguous, tokens in order):
//   lane[chain][t][j], j < Q:  {~(write code | read code << 16), w_j, r_j,
//                               write row offset}  (0 weights past W or R;
//                               the code word is inverted so that a zero --
//                               what a load past the end of a buffer returns
//                               -- reads as "none")
//   gofs[chain][t][j]:          byte offsets of write row j and read row j in
//                               the (b, h) memory plus 2^30 (0: no row), so a
//                               zero read past the end maps to an offset at
//                               or beyond 2^31, outside every memory; bit 31
//                               of the write offset set: the write is
//                               superseded (not stored).  The lane record
//                               repeats the write offset without that bit.
//   tok[chain][t][c], c < d_v/4: {a_t, v_t[4c .. 4c+3], b_t} as one 16-byte
//                               record (bf16 v: 2 words) or two (fp32 v:
//                               {a_t, b_t, 0, 0}, then the 4 values)
//
// One workgroup per (b, h, block of 32 tokens).  The write lists of the block
// and of the `window` tokens before it go into an LDS hash table keyed by
// slot (open addressing, linear probing; one bucket per (token, position), so
// a slot written by several tokens has several buckets); every query probes
// for its slot and keeps the latest writer inside its window, so the cost per
// query does not grow with the window.
#include "kernels.h"
#include "device_common.h"

namespace sdm {

constexpr int kPrBlock = 32;      // tokens per workgroup
constexpr int kPrThreads = 256;
constexpr int kPrBatch = 8;       // loads a thread issues together
constexpr int32_t kPrEmpty = INT32_MIN;
constexpr uint32_t kRowBias = 0x40000000u;

int scan_prep_hash_log2(int W, int window, int lookahead)
{
    const int entries = (kPrBlock + window + lookahead) * W;
    int lg = 6;
    while ((1 << lg) < 2 * entries) ++lg;   // load factor <= 1/2
    return lg;
}

__device__ __forceinline__ uint32_t pr_hash(int32_t slot, int lg)
{
    return ((uint32_t)slot * 0x9E3779B1u) >> (32 - lg);
}

__global__ void __launch_bounds__(kPrThreads) scan_prep_kernel(PrepArgs A)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int lg = A.hash_log2;
    const uint32_t hmask = (1u << lg) - 1u;
    int32_t *keys = reinterpret_cast<int32_t *>(smem);
    uint32_t *vals = reinterpret_cast<uint32_t *>(smem + sizeof(int32_t) * (1u << lg));
    const int tid = threadIdx.x;
    const int nblk = (int)((A.T + kPrBlock - 1) / kPrBlock);
    const int64_t ch = blockIdx.x / nblk;
    const int64_t t0 = (int64_t)(blockIdx.x % nblk) * kPrBlock;
    const int64_t bb = ch / A.H, h = ch % A.H;
    const int W = A.W, R = A.R, Q = A.Q, win = A.window;
    const int64_t tlo = t0 - win > 0 ? t0 - win : 0;
    const int64_t thi = t0 + kPrBlock < A.T ? t0 + kPrBlock : A.T;
    const int64_t look = (int64_t)A.lookahead;   // tokens past the block in the table
    const int64_t tend = thi + look < A.T ? thi + look : A.T;
    const int nrows = (int)(tend - tlo);
    const uint32_t rowb = (uint32_t)A.d_v * 4u;
    auto row_of = [&](int64_t t) { return (bb * A.T + t) * A.H + h; };

    for (uint32_t e = tid; e <= hmask; e += kPrThreads) keys[e] = kPrEmpty;
    // each thread's slots of kPrBatch entries are loaded together before any
    // of them is inserted (the loads are in flight at once); the first batch
    // is loaded while the table is cleared
    const int nins = nrows * W;
    int32_t sl[kPrBatch];
    auto load_batch = [&](int e0) {
#pragma unroll
        for (int u = 0; u < kPrBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            const int r = e / W, j = e - r * W;
            sl[u] = e < nins ? A.widx[row_of(tlo + r) * W + j] : 0;
        }
    };
    load_batch(tid);
    __syncthreads();
    for (int e0 = tid; e0 < nins; e0 += kPrThreads * kPrBatch) {
        if (e0 != tid) load_batch(e0);
#pragma unroll
        for (int u = 0; u < kPrBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            if (e >= nins) break;
            const int r = e / W, j = e - r * W;
            uint32_t b = pr_hash(sl[u], lg);
            while (true) {
                const int32_t old = atomicCAS(&keys[b], kPrEmpty, sl[u]);
                if (old == kPrEmpty) {
                    vals[b] = ((uint32_t)r << 6) | (uint32_t)j;
                    break;
                }
                b = (b + 1) & hmask;
            }
        }
    }
    __syncthreads();
    // latest writer of `slot` among local tokens [lo, hi] (local = t - tlo), as
    // (local token << 6 | position), or -1
    auto latest = [&](int32_t slot, int lo, int hi) {
        int best = -1;
        uint32_t b = pr_hash(slot, lg);
        while (true) {
            const int32_t k = keys[b];
            if (k == kPrEmpty) break;
            if (k == slot) {
                const int v = (int)vals[b];
                const int r = v >> 6;
                if (r >= lo && r <= hi && v > best) best = v;
            }
            b = (b + 1) & hmask;
        }
        return best;
    };
    const int ntok = (int)(thi - t0);
    // (token, position) queries, kPrBatch per thread at a time: their inputs
    // are loaded together, then the table is probed and the records written
    const int nq = ntok * Q;
    for (int e0 = tid; e0 < nq; e0 += kPrThreads * kPrBatch) {
        int32_t ws[kPrBatch], rs[kPrBatch];
        float wv[kPrBatch], rv[kPrBatch];
#pragma unroll
        for (int u = 0; u < kPrBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            const int tl = e / Q, j = e - tl * Q;
            const int64_t row = row_of(t0 + tl);
            const bool okw = e < nq && j < W, okr = e < nq && j < R;
            ws[u] = okw ? A.widx[row * W + j] : 0;
            wv[u] = okw ? A.wwt[row * W + j] : 0.f;
            rs[u] = okr ? A.ridx[row * R + j] : 0;
            rv[u] = okr ? A.rwt[row * R + j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kPrBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            if (e >= nq) break;
            const int tl = e / Q, j = e - tl * Q;
            const int64_t t = t0 + tl;
            const int ul = (int)(t - tlo);              // local index of this token
            const int lo = ul - win > 0 ? ul - win : 0;
            uint32_t cw = 0x7FFFu, cr = 0xFFFFu, gw = 0u, gr = 0u;
            if (j < W) {
                const int v = latest(ws[u], lo, ul - 1);
                if (v >= 0) cw = (uint32_t)((ul - (v >> 6)) * 64 + (v & 63));
                const int64_t last = (t / A.K) * A.K + look;   // <= t + look
                const int hi = (int)((last < tend - 1 ? last : tend - 1) - tlo);
                gw = (uint32_t)ws[u] * rowb + kRowBias;
                if (hi > ul && latest(ws[u], ul + 1, hi) >= 0) gw |= 0x80000000u;
            }
            if (j < R) {
                const int v = latest(rs[u], lo, ul);
                if (v >= 0) cr = (uint32_t)((ul - (v >> 6)) * 64 + (v & 63));
                gr = (uint32_t)rs[u] * rowb + kRowBias;
            }
            const int64_t s = (ch * A.T + t) * Q + j;
            A.st.lane[s] = make_uint4(~(cw | (cr << 16)), __float_as_uint(wv[u]), __float_as_uint(rv[u]),
                                      gw & 0x7FFFFFFFu);
            A.st.gofs[s] = make_uint2(gw, gr);
        }
    }
    // token records: a_t and the 4-column chunks of v_t (kPrBatch per thread
    // at a time, loads first)
    const int nchunk = A.d_v / 4;
    const int nt = ntok * nchunk;
    for (int e0 = tid; e0 < nt; e0 += kPrThreads * kPrBatch) {
        uint32_t av[kPrBatch], bv[kPrBatch];
        uint4 vv[kPrBatch];
#pragma unroll
        for (int u = 0; u < kPrBatch; ++u) {
            const int e = min(e0 + u * kPrThreads, nt - 1);
            const int tl = e / nchunk, c = e - tl * nchunk;
            const int64_t row = row_of(t0 + tl);
            av[u] = __float_as_uint(A.a[row]);
            bv[u] = __float_as_uint(A.b[row]);
            if (A.bf16) {
                const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(A.v) + row * A.d_v + 4 * c);
                vv[u] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                vv[u] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(A.v) + row * A.d_v + 4 * c);
            }
        }
#pragma unroll
        for (int u = 0; u < kPrBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            if (e >= nt) break;
            const int tl = e / nchunk, c = e - tl * nchunk;
            const int64_t s = (ch * A.T + t0 + tl) * nchunk + c;
            if (A.bf16) {
                A.st.tok[s] = make_uint4(av[u], vv[u].x, vv[u].y, bv[u]);
            } else {
                A.st.tok[2 * s] = make_uint4(av[u], bv[u], 0u, 0u);
                A.st.tok[2 * s + 1] = vv[u];
            }
        }
    }
}

hipError_t launch_scan_prep(const PrepArgs &A, hipStream_t stream)
{
    if (A.window < 0 || A.window > 511 || A.W > 64 || A.R > 64 || A.Q > 64 || A.hash_log2 > 14 ||
        A.K < 1 || kPrBlock % A.K != 0 || A.lookahead < A.K - 1 || A.lookahead > 511)
        return hipErrorInvalidValue;
    const int64_t nblk = (A.T + kPrBlock - 1) / kPrBlock;
    const int64_t grid = A.B * A.H * nblk;
    if (grid == 0) return hipSuccess;
    const size_t smem = (sizeof(int32_t) + sizeof(uint32_t)) * ((size_t)1 << A.hash_log2);
    hipError_t e = hipFuncSetAttribute((const void *)scan_prep_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_prep_kernel, dim3((unsigned)grid), dim3(kPrThreads), smem, stream, A);
    return hipGetLastError();
}

}  // namespace sdm
