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
//                               or beyond 2^31, outside every memory (one
//                               memory is at most 2 GiB, so offset + 2^30
//                               stays below 2^32); bit 0 of the write offset
//                               set: the write is superseded (not stored).
//                               Row offsets are multiples of d_v * 4 >= 128,
//                               so bit 0 is free.  The lane record repeats
//                               the write offset without that bit.
//   tok[chain][t][c], c < d_v/4: {a_t, v_t[4c .. 4c+3], b_t} as one 16-byte
//                               record (bf16 v: 2 words) or two (fp32 v:
//                               {a_t, b_t, 0, 0}, then the 4 values); when
//                               the caller passes the gates' pre-activations,
//                               a_t and b_t are formed here (gates_math.h)
//
// One workgroup per (b, h, block of 32 tokens).  The write lists of the block,
// of the `window` tokens before it and of the look-ahead after it go into an
// LDS hash table keyed by slot, with chained buckets: entry (local token r,
// position j) sits at index r * Q + j of an entry array holding its slot and
// the next entry of its bucket, and is put at the head of its bucket with one
// atomic exchange (no retries, so a thread's inserts are all in flight at
// once).  Every query walks its slot's bucket and keeps the latest writer
// inside its window, so the cost per query does not grow with the window; a
// thread walks the buckets of its queries together.
#include "kernels.h"
#include "device_common.h"
#include "gates_math.h"

namespace sdm {

constexpr int kPrBlock = 32;      // tokens per workgroup
constexpr int kPrThreads = 256;
constexpr int kPrBatch = 8;       // slots to insert a thread loads together
constexpr int kPrQBatch = 4;      // queries (and token records) a thread loads together
constexpr uint32_t kPrNone = 0xFFFFFFFFu;   // end of a bucket's chain
constexpr uint32_t kRowBias = 0x40000000u;

int scan_prep_hash_log2(int W, int window, int lookahead)
{
    const int entries = (kPrBlock + window + lookahead) * W;
    int lg = 6;
    while ((1 << lg) < 2 * entries) ++lg;   // at least two buckets per entry
    return lg;
}

// bucket heads, then the entries {slot, next entry of the bucket}
static size_t scan_prep_smem(const PrepArgs &A)
{
    return sizeof(uint32_t) * ((size_t)1 << A.hash_log2) +
           sizeof(uint2) * (size_t)(kPrBlock + A.window + A.lookahead) * (size_t)A.Q;
}

__device__ __forceinline__ uint32_t pr_hash(int32_t slot, int lg)
{
    return ((uint32_t)slot * 0x9E3779B1u) >> (32 - lg);
}

__global__ void __launch_bounds__(kPrThreads) scan_prep_kernel(PrepArgs A)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int lg = A.hash_log2;
    const uint32_t nbucket = 1u << lg;
    uint32_t *heads = reinterpret_cast<uint32_t *>(smem);
    uint2 *ent = reinterpret_cast<uint2 *>(smem + sizeof(uint32_t) * nbucket);
    const int qlog = __builtin_ctz((unsigned)A.Q);   // Q is a power of two
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

    const int ntok = (int)(thi - t0);
    const int nq = ntok * Q;               // (token, position) queries
    const int nchunk = A.d_v / 4;
    const int nt = ntok * nchunk;          // token records
    // Every load of the first batch of each phase (the slots to insert, the
    // query inputs, the token records) is issued before the table is
    // cleared, so the workgroup waits for one round trip instead of three.
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
    int32_t ws[kPrQBatch], rs[kPrQBatch];
    float wv[kPrQBatch], rv[kPrQBatch];
    auto load_queries = [&](int e0) {
#pragma unroll
        for (int u = 0; u < kPrQBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            const int tl = e / Q, j = e - tl * Q;
            const int64_t row = row_of(t0 + (e < nq ? tl : 0));
            const bool okw = e < nq && j < W, okr = e < nq && j < R;
            ws[u] = okw ? A.widx[row * W + j] : 0;
            wv[u] = okw ? A.wwt[row * W + j] : 0.f;
            rs[u] = okr ? A.ridx[row * R + j] : 0;
            rv[u] = okr ? A.rwt[row * R + j] : 0.f;
        }
    };
    uint32_t av[kPrQBatch], bv[kPrQBatch];
    uint4 vv[kPrQBatch];
    auto load_records = [&](int e0) {
#pragma unroll
        for (int u = 0; u < kPrQBatch; ++u) {
            const int e = min(e0 + u * kPrThreads, nt - 1);
            const int tl = e / nchunk, c = e - tl * nchunk;
            const int64_t row = row_of(t0 + tl);
            if (A.A_decay) {   // the gates from their pre-activations
                av[u] = __float_as_uint(gate_decay(A.a[row], A.dt_bias[h], A.A_decay[h]));
                bv[u] = __float_as_uint(gate_sigmoid(A.b[row]));
            } else {
                av[u] = __float_as_uint(A.a[row]);
                bv[u] = __float_as_uint(A.b[row]);
            }
            if (A.bf16) {
                const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(A.v) + row * A.d_v + 4 * c);
                vv[u] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                vv[u] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(A.v) + row * A.d_v + 4 * c);
            }
        }
    };
    load_batch(tid);
    load_queries(tid);
    load_records(tid);
    for (uint32_t e = tid; e < nbucket; e += kPrThreads) heads[e] = kPrNone;
    __syncthreads();
    for (int e0 = tid; e0 < nins; e0 += kPrThreads * kPrBatch) {
        if (e0 != tid) load_batch(e0);
#pragma unroll
        for (int u = 0; u < kPrBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            if (e >= nins) break;
            const int r = e / W, j = e - r * W;
            const uint32_t idx = ((uint32_t)r << qlog) | (uint32_t)j;
            ent[idx].x = (uint32_t)sl[u];
            ent[idx].y = atomicExch(&heads[pr_hash(sl[u], lg)], idx);
        }
    }
    __syncthreads();
    for (int e0 = tid; e0 < nq; e0 += kPrThreads * kPrQBatch) {
        if (e0 != tid) load_queries(e0);
        // per query: the chains of its write slot and of its read slot; the
        // latest earlier writer of each inside the window (entry index, or
        // -1), and whether the write slot is written again in the look-ahead
        uint32_t cw[kPrQBatch], cr[kPrQBatch];
        int bw[kPrQBatch], br[kPrQBatch], ul[kPrQBatch], lo[kPrQBatch], hi[kPrQBatch];
        bool later[kPrQBatch];
#pragma unroll
        for (int u = 0; u < kPrQBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            const int tl = e / Q, j = e - tl * Q;
            const int64_t t = t0 + tl;
            ul[u] = (int)(t - tlo);
            lo[u] = ul[u] - win > 0 ? ul[u] - win : 0;
            const int64_t last = (t / A.K) * A.K + look;   // <= t + look
            hi[u] = (int)((last < tend - 1 ? last : tend - 1) - tlo);
            cw[u] = e < nq && j < W ? heads[pr_hash(ws[u], lg)] : kPrNone;
            cr[u] = e < nq && j < R ? heads[pr_hash(rs[u], lg)] : kPrNone;
            bw[u] = br[u] = -1;
            later[u] = false;
        }
        while (true) {
            uint2 ew[kPrQBatch], er[kPrQBatch];
#pragma unroll
            for (int u = 0; u < kPrQBatch; ++u) {
                ew[u] = ent[cw[u] == kPrNone ? 0u : cw[u]];
                er[u] = ent[cr[u] == kPrNone ? 0u : cr[u]];
            }
            bool more = false;
#pragma unroll
            for (int u = 0; u < kPrQBatch; ++u) {
                if (cw[u] != kPrNone) {
                    if ((int32_t)ew[u].x == ws[u]) {
                        const int r = (int)(cw[u] >> qlog);
                        if (r >= lo[u] && r < ul[u] && (int)cw[u] > bw[u]) bw[u] = (int)cw[u];
                        if (r > ul[u] && r <= hi[u]) later[u] = true;
                    }
                    cw[u] = ew[u].y;
                }
                if (cr[u] != kPrNone) {
                    if ((int32_t)er[u].x == rs[u]) {
                        const int r = (int)(cr[u] >> qlog);
                        if (r >= lo[u] && r <= ul[u] && (int)cr[u] > br[u]) br[u] = (int)cr[u];
                    }
                    cr[u] = er[u].y;
                }
                more = more || cw[u] != kPrNone || cr[u] != kPrNone;
            }
            if (!more) break;
        }
#pragma unroll
        for (int u = 0; u < kPrQBatch; ++u) {
            const int e = e0 + u * kPrThreads;
            if (e >= nq) break;
            const int tl = e / Q, j = e - tl * Q;
            const int64_t t = t0 + tl;
            uint32_t code_w = 0x7FFFu, code_r = 0xFFFFu, gw = 0u, gr = 0u;
            if (j < W) {
                if (bw[u] >= 0) code_w = (uint32_t)((ul[u] - (bw[u] >> qlog)) * 64 + (bw[u] & (Q - 1)));
                gw = (uint32_t)ws[u] * rowb + kRowBias;
                if (later[u]) gw |= 1u;
            }
            if (j < R) {
                if (br[u] >= 0) code_r = (uint32_t)((ul[u] - (br[u] >> qlog)) * 64 + (br[u] & (Q - 1)));
                gr = (uint32_t)rs[u] * rowb + kRowBias;
            }
            const int64_t s = (ch * A.T + t) * Q + j;
            A.st.lane[s] = make_uint4(~(code_w | (code_r << 16)), __float_as_uint(wv[u]), __float_as_uint(rv[u]),
                                      gw & ~1u);
            A.st.gofs[s] = make_uint2(gw, gr);
        }
    }
    // token records: a_t and the 4-column chunks of v_t
    for (int e0 = tid; e0 < nt; e0 += kPrThreads * kPrQBatch) {
        if (e0 != tid) load_records(e0);
#pragma unroll
        for (int u = 0; u < kPrQBatch; ++u) {
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
    if (A.window < 0 || A.window > 511 || A.W > 64 || A.R > 64 || A.Q > 64 || (A.Q & (A.Q - 1)) != 0 ||
        A.Q < A.W || A.Q < A.R || A.hash_log2 > 14 ||
        A.K < 1 || kPrBlock % A.K != 0 || A.lookahead < A.K - 1 || A.lookahead > 511)
        return hipErrorInvalidValue;
    const int64_t nblk = (A.T + kPrBlock - 1) / kPrBlock;
    const int64_t grid = A.B * A.H * nblk;
    if (grid == 0) return hipSuccess;
    const size_t smem = scan_prep_smem(A);
    if (smem > 160 * 1024) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void *)scan_prep_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_prep_kernel, dim3((unsigned)grid), dim3(kPrThreads), smem, stream, A);
    return hipGetLastError();
}

}  // namespace sdm
