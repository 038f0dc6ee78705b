// sdm_scan_bwd_lanes.hip -- reverse-mode gradients of the prefill scan, many
// tokens in flight.
//
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 steps 2-3 (Eq. 4), differentiated with the chain rule (the pages
// print no backward pass).  With G = dL/dM, for each token t in reverse:
//     read part:   G[r_i] += r_i do_t                                 (i < R)
//     write part:  Y_j = G[s_j];  du = b sum_j w_j Y_j;  dp = -a du;
//                  G[s_j] = a Y_j + w_j dp                             (j < W)
// and the gradients of the token's inputs
//     dv = du;  dw_j = b <Y_j, u> + <dp, X_j>;  da = sum_j <Y_j, X_j> - <p, du>;
//     db = sum_j w_j <Y_j, u>;  dr_i = <do, Z_i>
// with p = sum_j w_j X_j, u = v - a p, X_j the write rows before the
// forward's write and Z_i the read rows after it (saved by the forward).
//
// Both parts of a token overwrite rows of G, and G's columns never interact.
// In processing order -- sub-token 2 (T - 1 - t) is the read part of token
// t, the next one its write part -- the parts form one sequence of row
// updates of the same per-column kind the forward scan runs (the write part
// is the forward's row update with v = 0), so the forward's structure
// carries over (sdm_scan_lanes.hip):
//   - a preparation pass (scan_bwd_prep_kernel) finds, for every sub-token
//     and list position, the latest earlier sub-token inside the window that
//     updated the same slot (an exact forwarding code), whether a later one
//     inside the look-ahead supersedes this update (then it is not stored),
//     and repacks the per-token inputs into contiguous per-chain streams;
//   - the lane-parallel kernel (sdm_scan_bwd_lanes_kernel) advances K = 64/Q
//     sub-tokens per step, one wave per 4-column chunk, G waves per row
//     segment; it gathers the rows of step s + D at the end of step s into
//     LDS, takes rows updated in between from an LDS ring of the last 2D
//     steps' rows, and runs sub-tokens of one step that depend on each other
//     in rounds;
//   - dw_j, da and db are sums over all d_v columns, held by many waves:
//     each wave stores its chunk's partial sums per token (with 8-wave
//     workgroups, the waves first add their parts through LDS and the
//     workgroup stores its row segment's), and scan_bwd_reduce_kernel adds
//     them in a fixed order; it also forms dr_i = <do, Z_i> from the saved
//     read rows.
// A read slot listed at several positions of one token: its last position
// carries the sum of their weights (in list order) and the earlier positions
// are not stored, so G receives the term once.  Every sum has a fixed order:
// results are deterministic.
#include "kernels.h"
#include "lanes_common.h"
#include "scan_lanes.h"

namespace sdm {

using namespace lanes;

namespace {

constexpr int kBpBlock = 32;      // sub-tokens per preparation workgroup
constexpr int kBpThreads = 256;
constexpr int kBpBatch = 8;       // slots to insert a thread loads together
constexpr int kBpQBatch = 4;      // queries (and sub-token records) a thread loads together
constexpr uint32_t kBpNone = 0xFFFFFFFFu;   // end of a bucket's chain

struct BwdStreams {
    uint2 *lane;      // [chain][u][Q]: {~forwarding code, weight}
    uint32_t *gofs;   // [chain][u][Q]: row byte offset + 2^30 (0: no row), bit 0 = superseded
    uint4 *tok;       // [chain][u][d_v/4][NTR]: read part {do chunk};
                      //   write part {a, v chunk, b} (bf16 v) or {a, b, 0, 0}{v chunk} (fp32 v)
    float *part;      // [chain][T][nseg][Q + 2]: dw_j parts (j < W), then the da and db parts, per
                      //   row segment (workgroup) when G = 8, else per 4-column chunk
};

struct BwdPrepArgs {
    const int32_t *widx, *ridx;
    const float *wwt, *rwt, *a, *b, *dout;
    const void *v;
    BwdStreams st;
    int64_t B, T, H;
    int W, R, Q, K, window, lookahead, hash_log2, d_v, bf16;
};

__device__ __forceinline__ uint32_t bp_hash(int32_t slot, int lg)
{
    return ((uint32_t)slot * 0x9E3779B1u) >> (32 - lg);
}

// sub-token u: token T - 1 - u/2, its read list (u even) or write list (u
// odd).  Plain functions of values: a list length selected between two
// variables that a lambda holds (by reference or by value) compiles to a
// two-entry table in scratch memory and a dependent load per use.
__device__ __forceinline__ int64_t bp_row(int64_t u, int64_t bb, int64_t T, int64_t H, int64_t h)
{
    return (bb * T + (T - 1 - (u >> 1))) * H + h;
}

__device__ __forceinline__ int bp_len(int64_t u, int W, int R)
{
    return (u & 1) ? W : R;
}

// Preparation pass.  One workgroup per (chain, block of 32 sub-tokens).  The
// lists of the block, of the `window` sub-tokens before it and of the
// `lookahead` sub-tokens after it go into an LDS hash table keyed by slot,
// with chained buckets: entry (local sub-token r, position j) sits at index
// r * Q + j of an entry array holding its slot and the next entry of its
// bucket, and is put at the head of its bucket with one atomic exchange.
// Each (sub-token, position) query walks its slot's bucket once; a thread
// walks the buckets of its queries together.
__global__ void __launch_bounds__(kBpThreads) scan_bwd_prep_kernel(BwdPrepArgs A)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int lg = A.hash_log2;
    const uint32_t nbucket = 1u << lg;
    uint32_t *heads = reinterpret_cast<uint32_t *>(smem);
    uint2 *ent = reinterpret_cast<uint2 *>(smem + sizeof(uint32_t) * nbucket);
    const int qlog = __builtin_ctz((unsigned)A.Q);   // Q is a power of two
    const int tid = threadIdx.x;
    const int64_t U = 2 * A.T;
    const int64_t nblk = (U + kBpBlock - 1) / kBpBlock;
    const int64_t ch = blockIdx.x / nblk;
    const int64_t u0 = (blockIdx.x % nblk) * kBpBlock;
    const int64_t bb = ch / A.H, h = ch % A.H;
    const int W = A.W, R = A.R, Q = A.Q, win = A.window;
    const int64_t ulo = u0 - win > 0 ? u0 - win : 0;
    const int64_t uhi = u0 + kBpBlock < U ? u0 + kBpBlock : U;
    const int64_t uend = uhi + A.lookahead < U ? uhi + A.lookahead : U;
    const int nsub = (int)(uend - ulo);
    const uint32_t rowb = (uint32_t)A.d_v * 4u;
    const int64_t T = A.T, H = A.H;
    auto row_of = [bb, T, H, h](int64_t u) { return bp_row(u, bb, T, H, h); };
    auto len_of = [W, R](int64_t u) { return bp_len(u, W, R); };

    const int ntok = (int)(uhi - u0);
    const int nq = ntok * Q;               // (sub-token, position) queries
    const int nchunk = A.d_v / 4;
    const int nt = ntok * nchunk;          // sub-token records
    // The first batch of each phase's loads (the slots to insert, the query
    // inputs, the sub-token records) is issued before the table is cleared,
    // so the workgroup waits for one round trip instead of three.
    const int nins = nsub * Q;
    int32_t sl[kBpBatch];
    auto load_batch = [&](int e0) {
#pragma unroll
        for (int k = 0; k < kBpBatch; ++k) {
            const int e = e0 + k * kBpThreads;
            const int r = e / Q, j = e - r * Q;
            const int64_t u = ulo + r;
            const bool ok = e < nins && j < len_of(u);
            const int64_t row = row_of(ok ? u : ulo);
            sl[k] = ok ? ((u & 1) ? A.widx[row * W + j] : A.ridx[row * R + j]) : 0;
        }
    };
    int32_t ss[kBpQBatch];
    float wv[kBpQBatch];
    auto load_queries = [&](int e0) {
#pragma unroll
        for (int k = 0; k < kBpQBatch; ++k) {
            const int e = e0 + k * kBpThreads;
            const int tl = e / Q, j = e - tl * Q;
            const int64_t u = u0 + tl;
            const bool on = e < nq && j < len_of(u);
            const int64_t row = row_of(on ? u : u0);
            ss[k] = on ? ((u & 1) ? A.widx[row * W + j] : A.ridx[row * R + j]) : 0;
            wv[k] = on ? ((u & 1) ? A.wwt[row * W + j] : A.rwt[row * R + j]) : 0.f;
        }
    };
    uint4 r0[kBpQBatch], r1[kBpQBatch];
    auto load_records = [&](int e0) {
#pragma unroll
        for (int k = 0; k < kBpQBatch; ++k) {
            const int e = min(e0 + k * kBpThreads, nt - 1);
            const int tl = e / nchunk, c = e - tl * nchunk;
            const int64_t u = u0 + tl;
            const int64_t row = row_of(u);
            if (u & 1) {
                const uint32_t av = __float_as_uint(A.a[row]), bv = __float_as_uint(A.b[row]);
                if (A.bf16) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(A.v) +
                                                                     row * A.d_v + 4 * c);
                    r0[k] = make_uint4(av, v.x, v.y, bv);
                    r1[k] = make_uint4(0u, 0u, 0u, 0u);
                } else {
                    r0[k] = make_uint4(av, bv, 0u, 0u);
                    r1[k] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(A.v) + row * A.d_v + 4 * c);
                }
            } else {
                r0[k] = *reinterpret_cast<const uint4 *>(A.dout + row * A.d_v + 4 * c);
                r1[k] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    load_batch(tid);
    load_queries(tid);
    load_records(tid);
    for (uint32_t e = tid; e < nbucket; e += kBpThreads) heads[e] = kBpNone;
    __syncthreads();
    for (int e0 = tid; e0 < nins; e0 += kBpThreads * kBpBatch) {
        if (e0 != tid) load_batch(e0);
#pragma unroll
        for (int k = 0; k < kBpBatch; ++k) {
            const int e = e0 + k * kBpThreads;   // entry index r * Q + j
            if (e >= nins) break;
            const int r = e / Q, j = e - r * Q;
            if (j >= len_of(ulo + r)) continue;
            ent[e].x = (uint32_t)sl[k];
            ent[e].y = atomicExch(&heads[bp_hash(sl[k], lg)], (uint32_t)e);
        }
    }
    __syncthreads();

    for (int e0 = tid; e0 < nq; e0 += kBpThreads * kBpQBatch) {
        if (e0 != tid) load_queries(e0);
        // per query: the latest earlier entry of its slot inside the window
        // (entry index, or -1); another position of the same sub-token with
        // the slot (dup), a later one (later_same); a later sub-token in the
        // look-ahead with it (later_other)
        uint32_t cur[kBpQBatch];
        int best[kBpQBatch], ul[kBpQBatch], lo[kBpQBatch], hi[kBpQBatch];
        bool later_same[kBpQBatch], later_other[kBpQBatch], dup[kBpQBatch];
#pragma unroll
        for (int k = 0; k < kBpQBatch; ++k) {
            const int e = e0 + k * kBpThreads;
            const int tl = e / Q, j = e - tl * Q;
            const int64_t u = u0 + tl;
            ul[k] = (int)(u - ulo);
            lo[k] = ul[k] - win > 0 ? ul[k] - win : 0;
            // the look-ahead ends with the step D - 1 steps after this one
            const int64_t last = (u / A.K) * A.K + A.lookahead;
            hi[k] = (int)((last < uend - 1 ? last : uend - 1) - ulo);
            cur[k] = e < nq && j < len_of(u) ? heads[bp_hash(ss[k], lg)] : kBpNone;
            best[k] = -1;
            later_same[k] = later_other[k] = dup[k] = false;
        }
        while (true) {
            uint2 en[kBpQBatch];
#pragma unroll
            for (int k = 0; k < kBpQBatch; ++k) en[k] = ent[cur[k] == kBpNone ? 0u : cur[k]];
            bool more = false;
#pragma unroll
            for (int k = 0; k < kBpQBatch; ++k) {
                if (cur[k] != kBpNone) {
                    if ((int32_t)en[k].x == ss[k]) {
                        const int v = (int)cur[k];
                        const int r = v >> qlog, p = v & (Q - 1);
                        const int j = (e0 + k * kBpThreads) & (Q - 1);
                        if (r >= lo[k] && r < ul[k] && v > best[k]) best[k] = v;
                        if (r == ul[k] && p != j) {
                            dup[k] = true;
                            if (p > j) later_same[k] = true;
                        }
                        if (r > ul[k] && r <= hi[k]) later_other[k] = true;
                    }
                    cur[k] = en[k].y;
                }
                more = more || cur[k] != kBpNone;
            }
            if (!more) break;
        }
#pragma unroll
        for (int k = 0; k < kBpQBatch; ++k) {
            const int e = e0 + k * kBpThreads;
            if (e >= nq) break;
            const int tl = e / Q, j = e - tl * Q;
            const int64_t u = u0 + tl;
            uint32_t code = 0x7FFFu, go = 0u;
            float wt = 0.f;
            if (j < len_of(u)) {
                const int32_t slot = ss[k];
                wt = wv[k];
                if (best[k] >= 0) code = (uint32_t)((ul[k] - (best[k] >> qlog)) * 64 + (best[k] & (Q - 1)));
                go = (uint32_t)slot * rowb + kRowBias;
                if (later_same[k] || later_other[k]) go |= 1u;
                if (!(u & 1) && dup[k] && !later_same[k]) {
                    // the last position of a repeated read slot: the sum of
                    // the positions' weights, in list order
                    const int64_t row = row_of(u);
                    float s = 0.f;
                    for (int p = 0; p < R; ++p)
                        if (A.ridx[row * R + p] == slot) s += A.rwt[row * R + p];
                    wt = s;
                }
            }
            const int64_t sidx = (ch * U + u) * Q + j;
            A.st.lane[sidx] = make_uint2(~code, __float_as_uint(wt));
            A.st.gofs[sidx] = go;
        }
    }

    // sub-token records
    for (int e0 = tid; e0 < nt; e0 += kBpThreads * kBpQBatch) {
        if (e0 != tid) load_records(e0);
#pragma unroll
        for (int k = 0; k < kBpQBatch; ++k) {
            const int e = e0 + k * kBpThreads;
            if (e >= nt) break;
            const int tl = e / nchunk, c = e - tl * nchunk;
            const int64_t s = (ch * U + u0 + tl) * nchunk + c;
            if (A.bf16) {
                A.st.tok[s] = r0[k];
            } else {
                A.st.tok[2 * s] = r0[k];
                A.st.tok[2 * s + 1] = r1[k];
            }
        }
    }
}

// Sum over the aligned group of Q lanes holding this lane, in every lane of it.
template <int Q>
__device__ __forceinline__ float group_sum1(float x)
{
    if constexpr (Q >= 2) x += __uint_as_float(lane_xor<1>(__float_as_uint(x)));
    if constexpr (Q >= 4) x += __uint_as_float(lane_xor<2>(__float_as_uint(x)));
    if constexpr (Q >= 8) x += __uint_as_float(lane_xor<4>(__float_as_uint(x)));
    if constexpr (Q >= 16) x += __uint_as_float(lane_xor<8>(__float_as_uint(x)));
    if constexpr (Q >= 32) x += __uint_as_float(lane_xor<16>(__float_as_uint(x)));
    if constexpr (Q >= 64) x += __uint_as_float(lane_xor<32>(__float_as_uint(x)));
    return x;
}

__device__ __forceinline__ float dot4(f32x4 x, f32x4 y)
{
    return __builtin_fmaf(x.w, y.w, __builtin_fmaf(x.z, y.z, __builtin_fmaf(x.y, y.y, x.x * y.x)));
}

__device__ __forceinline__ f32x4 as_f32x4(uint4 r)
{
    return (f32x4){__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w)};
}

}  // namespace

template <int Q, int D, int G, bool BF16>
__global__ void __launch_bounds__(64 * G) sdm_scan_bwd_lanes_kernel(BwdArgs A, BwdStreams S)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int K = kWave / Q;                 // sub-tokens per step
    constexpr int LQ = ilog2(Q), LK = ilog2(K);
    static_assert((1 << LQ) == Q, "Q is a power of two");
    constexpr int NTR = BF16 ? 1 : 2;            // 16-byte token records per chunk
    // vector-memory instructions per step (fixed): the gather, the row
    // offsets, the lane record, NTR token records, the saved row X; the row
    // store, dv, the dw parts, the da and db parts
    constexpr int NVM = 8 + NTR;
    static_assert((D - 1) * NVM <= 63, "pipeline deeper than the vmcnt range");
    static_assert(G == 2 || G == 4 || G == 8, "2, 4 or 8 waves per workgroup");
    constexpr int RPW = kWave / G;               // rows of a step each wave moves
    constexpr int PQ = Q + 2;                    // floats of a partial-sum record
    // 8-wave workgroups add their waves' parts before storing them (an 8x
    // smaller partial-sum stream); narrower ones, whose steps are shorter
    // and latency-bound, store each wave's
    constexpr bool RED = G == 8;

    // Row r of a step is sub-token r / Q, list position r % Q (r = the lane
    // of the compute layout).  Chunk c of row r sits at position (c + r) % G.
    __shared__ f32x4 gath[D][kWave][G];          // gathered rows of the steps in flight
    __shared__ f32x4 ring[2 * D][kWave][G];      // rows updated by the last 2D steps
    __shared__ float red[RED ? G : 1][kWave];    // each wave's dw_j parts of the step (RED)
    __shared__ float red2[RED ? G : 1][K][2];    // each wave's da, db parts per sub-token (RED)

    const uint32_t d_v = (uint32_t)A.d_v;
    const uint32_t nline = d_v / 32u;
    uint32_t grp, mem;
    xcd_decode(blockIdx.x, (uint32_t)(A.B * A.H) * nline, 8u / G, grp, mem);
    const uint32_t chu = __builtin_amdgcn_readfirstlane(grp / nline);
    const uint32_t seg = __builtin_amdgcn_readfirstlane((grp - chu * nline) * (8u / G) + mem);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int64_t ch = chu;
    const int64_t H = A.H, T = A.T, U = 2 * A.T;
    const int64_t bb = ch / H, h = ch - bb * H;
    const int lane = lane_id();
    const int i = lane >> LQ;                                // compute layout: sub-token of the step
    const int j = lane & (Q - 1);                            //   and list position
    const int rg = wave * RPW + lane / G;                   // memory layout: row ...
    const int pg = lane % G;                                //   ... and its position
    const uint32_t cg = (uint32_t)((pg - rg) & (G - 1));    //   = chunk cg of that row
    const uint32_t nchunk = d_v / 4u;
    const uint32_t chunk = seg * G + (uint32_t)wave;
    const uint32_t segb = seg * G * 16u;
    const uint32_t colb = segb + (uint32_t)wave * 16u;
    const uint32_t W = (uint32_t)A.W;
    const __amdgpu_buffer_rsrc_t Mrs =
        make_rsrc(A.dM + (size_t)ch * A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
    // this chain's streams and saved rows, its dv rows and partial sums
    // (every range checked on the host to be < 2 GiB)
    const uint64_t uq = (uint64_t)U * Q;
    const __amdgpu_buffer_rsrc_t R1 = make_rsrc(S.lane + ch * uq, (uint32_t)(uq * 8u));
    const __amdgpu_buffer_rsrc_t R2 = make_rsrc(S.gofs + ch * uq, (uint32_t)(uq * 4u));
    const uint64_t uc = (uint64_t)U * nchunk * NTR;
    const __amdgpu_buffer_rsrc_t R3 = make_rsrc(S.tok + ch * uc, (uint32_t)(uc * 16u));
    const __amdgpu_buffer_rsrc_t Xrs =
        make_rsrc(A.xsave + (size_t)ch * T * W * d_v, (uint32_t)((uint64_t)T * W * d_v * 4u));
    const __amdgpu_buffer_rsrc_t Vrs =
        make_rsrc(A.dv + (size_t)(bb * T * H + h) * d_v, (uint32_t)((uint64_t)((T - 1) * H + 1) * d_v * 4u));
    const uint32_t nseg = RED ? nchunk / G : nchunk;        // partial-sum records per chain and token
    const uint64_t pc = (uint64_t)T * nseg * PQ;
    const __amdgpu_buffer_rsrc_t Prs = make_rsrc(S.part + ch * pc, (uint32_t)(pc * 4u));
    // the step's row whose dw_j parts this lane adds over the waves: row
    // `rsum` (compute-layout lane) of wave lane % G
    const int rsum = wave * (kWave / G) + lane / G;
    const int64_t nsteps = (U + K - 1) / K;

    // running byte offsets of the next loads: lane records and token records
    // of step s + D, row offsets of step s + 2D
    uint32_t p1 = (uint32_t)lane * 8u;
    uint32_t p2 = (uint32_t)rg * 4u;
    uint32_t p3 = ((uint32_t)i * nchunk + chunk) * (16u * NTR);
    constexpr uint32_t st1 = kWave * 8u, st2 = kWave * 4u;
    const uint32_t st3 = (uint32_t)K * nchunk * (16u * NTR);
    // the token of a sub-token, and whether it is a write part
    auto token_of = [&](int64_t u) { return T - 1 - (u >> 1); };
    // byte offset of this lane's saved write row X for the sub-token u (past
    // the range unless u is a write part and j < W)
    auto x_off = [&](int64_t u) {
        const bool on = u < U && (u & 1) && (uint32_t)j < W;
        return on ? (((uint32_t)token_of(u) * nchunk + chunk) * W + (uint32_t)j) * 16u : kOOB;
    };

    // register ring, slot = step % D
    uint2 lr[D];              // lane record of step s
    uint4 tr[D][NTR];         // token record (this wave's chunk) of step s
    f32x4 xr[D];              // saved write row of step s
    uint32_t go[D];           // row offset (memory layout) of step s + D
    uint32_t ofw[D];          // store offset (memory layout) of step s

    auto idx_load = [&](int sl) __attribute__((always_inline)) {
        go[sl] = __builtin_amdgcn_raw_buffer_load_b32(R2, p2, 0, 0);
        p2 += st2;
    };
    auto meta_load = [&](int sl, int64_t step) __attribute__((always_inline)) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(R1, p1, 0, 0);
        lr[sl] = make_uint2(x[0], x[1]);
#pragma unroll
        for (int q = 0; q < NTR; ++q) {
            const auto y = __builtin_amdgcn_raw_buffer_load_b128(R3, p3 + 16u * q, 0, 0);
            tr[sl][q] = make_uint4(y[0], y[1], y[2], y[3]);
        }
        xr[sl] = __builtin_amdgcn_raw_buffer_load_b128(Xrs, x_off(step * K + i), 0, 0);
        p1 += st1;
        p3 += st3;
    };
    // this wave's share of the gathers of a step (rows RPW*w .. RPW*w+RPW-1,
    // whole segments) into gath[sl] from the row offsets in go[sl]; bit 0 of
    // an offset marks an update superseded within the next D - 1 steps: its
    // store goes past the range and is dropped
    auto gathers = [&](int sl) __attribute__((always_inline)) {
        const uint32_t ofg = (go[sl] & ~1u) - kRowBias + segb + cg * 16u;
        ofw[sl] = (go[sl] & 1u) ? kOOB : ofg;
        asm volatile("" : "+v"(ofw[sl]));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            Mrs, (__attribute__((address_space(3))) void *)&gath[sl][wave * RPW][0], 16, ofg, 0, 0, 0);
    };

    for (uint32_t e = threadIdx.x; e < sizeof(gath) / 16; e += 64 * G)
        reinterpret_cast<f32x4 *>(&gath[0][0][0])[e] = (f32x4){0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    static_for<0, D>([&](auto s_c) __attribute__((always_inline)) { idx_load(decltype(s_c)::value); });
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    static_for<0, D>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        gathers(s);
        idx_load(s);
        meta_load(s, s);
    });
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");

    const int pos_own = (wave + lane) & (G - 1);
    for (int64_t s0 = 0; s0 < nsteps; s0 += D) {
        static_for<0, D>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            const int64_t step = s0 + s;
            const int rs = (int)((uint64_t)step % (2 * D));
            wait_vmcnt<(D - 1) * NVM>();
            // the step's records are used only from here on (otherwise the
            // compiler may hoist their first use above the previous step's
            // issue, with a wait tighter than the pipeline needs)
            asm volatile("" : "+v"(lr[s].x), "+v"(lr[s].y), "+v"(xr[s]));
            const uint32_t code = ~lr[s].x;   // stored inverted: a load past the range reads "none"
            const float wj = __uint_as_float(lr[s].y);
            const uint32_t cw = code & 0x7FFFu;
            const int dd = (int)(cw >> 6);
            const bool hw = cw != 0x7FFFu;
            const bool inw = hw && dd <= i;   // the source is an earlier sub-token of this step
            const int64_t u = step * K + i;
            auto ring_addr = [&](int d, uint32_t c) {
                const int64_t up = u - d;
                const int r = (((int)up & (K - 1)) << LQ) | (int)(c & (Q - 1));
                return lds_addr(&ring[(uint32_t)(up >> LK) % (uint32_t)(2 * D)][r][(wave + r) & (G - 1)]);
            };
            const uint32_t ga = lds_addr(&gath[s][lane][pos_own]);
            const uint32_t aw = hw && !inw ? ring_addr(dd, cw) : ga;
            const bool intra = __builtin_amdgcn_ballot_w64(inw) != 0;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            const f32x4 y = lds_read16(aw);
            const bool wpart = (u & 1) != 0;
            const f32x4 r0 = as_f32x4(tr[s][0]);
            const float at = r0.x, bt = BF16 ? r0.w : r0.y;     // write part
            f32x4 v4;
            if constexpr (BF16)
                v4 = v_chunk(make_uint2(tr[s][0].y, tr[s][0].z));
            else
                v4 = as_f32x4(tr[s][NTR - 1]);
            const f32x4 X = xr[s];
            // the new row of this lane for a given current value yy, and the
            // group's du (meaningful in write parts)
            auto update = [&](f32x4 yy, f32x4 &du) {
                du = mul4(bt, weighted_rows<Q>(wj, yy));
                const f32x4 dp = mul4(-at, du);
                const f32x4 nw = {__builtin_fmaf(at, yy.x, wj * dp.x), __builtin_fmaf(at, yy.y, wj * dp.y),
                                  __builtin_fmaf(at, yy.z, wj * dp.z), __builtin_fmaf(at, yy.w, wj * dp.w)};
                const f32x4 nr = {__builtin_fmaf(wj, r0.x, yy.x), __builtin_fmaf(wj, r0.y, yy.y),
                                  __builtin_fmaf(wj, r0.z, yy.z), __builtin_fmaf(wj, r0.w, yy.w)};
                return wpart ? nw : nr;
            };
            f32x4 du, yk = y;
            if (!intra) {
                ring[rs][lane][pos_own] = update(y, du);
            } else {
                // Rounds: a sub-token commits (writes its ring row) once every
                // earlier sub-token of the step it takes a row from has
                // committed; the first uncommitted one is always ready.
                uint32_t dep = inw ? (1u << (i - dd)) : 0u;
                dep = group_or<Q>(dep);
                const uint32_t aw2 = inw ? ring_addr(dd, cw) : ga;
                uint32_t done = 0;
                du = (f32x4){0.f, 0.f, 0.f, 0.f};
                while (true) {
                    const bool ready = ((dep | (1u << i)) & ~done) == (1u << i);
                    f32x4 yy = lds_read16(aw2);
                    if (!inw) yy = y;
                    f32x4 du2;
                    const f32x4 n2 = update(yy, du2);
                    if (ready) {
                        ring[rs][lane][pos_own] = n2;
                        yk = yy;
                        du = du2;
                    }
                    wave_lds_sync();
                    const uint64_t rb = __builtin_amdgcn_ballot_w64(ready);
#pragma unroll
                    for (int t = 0; t < K; ++t) done |= (uint32_t)((rb >> (t * Q)) & 1u) << t;
                    if (done == (1u << K) - 1u) break;
                }
            }
            // partial sums of this chunk (write parts): dw_j, da, db
            const f32x4 p = weighted_rows<Q>(wj, X);
            const f32x4 dp = mul4(-at, du);
            const f32x4 uu = {__builtin_fmaf(-at, p.x, v4.x), __builtin_fmaf(-at, p.y, v4.y),
                              __builtin_fmaf(-at, p.z, v4.z), __builtin_fmaf(-at, p.w, v4.w)};
            const float yu = dot4(yk, uu);
            const float dwp = __builtin_fmaf(bt, yu, dot4(dp, X));
            const float sa = group_sum1<Q>(dot4(yk, X)) - dot4(p, du);
            const float sb = group_sum1<Q>(wj * yu);
            if constexpr (RED) {
                red[wave][lane] = dwp;
                if (j == 0) {
                    red2[wave][i][0] = sa;
                    red2[wave][i][1] = sb;
                }
            }
            // ---- stores: whole segments of the updated rows (every wave's
            // chunks), this wave's chunk of dv, the segment's partial sums
            // (the parts of its G waves added here) ----
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_raw_buffer_store_b128(lds_read16(lds_addr(&ring[rs][rg][pg])), Mrs, ofw[s], 0, 0);
            {
                const bool live = u < U && wpart;
                const uint32_t t32 = (uint32_t)token_of(u < U ? u : U - 1);
                const uint32_t ov = live && j == 0 ? t32 * (uint32_t)H * d_v * 4u + colb : kOOB;
                __builtin_amdgcn_raw_buffer_store_b128(du, Vrs, ov, 0, 0);
                // (the b32 and b64 forms take integer data: pass the bits)
                if constexpr (!RED) {
                    const uint32_t rec = (t32 * nseg + chunk) * (uint32_t)PQ;
                    const uint32_t ow = live && (uint32_t)j < W ? (rec + (uint32_t)j) * 4u : kOOB;
                    const uint32_t oab = live && j == 0 ? (rec + (uint32_t)Q) * 4u : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dwp), Prs, ow, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b64(
                        (uint32_t __attribute__((ext_vector_type(2)))){__float_as_uint(sa), __float_as_uint(sb)}, Prs,
                        oab, 0, 0);
                } else {
                    // dw_j of row rsum: the G waves' parts, added by a butterfly
                    // over the G lanes that hold them
                    float sdw = red[lane % G][rsum];
                    sdw += __uint_as_float(lane_xor<1>(__float_as_uint(sdw)));
                    if constexpr (G >= 4) sdw += __uint_as_float(lane_xor<2>(__float_as_uint(sdw)));
                    if constexpr (G >= 8) sdw += __uint_as_float(lane_xor<4>(__float_as_uint(sdw)));
                    const int64_t us = step * K + (rsum >> LQ);
                    const uint32_t js = (uint32_t)(rsum & (Q - 1));
                    const bool lw = us < U && (us & 1) && js < W && lane % G == 0;
                    const uint32_t ts = (uint32_t)token_of(us < U ? us : U - 1);
                    const uint32_t ow = lw ? ((ts * nseg + seg) * (uint32_t)PQ + js) * 4u : kOOB;
                    // da, db of sub-token `lane` (wave 0, lanes < K): the waves' parts in order
                    float ta = 0.f, tb = 0.f;
                    const int il = lane < K ? lane : 0;
                    if (wave == 0) {
#pragma unroll
                        for (int w = 0; w < G; ++w) {
                            ta += red2[w][il][0];
                            tb += red2[w][il][1];
                        }
                    }
                    const int64_t ua = step * K + il;
                    const bool la = wave == 0 && lane < K && ua < U && (ua & 1);
                    const uint32_t ta32 = (uint32_t)token_of(ua < U ? ua : U - 1);
                    const uint32_t oab = la ? ((ta32 * nseg + seg) * (uint32_t)PQ + (uint32_t)Q) * 4u : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sdw), Prs, ow, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b64(
                        (uint32_t __attribute__((ext_vector_type(2)))){__float_as_uint(ta), __float_as_uint(tb)}, Prs, oab,
                        0, 0);
                }
            }
            // ---- issue step + D ----
            gathers(s);
            idx_load(s);
            meta_load(s, step + D);
            asm volatile("" ::: "memory");
        });
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
#endif  // __HIP_DEVICE_COMPILE__
}

// dw_j, da, db: the nseg partial-sum records of a token (per chunk or per
// row segment) added in order; dr_i = <do, Z_i> with the chunks' dot
// products added in chunk order.  One wave per token-head row (b, t, h).
// One wave per (b, t, h).  For dr_i = <do, Z_i>, P = 64 / Q lanes share read
// position i: lane (g, i) = (lane / Q, lane % Q) adds the chunks g, g + P,
// g + 2P, ... with several loads in flight (each chunk's Q lanes read
// consecutive 16-byte pieces), then the P lanes add their sums in a fixed
// butterfly.
template <int Q>
__global__ void __launch_bounds__(256) scan_bwd_reduce_kernel(BwdArgs A, const float *part, int nseg)
{
    constexpr int P = kWave / Q;
    const int64_t rows = A.B * A.T * A.H;
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / kWave;
    if (row >= rows) return;   // whole waves
    const int lane = lane_id();
    const int64_t TH = A.T * A.H;
    const int64_t bb = row / TH, rem = row - bb * TH;
    const int64_t t = rem / A.H, h = rem - t * A.H;
    const int64_t ch = bb * A.H + h;
    const int nchunk = A.d_v / 4, PQ = Q + 2;
    const float *pp = part + (ch * A.T + t) * (int64_t)nseg * PQ;
    for (int e = lane; e < PQ; e += kWave) {
        if (e < A.W || e == Q || e == Q + 1) {
            float s = 0.f;
            for (int c = 0; c < nseg; ++c) s += pp[c * PQ + e];
            if (e < A.W) A.dw[row * A.W + e] = s;
            else if (e == Q) A.da[row] = s;
            else A.db[row] = s;
        }
    }
    const int i = lane % Q, g = lane / Q;
    float s = 0.f;
    if (i < A.R) {
        const float *Z = A.zsave + ((ch * A.T + t) * (int64_t)nchunk * A.R + i) * 4;
        const float *dop = A.dout + row * A.d_v;
#pragma unroll 8
        for (int c = g; c < nchunk; c += P) {
            const f32x4 z = *reinterpret_cast<const f32x4 *>(Z + (int64_t)c * A.R * 4);
            const f32x4 dv = *reinterpret_cast<const f32x4 *>(dop + 4 * c);
            s += dot4(dv, z);
        }
    }
    if constexpr (P >= 2) s += __uint_as_float(lane_xor<Q>(__float_as_uint(s)));
    if constexpr (P >= 4) s += __uint_as_float(lane_xor<2 * Q>(__float_as_uint(s)));
    if constexpr (P >= 8) s += __uint_as_float(lane_xor<4 * Q>(__float_as_uint(s)));
    if constexpr (P >= 16) s += __uint_as_float(lane_xor<8 * Q>(__float_as_uint(s)));
    if (g == 0 && i < A.R) A.dr[row * A.R + i] = s;
}

namespace {

int bwd_lanes_q(int W, int R)
{
    int q = 4;
    while (q < W || q < R) q *= 2;
    return q;
}

struct BwdWsLayout {
    size_t lane, gofs, tok, part, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdShape {
    int G, D;
};

// as the forward's: the widest segment that still gives every CU a workgroup
BwdShape bwd_lanes_shape(int64_t chunks)
{
    constexpr int64_t kCUs = 256;
    if (chunks / 8 >= 2 * kCUs) return {8, 2};
    if (chunks / 8 >= kCUs) return {8, 4};
    if (chunks / 4 >= kCUs) return {4, 4};
    return {2, 4};
}

BwdWsLayout bwd_ws_layout(int64_t B, int64_t T, int64_t H, int W, int R, int d_v, bool bf16)
{
    const size_t chains = (size_t)(B * H), U = 2 * (size_t)T;
    const size_t q = (size_t)bwd_lanes_q(W, R), nchunk = (size_t)d_v / 4;
    const int G = bwd_lanes_shape(B * H * (d_v / 4)).G;
    const size_t nseg = G == 8 ? nchunk / 8 : nchunk;   // the kernel's partial-sum records per token
    BwdWsLayout L;
    L.lane = 0;
    L.gofs = L.lane + align256(chains * U * q * 8);
    L.tok = L.gofs + align256(chains * U * q * 4);
    L.part = L.tok + align256(chains * U * nchunk * (bf16 ? 16 : 32));
    L.total = L.part + align256(chains * (size_t)T * nseg * (q + 2) * 4);
    return L;
}

// every per-chain range the lanes kernel addresses with 32-bit offsets
bool bwd_lanes_fits(int64_t T, int64_t H, int W, int R, int d_v, bool bf16)
{
    const uint64_t lim = 1ull << 31, U = 2 * (uint64_t)T;
    const uint64_t q = (uint64_t)bwd_lanes_q(W, R), nchunk = (uint64_t)d_v / 4;
    return U * q * 8 < lim && U * nchunk * (bf16 ? 16 : 32) < lim && (uint64_t)T * W * d_v * 4 < lim &&
           (uint64_t)T * H * d_v * 4 < lim && (uint64_t)T * nchunk * (q + 2) * 4 < lim;
}

int bwd_hash_log2(int q, int window, int lookahead)
{
    const int entries = (kBpBlock + window + lookahead) * q;
    int lg = 6;
    while ((1 << lg) < 2 * entries) ++lg;
    return lg;
}

template <int Q, int D, int G>
hipError_t launch_bwd_lanes(const BwdArgs &A, bool bf16, const BwdStreams &S, hipStream_t st)
{
    const int64_t groups = A.B * A.H * (A.d_v / 4) / G;
    if (bf16)
        hipLaunchKernelGGL((sdm_scan_bwd_lanes_kernel<Q, D, G, true>), dim3((unsigned)groups), dim3(64 * G), 0, st, A, S);
    else
        hipLaunchKernelGGL((sdm_scan_bwd_lanes_kernel<Q, D, G, false>), dim3((unsigned)groups), dim3(64 * G), 0, st, A,
                           S);
    return hipGetLastError();
}

template <int Q>
hipError_t launch_bwd_lanes_q(const BwdArgs &A, bool bf16, const BwdStreams &S, int G, int D, hipStream_t st)
{
    if (G == 8 && D == 2) return launch_bwd_lanes<Q, 2, 8>(A, bf16, S, st);
    if (G == 8 && D == 4) return launch_bwd_lanes<Q, 4, 8>(A, bf16, S, st);
    if (G == 4 && D == 4) return launch_bwd_lanes<Q, 4, 4>(A, bf16, S, st);
    if (G == 2 && D == 4) return launch_bwd_lanes<Q, 4, 2>(A, bf16, S, st);
    return hipErrorInvalidValue;
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int d_v, bool bf16)
{
    if (B * T == 0 || !bwd_lanes_fits(T, H, W, R, d_v, bf16)) return 0;
    return bwd_ws_layout(B, T, H, W, R, d_v, bf16).total;
}

hipError_t launch_scan_backward_lanes(const BwdArgs &A, bool bf16, void *ws, hipStream_t stream)
{
    if (A.B * A.H == 0 || A.T == 0) return hipSuccess;
    const int Q = bwd_lanes_q(A.W, A.R);
    const int K = 64 / Q;
    const BwdShape sh = bwd_lanes_shape(A.B * A.H * (A.d_v / 4));
    const int D = sh.D;
    const int window = 2 * D * K - 1, lookahead = D * K - 1;
    const BwdWsLayout L = bwd_ws_layout(A.B, A.T, A.H, A.W, A.R, A.d_v, bf16);
    unsigned char *base = static_cast<unsigned char *>(ws);
    BwdStreams S{reinterpret_cast<uint2 *>(base + L.lane), reinterpret_cast<uint32_t *>(base + L.gofs),
                 reinterpret_cast<uint4 *>(base + L.tok), reinterpret_cast<float *>(base + L.part)};
    BwdPrepArgs P{A.widx, A.ridx, A.wwt, A.rwt, A.a, A.b, A.dout, A.v, S, A.B, A.T, A.H,
                  A.W, A.R, Q, K, window, lookahead, bwd_hash_log2(Q, window, lookahead), A.d_v, bf16 ? 1 : 0};
    if (P.hash_log2 > 14) return hipErrorInvalidValue;
    const int64_t nblk = (2 * A.T + kBpBlock - 1) / kBpBlock;
    // bucket heads, then the entries {slot, next entry of the bucket}
    const size_t smem = sizeof(uint32_t) * ((size_t)1 << P.hash_log2) +
                        sizeof(uint2) * (size_t)(kBpBlock + window + lookahead) * (size_t)Q;
    if (smem > 160 * 1024) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void *)scan_bwd_prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_bwd_prep_kernel, dim3((unsigned)(A.B * A.H * nblk)), dim3(kBpThreads), smem, stream, P);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (Q) {
    case 4: e = launch_bwd_lanes_q<4>(A, bf16, S, sh.G, D, stream); break;
    case 8: e = launch_bwd_lanes_q<8>(A, bf16, S, sh.G, D, stream); break;
    case 16: e = launch_bwd_lanes_q<16>(A, bf16, S, sh.G, D, stream); break;
    case 32: e = launch_bwd_lanes_q<32>(A, bf16, S, sh.G, D, stream); break;
    case 64: e = launch_bwd_lanes_q<64>(A, bf16, S, sh.G, D, stream); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t rows = A.B * A.T * A.H;
    const int nseg = sh.G == 8 ? A.d_v / 32 : A.d_v / 4;
    const dim3 grid((unsigned)((rows + 3) / 4));
    switch (Q) {
    case 4: hipLaunchKernelGGL(scan_bwd_reduce_kernel<4>, grid, dim3(256), 0, stream, A, S.part, nseg); break;
    case 8: hipLaunchKernelGGL(scan_bwd_reduce_kernel<8>, grid, dim3(256), 0, stream, A, S.part, nseg); break;
    case 16: hipLaunchKernelGGL(scan_bwd_reduce_kernel<16>, grid, dim3(256), 0, stream, A, S.part, nseg); break;
    case 32: hipLaunchKernelGGL(scan_bwd_reduce_kernel<32>, grid, dim3(256), 0, stream, A, S.part, nseg); break;
    default: hipLaunchKernelGGL(scan_bwd_reduce_kernel<64>, grid, dim3(256), 0, stream, A, S.part, nseg); break;
    }
    return hipGetLastError();
}

}  // namespace sdm
