// sdm_scan_lanes.hip -- lane-parallel prefill scan.
//
// The recurrence is the sparse gated delta rule of "Sparse Delta Memory:
// Scaling the State of Linear RNNs through Sparsity", Sec. 3.1 steps 2-3
// (Eq. 4): per token, p = sum_j w_j M[s_j] over the W write rows, then
// M[s_j] = a M[s_j] + b w_j (v - a p) for all j at once, then
// o = sum_j r_j M[s'_j] over the R read rows after the write.
//
// Work unit: one wave per (sequence, head, 4-column chunk) -- columns never
// interact, so every 16-byte column chunk of the memory is an independent
// recurrence over the same slot lists.  The G waves (G = 2, 4 or 8) of the
// chunks that make up one G*16-byte row segment form a workgroup.  Memory is
// accessed cooperatively in whole segments: each wave gathers and stores
// whole segments of 64/G of the step's rows (G consecutive lanes per row, so
// a row segment is one coalesced access) through LDS, and computes on its
// own chunk of every row; two barriers per step separate the phases.  When G
// < 8, the 8/G workgroups that share 128-byte lines run on the same XCD,
// whose L2 then serves each line once (the host picks the widest G that
// still gives a workgroup to every CU).  Within the wave, lane (i, j) =
// (lane / Q, lane % Q) holds column chunk `chunk` of write row j and of read
// row j of token i of the current step, Q = the power of two >= max(W, R):
// a step advances K = 64 / Q consecutive tokens at once.  The sums over rows
// are all-reductions over aligned groups of Q lanes (DPP quad_perm and
// row_half_mirror / row_mirror adds, then the gfx950 permlane16/32 swaps).
//
// Tokens of one step run concurrently unless one of them needs a row that
// an earlier token of the same step writes (forwarding code with 1 <= delta
// <= its position in the step); such a step runs in rounds, a token
// committing once the tokens it takes rows from have (exact, rare for
// scattered addressing, usually two rounds).  Two tokens of a step never
// store the same row: a write superseded later in the step is dropped.
// Every row a lane needs comes from one LDS read placed before the step's
// compute: the gathered row, or the ring row of its latest writer.
//
// Latency: the gathers of step s + D are issued at the end of step s with the
// LDS-destination form of buffer_load (one 1 KB instruction per row kind),
// and the per-token metadata of step s + D (the slot lists of step s + 2D)
// is loaded into a register ring at the same time.  Every step issues the
// same fixed list of vector-memory instructions (lanes with nothing to do
// use an offset past the buffer range: loads return zero, stores are
// dropped), so the wait for a step's data is an exact compile-time vmcnt.
// A gather issued D steps early misses the writes of the tokens in between;
// those rows are taken from an LDS ring of recently written rows, following
// exact forwarding codes computed beforehand (scan_prep.hip).  A row stored
// by one wave is gathered by another only after the storing wave waited for
// the store and both passed a barrier: a store of step s is complete before
// its wave passes the first barrier of step s + D, and the gathers issued at
// the end of step s' see it from s' >= s + D on, so the codes cover the
// rows written by the last 2D steps, which the ring holds.  A write that is
// written again within the next D - 1 steps is not stored at all (the later
// one is), so stores of one row are at least D steps apart and land in order.
#include "kernels.h"
#include "lanes_common.h"
#include "scan_lanes.h"

namespace sdm {

using namespace lanes;

template <int Q, int D, int G, bool BF16, bool SAVE>
__global__ void __launch_bounds__(64 * G) sdm_scan_lanes_kernel(ScanArgs A, ScanStreams S)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int K = kWave / Q;
    constexpr int LQ = ilog2(Q), LK = ilog2(K);
    static_assert((1 << LQ) == Q, "Q is a power of two");
    constexpr int NTR = BF16 ? 1 : 2;            // 16-byte token records per chunk
    constexpr int NVM = 6 + NTR + (SAVE ? 2 : 0);   // vector-memory instructions per step (fixed)
    static_assert((D - 1) * NVM <= 63, "pipeline deeper than the vmcnt range");

    static_assert(G == 2 || G == 4 || G == 8, "2, 4 or 8 waves per workgroup");
    constexpr int RPW = kWave / G;               // rows of a step each wave moves

    // Row r of a step is token r / Q, list position r % Q (r = the lane of
    // the compute layout).  Row segments are G chunks of 16 bytes; chunk c of
    // row r sits at position (c + r) % G (so that the compute waves, which
    // read one chunk of 64 consecutive rows, spread over the LDS banks).
    __shared__ f32x4 gath[D][2][kWave][G];      // gathered write / read rows of the steps in flight
    __shared__ f32x4 ring[2 * D][kWave][G];     // rows written by the last 2D steps

    const uint32_t d_v = (uint32_t)A.d_v;
    const uint32_t nline = d_v / 32u;            // 128-byte lines per row
    uint32_t grp, part;
    xcd_decode(blockIdx.x, (uint32_t)(A.B * A.H) * nline, 8u / G, grp, part);
    const uint32_t chu = __builtin_amdgcn_readfirstlane(grp / nline);
    const uint32_t seg = __builtin_amdgcn_readfirstlane((grp - chu * nline) * (8u / G) + part);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));   // compute chunk
    const int64_t ch = chu;
    const int64_t H = A.H, T = A.T;
    const int64_t bb = ch / H, h = ch - bb * H;
    const int lane = lane_id();
    const int i = lane >> LQ;                                // compute layout: token of the step
    const int rg = wave * RPW + lane / G;                   // memory layout: row ...
    const int pg = lane % G;                                //   ... and its position
    const uint32_t cg = (uint32_t)((pg - rg) & (G - 1));    //   = chunk cg of that row
    const uint32_t nchunk = d_v / 4u;
    const uint32_t chunk = seg * G + (uint32_t)wave;
    const uint32_t segb = seg * G * 16u;                    // byte offset of the segment in a row
    const uint32_t colb = segb + (uint32_t)wave * 16u;      // byte offset of this wave's chunk
    const __amdgpu_buffer_rsrc_t Mrs =
        make_rsrc(A.M + (size_t)ch * A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
    // this chain's streams (sizes checked on the host to be < 2 GiB)
    const uint64_t tq = (uint64_t)T * Q;
    const __amdgpu_buffer_rsrc_t R1 = make_rsrc(S.lane + ch * tq, (uint32_t)(tq * 16u));
    const __amdgpu_buffer_rsrc_t R2 = make_rsrc(S.gofs + ch * tq, (uint32_t)(tq * 8u));
    const uint64_t tc = (uint64_t)T * nchunk * NTR;
    const __amdgpu_buffer_rsrc_t R3 = make_rsrc(S.tok + ch * tc, (uint32_t)(tc * 16u));
    const int64_t nsteps = (T + K - 1) / K;

    // running byte offsets of the next loads: lane records and token records
    // of step s + D, row offsets of step s + 2D
    uint32_t p1 = (uint32_t)lane * 16u;
    uint32_t p2 = (uint32_t)rg * 8u;
    uint32_t p3 = ((uint32_t)i * nchunk + chunk) * (16u * NTR);
    constexpr uint32_t st1 = kWave * 16u, st2 = kWave * 8u;
    const uint32_t st3 = (uint32_t)K * nchunk * (16u * NTR);
    // output window of a step: K tokens from its first
    const uint32_t otok = (uint32_t)(H * d_v * 4u);
    const uint32_t offO = (lane & (Q - 1)) == 0 ? (uint32_t)i * otok + colb : kOOB;
    float *obase = A.o + (size_t)(bb * T * H + h) * d_v;
    const uint32_t orec = (uint32_t)(K - 1) * otok + d_v * 4u;
    // saved rows of this chain: [T][d_v/4][W or R][4] (sizes checked on the host)
    const __amdgpu_buffer_rsrc_t Xrs =
        SAVE ? make_rsrc(A.xsave + (size_t)ch * T * A.W * d_v, (uint32_t)((uint64_t)T * A.W * d_v * 4u))
             : make_rsrc(A.o, 0u);
    const __amdgpu_buffer_rsrc_t Zrs =
        SAVE ? make_rsrc(A.zsave + (size_t)ch * T * A.R * d_v, (uint32_t)((uint64_t)T * A.R * d_v * 4u))
             : make_rsrc(A.o, 0u);

    // register ring, slot = step % D
    uint4 lr[D];              // lane record of step s
    uint4 tr[D][NTR];         // token record (this wave's chunk) of step s
    uint2 go[D];              // row offsets (memory layout) of step s + D
    uint32_t ofw[D];          // store offsets of the write rows (memory layout) of step s

    auto idx_load = [&](int sl) __attribute__((always_inline)) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(R2, p2, 0, 0);
        go[sl] = make_uint2(x[0], x[1]);
        p2 += st2;
    };
    auto meta_load = [&](int sl) __attribute__((always_inline)) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(R1, p1, 0, 0);
        lr[sl] = make_uint4(x[0], x[1], x[2], x[3]);
#pragma unroll
        for (int q = 0; q < NTR; ++q) {
            const auto y = __builtin_amdgcn_raw_buffer_load_b128(R3, p3 + 16u * q, 0, 0);
            tr[sl][q] = make_uint4(y[0], y[1], y[2], y[3]);
        }
        p1 += st1;
        p3 += st3;
    };
    // this wave's share of the gathers of a step (rows RPW*w .. RPW*w+RPW-1 of
    // the write and of the read rows, whole segments) into gath[sl], from the
    // row offsets in go[sl]; a zero offset record lands at or beyond 2^31
    // (bit 0 of a write-row offset marks a write superseded within the next
    // D - 1 steps: its store goes to kOOB, past the range, and is dropped)
    auto gathers = [&](int sl) __attribute__((always_inline)) {
        const uint32_t ofg = (go[sl].x & ~1u) - kRowBias + segb + cg * 16u;
        ofw[sl] = (go[sl].x & 1u) ? kOOB : ofg;
        // formed here, so that the row offset register is free for the next
        // load into the same ring slot (a copy at the loop edge would wait
        // for that load)
        asm volatile("" : "+v"(ofw[sl]));
        const uint32_t ofr = go[sl].y - kRowBias + segb + cg * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            Mrs, (__attribute__((address_space(3))) void *)&gath[sl][0][wave * RPW][0], 16, ofg, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            Mrs, (__attribute__((address_space(3))) void *)&gath[sl][1][wave * RPW][0], 16, ofr, 0, 0, 0);
    };

    // Rows past W or R are gathered from past the buffer range; make every
    // LDS byte they could leave untouched a finite zero once.
    for (uint32_t e = threadIdx.x; e < sizeof(gath) / 16; e += 64 * G)
        reinterpret_cast<f32x4 *>(&gath[0][0][0][0])[e] = (f32x4){0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    // ---- prologue: row offsets of steps 0..D-1, then the steady-state issue
    // order (gathers of s, row offsets of s + D, records of s) for s < D.
    static_for<0, D>([&](auto s_c) __attribute__((always_inline)) { idx_load(decltype(s_c)::value); });
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    static_for<0, D>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        gathers(s);
        idx_load(s);
        meta_load(s);
    });
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the loop starts with nothing pending
    asm volatile("" ::: "memory");

    const int pos_own = (wave + lane) & (G - 1);   // position of this wave's chunk in row `lane`
    for (int64_t s0 = 0; s0 < nsteps; s0 += D) {
        static_for<0, D>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            const int64_t step = s0 + s;
            const int rs = (int)((uint64_t)step % (2 * D));   // ring slot of this step
            // ---- this step's gathers (every wave's share) and records ----
            wait_vmcnt<(D - 1) * NVM>();
            const uint32_t code = ~lr[s].x;   // stored inverted: a load past the range reads "none"
            const float wj = __uint_as_float(lr[s].y), rj = __uint_as_float(lr[s].z);
            const uint32_t cw = code & 0x7FFFu, cr = code >> 16;
            const int dw = (int)(cw >> 6), dr = (int)(cr >> 6);
            const bool hw = cw != 0x7FFFu, hr = cr != 0xFFFFu;
            // sources inside this step: the writer is an earlier token of it
            const bool inw = hw && dw <= i, inr = hr && dr >= 1 && dr <= i;
            const int64_t u = step * K + i;   // this lane's token
            // LDS address of this wave's chunk of the row written by token
            // u - d at list position c (ring slot of that token's step)
            auto ring_addr = [&](int d, uint32_t c) {
                const int64_t up = u - d;
                const int r = (((int)up & (K - 1)) << LQ) | (int)(c & (Q - 1));
                return lds_addr(&ring[(uint32_t)(up >> LK) % (uint32_t)(2 * D)][r][(wave + r) & (G - 1)]);
            };
            // where this lane's write and read rows come from: the gathered
            // row, or the ring row of the latest earlier writer in the window
            const uint32_t gaw = lds_addr(&gath[s][0][lane][pos_own]), gar = lds_addr(&gath[s][1][lane][pos_own]);
            const uint32_t aw = hw && !inw ? ring_addr(dw, cw) : gaw;
            const uint32_t ar = hr && dr > i ? ring_addr(dr, cr) : gar;
            const bool intra = __builtin_amdgcn_ballot_w64(inw || inr) != 0;
            const bool d0 = __builtin_amdgcn_ballot_w64(hr && dr == 0) != 0;
            // this wave's LDS writes of the previous step complete before the
            // barrier (a workgroup-scope publish of LDS needs lgkmcnt(0))
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            f32x4 xw, xr;
            lds_read2(xw, xr, aw, ar);
            const float at = __uint_as_float(tr[s][0].x);
            const float bwj = __uint_as_float(BF16 ? tr[s][0].w : tr[s][0].y) * wj;   // b_t * w_j
            f32x4 v4;
            if constexpr (BF16)
                v4 = v_chunk(make_uint2(tr[s][0].y, tr[s][0].z));
            else
                v4 = (f32x4){__uint_as_float(tr[s][NTR - 1].x), __uint_as_float(tr[s][NTR - 1].y),
                             __uint_as_float(tr[s][NTR - 1].z), __uint_as_float(tr[s][NTR - 1].w)};
            auto own_row = [&](uint32_t c) {   // this token's write at position c
                const int r = (i << LQ) | (int)(c & (Q - 1));
                return lds_read16(lds_addr(&ring[rs][r][(wave + r) & (G - 1)]));
            };
            f32x4 o;
            f32x4 sw = xw, sr = xr;   // the write row before, the read row after (saved)
            if (!intra) {
                const f32x4 p = weighted_rows<Q>(wj, xw);
                o = weighted_rows<Q>(rj, xr);
                ring[rs][lane][pos_own] = written_row(xw, at, bwj, v4, p);
                if (d0) {
                    wave_lds_sync();
                    const f32x4 own = own_row(cr);
                    if (hr && dr == 0) xr = own;
                    o = weighted_rows<Q>(rj, xr);
                }
                sr = xr;
            } else {
                // Rounds: a token commits (writes its rows, takes its output)
                // once every earlier token of the step it takes a row from has
                // committed; the first uncommitted token is always ready, so
                // at most K rounds, usually two.  Rows from earlier steps keep
                // the values read above (the ring slot of step s - 2D is this
                // step's, and committing tokens overwrite it).
                uint32_t dep = 0;   // tokens of the step this token waits for (bit per token)
                if (inw) dep |= 1u << (i - dw);
                if (inr) dep |= 1u << (i - dr);
                dep = group_or<Q>(dep);
                const uint32_t aw2 = inw ? ring_addr(dw, cw) : gaw, ar2 = inr ? ring_addr(dr, cr) : gar;
                uint32_t done = 0;
                f32x4 ok = xr;
                while (true) {
                    const bool ready = ((dep | (1u << i)) & ~done) == (1u << i);
                    f32x4 yw, yr;
                    lds_read2(yw, yr, aw2, ar2);
                    if (!inw) yw = xw;
                    if (!inr) yr = xr;
                    const f32x4 p = weighted_rows<Q>(wj, yw);
                    const f32x4 n2 = written_row(yw, at, bwj, v4, p);
                    if (ready) ring[rs][lane][pos_own] = n2;
                    wave_lds_sync();
                    const f32x4 own = own_row(cr);
                    if (hr && dr == 0) yr = own;
                    const f32x4 o2 = weighted_rows<Q>(rj, yr);
                    if (ready) {
                        ok = o2;
                        sw = yw;
                        sr = yr;
                    }
                    const uint64_t rb = __builtin_amdgcn_ballot_w64(ready);
#pragma unroll
                    for (int t = 0; t < K; ++t) done |= (uint32_t)((rb >> (t * Q)) & 1u) << t;
                    if (done == (1u << K) - 1u) break;
                }
                o = ok;
            }
            // ---- stores: whole segments of the written rows (every wave's
            // chunks), and this wave's chunk of the outputs; the ring rows
            // written above are complete before the barrier ----
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_raw_buffer_store_b128(lds_read16(lds_addr(&ring[rs][rg][pg])), Mrs, ofw[s], 0, 0);
            {
                const int64_t rem = T - step * K;   // live tokens of this step: i < rem
                const __amdgpu_buffer_rsrc_t Ors = make_rsrc(obase, orec);
                __builtin_amdgcn_raw_buffer_store_b128(o, Ors, i < rem ? offO : kOOB, 0, 0);
                obase += (size_t)K * H * d_v;
                if constexpr (SAVE) {
                    const int j = lane & (Q - 1);
                    const uint32_t ut = (uint32_t)u;
                    // [T][d_v/4][W or R][4]: the Q lanes of a token write consecutive 16-byte pieces
                    const uint32_t tck = ut * nchunk + chunk;
                    const uint32_t offx = (i < rem && j < A.W) ? (tck * (uint32_t)A.W + j) * 16u : kOOB;
                    const uint32_t offz = (i < rem && j < A.R) ? (tck * (uint32_t)A.R + j) * 16u : kOOB;
                    // read once, by the backward, much later: non-temporal (cache policy nt)
                    __builtin_amdgcn_raw_buffer_store_b128(sw, Xrs, offx, 0, 2);
                    __builtin_amdgcn_raw_buffer_store_b128(sr, Zrs, offz, 0, 2);
                }
            }
            // ---- issue step + D (its gathers overwrite gath[s], read by
            // every wave before the barrier above) ----
            gathers(s);
            idx_load(s);
            meta_load(s);
            asm volatile("" ::: "memory");
        });
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
#endif  // __HIP_DEVICE_COMPILE__
}

template <int Q, int D, int G, bool BF16>
static hipError_t launch_lanes(const ScanArgs &A, const ScanStreams &S, hipStream_t st)
{
    const int64_t groups = A.B * A.H * (A.d_v / 4) / G;
    if (A.xsave)
        hipLaunchKernelGGL((sdm_scan_lanes_kernel<Q, D, G, BF16, true>), dim3((unsigned)groups), dim3(64 * G), 0, st,
                           A, S);
    else
        hipLaunchKernelGGL((sdm_scan_lanes_kernel<Q, D, G, BF16, false>), dim3((unsigned)groups), dim3(64 * G), 0,
                           st, A, S);
    return hipGetLastError();
}

template <int Q>
static hipError_t launch_lanes_q(const ScanArgs &A, bool bf16, const ScanStreams &S, int G, int D, hipStream_t st)
{
#define SDM_LANES_GD(GV, DV)                                                                      \
    if (G == GV && D == DV)                                                                        \
        return bf16 ? launch_lanes<Q, DV, GV, true>(A, S, st) : launch_lanes<Q, DV, GV, false>(A, S, st);
    SDM_LANES_GD(8, 2)
    SDM_LANES_GD(8, 4)
    SDM_LANES_GD(4, 4)
    SDM_LANES_GD(2, 4)
#undef SDM_LANES_GD
    return hipErrorInvalidValue;
}

hipError_t launch_scan_lanes(const ScanArgs &A, bool bf16, const ScanStreams &S, int Q, int G, int D,
                             hipStream_t st)
{
    if (A.B * A.H * (A.d_v / 4) == 0 || A.T == 0) return hipSuccess;
    switch (Q) {
    case 4: return launch_lanes_q<4>(A, bf16, S, G, D, st);
    case 8: return launch_lanes_q<8>(A, bf16, S, G, D, st);
    case 16: return launch_lanes_q<16>(A, bf16, S, G, D, st);
    case 32: return launch_lanes_q<32>(A, bf16, S, G, D, st);
    case 64: return launch_lanes_q<64>(A, bf16, S, G, D, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sdm
