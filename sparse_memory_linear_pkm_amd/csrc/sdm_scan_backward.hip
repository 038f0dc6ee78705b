// sdm_scan_backward.hip -- reverse-mode gradients of the prefill scan.
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 steps 2-3 (Eq. 4), differentiated with the chain rule (the pages
// print no backward pass).  For token t of a (b, h) chain, in reverse, with
// G = dL/dM after the token (initially dL/dM_T, the caller's dM):
//     dr_i = <do, Z_i>;  G[r_i] += r_i do
//     dY_j = G[s_j];  p = sum_j w_j X_j;  u = v - a p
//     du = b sum_j w_j dY_j;  dv = du;  dp = -a du
//     da = sum_j <dY_j, X_j> - <p, du>;  db = sum_j w_j <dY_j, u>
//     dw_j = b <dY_j, u> + <dp, X_j>;  G[s_j] = a dY_j + w_j dp
// where X_j (the write rows before the write) and Z_i (the read rows after
// it) were saved by the forward scan.  On exit G = dL/dM before the call.
//
// Columns never interact here either: each 4-column chunk of a chain is an
// independent reverse recurrence on its chunk of G, so one lane owns one
// chunk for the whole sequence and its read-modify-writes of G are ordered
// by program order alone (no other lane touches those bytes).  A chain's
// chunks sit in an aligned group of QC lanes (the power of two >= d_v / 4),
// which sums the per-chunk parts of the scalar gradients (dr_i, dw_j, da,
// db) with a butterfly in a fixed order.
#include "device_common.h"
#include "kernels.h"
#include "scan_lanes.h"

#include <type_traits>

namespace sdm {

namespace {

template <int QC>
__device__ __forceinline__ float group_sum_qc(float x)
{
    if constexpr (QC >= 2) x += __uint_as_float(lane_xor<1>(__float_as_uint(x)));
    if constexpr (QC >= 4) x += __uint_as_float(lane_xor<2>(__float_as_uint(x)));
    if constexpr (QC >= 8) x += __uint_as_float(lane_xor<4>(__float_as_uint(x)));
    if constexpr (QC >= 16) x += __uint_as_float(lane_xor<8>(__float_as_uint(x)));
    if constexpr (QC >= 32) x += __uint_as_float(lane_xor<16>(__float_as_uint(x)));
    if constexpr (QC >= 64) x += __uint_as_float(lane_xor<32>(__float_as_uint(x)));
    return x;
}

__device__ __forceinline__ float dot4(f32x4 x, f32x4 y)
{
    return __builtin_fmaf(x.w, y.w, __builtin_fmaf(x.z, y.z, __builtin_fmaf(x.y, y.y, x.x * y.x)));
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

template <bool BF16>
__device__ __forceinline__ f32x4 ld_v4(const void *p, int64_t e)
{
    if constexpr (BF16) {
        const uint2 r = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + e);
        return (f32x4){__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
    } else {
        return ld4(static_cast<const float *>(p) + e);
    }
}

}  // namespace

template <int QC, bool BF16>
__global__ void __launch_bounds__(256) sdm_scan_backward_kernel(BwdArgs A)
{
    constexpr int kChainsPerBlock = 256 / QC;
    const int64_t chains = A.B * A.H;
    const int64_t chain0 = (int64_t)blockIdx.x * kChainsPerBlock + threadIdx.x / QC;
    const int c0 = (int)(threadIdx.x % QC);
    const int nchunk = A.d_v / 4;
    const bool live = chain0 < chains && c0 < nchunk;
    // dead lanes read a valid chunk, use zeros, and store nothing
    const int64_t chain = chain0 < chains ? chain0 : chains - 1;
    const int c = c0 < nchunk ? c0 : nchunk - 1;
    const int64_t bb = chain / A.H, h = chain - bb * A.H;
    const int64_t T = A.T, d_v = A.d_v, W = A.W, R = A.R;
    const int64_t col = (int64_t)c * 4;
    // G through a buffer resource: a slot outside [0, N) is dropped by the
    // hardware bounds check (loads read zeros) instead of faulting
    const __amdgpu_buffer_rsrc_t Grs = make_rsrc(A.dM + chain * (int64_t)A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
    constexpr uint32_t kOOB = 0x80000000u;   // past every range (all < 2 GiB)
    const uint32_t rowb = (uint32_t)d_v * 4u, colb = (uint32_t)col * 4u;
    auto goff = [&](int32_t slot) { return (slot >= 0 && slot < A.N) ? (uint32_t)slot * rowb + colb : kOOB; };
    auto gld = [&](uint32_t off) -> f32x4 { return __builtin_amdgcn_raw_buffer_load_b128(Grs, off, 0, 0); };
    // a lane's loads of G after its stores to the same bytes see them (one
    // lane, program order); the empty asm keeps the compiler from moving
    // later G loads above a store
    auto gst = [&](f32x4 x, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b128(x, Grs, live ? off : kOOB, 0, 0);
        asm volatile("" ::: "memory");
    };
    // saved rows [T][d_v/4][W or R][4] of this chain
    const int64_t nch = d_v / 4;
    const float *X = A.xsave + chain * T * W * d_v;
    const float *Z = A.zsave + chain * T * R * d_v;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bool lead = c0 == 0 && chain0 < chains;   // the lane that stores a chain's scalars

    for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t row = (bb * T + t) * A.H + h;
        const f32x4 dov = live ? ld4(A.dout + row * d_v + col) : zero;
        const f32x4 v4 = live ? ld_v4<BF16>(A.v, row * d_v + col) : zero;
        const float at = A.a[row], bt = A.b[row];
        // the read rows: their outputs' gradients, then into G
        for (int64_t i = 0; i < R; ++i) {
            const int32_t ri = A.ridx[row * R + i];
            const float rw = A.rwt[row * R + i];
            const f32x4 z = live ? ld4(Z + ((t * nch + c) * R + i) * 4) : zero;
            const uint32_t off = goff(ri);
            const f32x4 gv = gld(off);
            gst((f32x4){__builtin_fmaf(rw, dov.x, gv.x), __builtin_fmaf(rw, dov.y, gv.y),
                        __builtin_fmaf(rw, dov.z, gv.z), __builtin_fmaf(rw, dov.w, gv.w)},
                off);
            const float drs = group_sum_qc<QC>(dot4(dov, z));
            if (lead) A.dr[row * R + i] = drs;
        }
        // the write rows, first pass: the prediction and du
        f32x4 p = zero, du = zero;
        for (int64_t j = 0; j < W; ++j) {
            const int32_t wi = A.widx[row * W + j];
            const float ww = A.wwt[row * W + j];
            const f32x4 x = live ? ld4(X + ((t * nch + c) * W + j) * 4) : zero;
            const f32x4 dy = live ? gld(goff(wi)) : zero;
            p = (f32x4){__builtin_fmaf(ww, x.x, p.x), __builtin_fmaf(ww, x.y, p.y), __builtin_fmaf(ww, x.z, p.z),
                        __builtin_fmaf(ww, x.w, p.w)};
            du = (f32x4){__builtin_fmaf(ww, dy.x, du.x), __builtin_fmaf(ww, dy.y, du.y),
                         __builtin_fmaf(ww, dy.z, du.z), __builtin_fmaf(ww, dy.w, du.w)};
        }
        du = (f32x4){bt * du.x, bt * du.y, bt * du.z, bt * du.w};
        const f32x4 u = {__builtin_fmaf(-at, p.x, v4.x), __builtin_fmaf(-at, p.y, v4.y),
                         __builtin_fmaf(-at, p.z, v4.z), __builtin_fmaf(-at, p.w, v4.w)};
        const f32x4 dp = {-at * du.x, -at * du.y, -at * du.z, -at * du.w};
        if (live) *reinterpret_cast<f32x4 *>(A.dv + row * d_v + col) = du;
        float sa = -dot4(p, du), sb = 0.f;
        // second pass: the scalar gradients and the new G rows
        for (int64_t j = 0; j < W; ++j) {
            const int32_t wi = A.widx[row * W + j];
            const float ww = A.wwt[row * W + j];
            const f32x4 x = live ? ld4(X + ((t * nch + c) * W + j) * 4) : zero;
            const uint32_t off = goff(wi);
            const f32x4 dy = live ? gld(off) : zero;
            const float yu = dot4(dy, u), px = dot4(dp, x);
            gst((f32x4){__builtin_fmaf(at, dy.x, ww * dp.x), __builtin_fmaf(at, dy.y, ww * dp.y),
                        __builtin_fmaf(at, dy.z, ww * dp.z), __builtin_fmaf(at, dy.w, ww * dp.w)},
                off);
            const float dws = group_sum_qc<QC>(__builtin_fmaf(bt, yu, px));
            if (lead) A.dw[row * W + j] = dws;
            sa += dot4(dy, x);
            sb = __builtin_fmaf(ww, yu, sb);
        }
        sa = group_sum_qc<QC>(sa);
        sb = group_sum_qc<QC>(sb);
        if (lead) {
            A.da[row] = sa;
            A.db[row] = sb;
        }
    }
}

hipError_t launch_scan_backward_chunks(const BwdArgs &A, bool bf16, hipStream_t stream);

// The same recurrence with the rows of a token spread over lanes: lane
// (chunk cl, list position j) of a wave, Q = the power of two >= max(W, R)
// lanes per chunk, 64/Q chunks per wave, and one workgroup per chain holding
// all its chunks (at most 16 waves).  Per token a lane read-modify-writes
// its read row's chunk of G, then its write row's (one wave's stores precede
// its later loads, and no other wave touches these bytes), the prediction
// and du are sums over the Q lanes of a chunk, and the scalar gradients are
// summed over the chunks: within a wave by a butterfly, across the waves
// through LDS (double-buffered by token, one barrier per token).  The
// token's inputs other than G (slots, weights, saved rows, dL/do, v, gates)
// are loaded one token ahead.
template <int Q, bool BF16>
struct BwdTok {
    int32_t ri, wi;
    float rw, ww, a, b;
    f32x4 z, x, dov;
    uint32_t v[BF16 ? 2 : 4];
};

template <int Q, bool BF16>
__global__ void __launch_bounds__(1024) sdm_scan_backward_rows_kernel(BwdArgs A)
{
    constexpr int CPW = kWave / Q;               // chunks per wave
    __shared__ float part[2][16][2 * kWave + 2]; // per wave: dw_j, dr_j, da, db
    const int64_t chain = blockIdx.x;
    const int64_t bb = chain / A.H, h = chain - bb * A.H;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int nwaves = blockDim.x / kWave;
    const int lane = lane_id();
    const int j = lane % Q, cl = lane / Q;
    const int nchunk = A.d_v / 4;
    const int c0 = wave * CPW + cl;
    const bool live = c0 < nchunk;
    const int c = live ? c0 : nchunk - 1;
    const int64_t T = A.T, d_v = A.d_v, W = A.W, R = A.R;
    const bool jw = j < W, jr = j < R;
    const int jwc = jw ? j : 0, jrc = jr ? j : 0;   // valid positions for the loads of idle lanes
    const int64_t col = (int64_t)c * 4;
    const __amdgpu_buffer_rsrc_t Grs = make_rsrc(A.dM + chain * (int64_t)A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
    constexpr uint32_t kOOB = 0x80000000u;
    const uint32_t rowb = (uint32_t)d_v * 4u, colb = (uint32_t)col * 4u;
    auto goff = [&](bool on, int32_t slot) {
        return (on && live && slot >= 0 && slot < A.N) ? (uint32_t)slot * rowb + colb : kOOB;
    };
    // saved rows [T][d_v/4][W or R][4] of this chain
    const float *X = A.xsave + chain * T * W * d_v;
    const float *Z = A.zsave + chain * T * R * d_v;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    auto load_tok = [&](int64_t t, BwdTok<Q, BF16> &k) {
        const int64_t tt = t >= 0 ? t : 0;       // before the first token: a valid one, never used
        const int64_t row = (bb * T + tt) * A.H + h;
        k.ri = A.ridx[row * R + jrc];
        k.rw = A.rwt[row * R + jrc];
        k.wi = A.widx[row * W + jwc];
        k.ww = A.wwt[row * W + jwc];
        k.a = A.a[row];
        k.b = A.b[row];
        // the saved rows are read once: non-temporal loads
        k.z = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Z + ((tt * nchunk + c) * R + jrc) * 4));
        k.x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(X + ((tt * nchunk + c) * W + jwc) * 4));
        k.dov = ld4(A.dout + row * d_v + col);
        if constexpr (BF16) {
            const uint2 r = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(A.v) + row * d_v + col);
            k.v[0] = r.x; k.v[1] = r.y;
        } else {
            const f32x4 r = ld4(static_cast<const float *>(A.v) + row * d_v + col);
            k.v[0] = __float_as_uint(r.x); k.v[1] = __float_as_uint(r.y);
            k.v[2] = __float_as_uint(r.z); k.v[3] = __float_as_uint(r.w);
        }
    };

    auto step = [&](const BwdTok<Q, BF16> &k, int64_t t) {
        const int64_t row = (bb * T + t) * A.H + h;
        const int buf = (int)(t & 1);
        const f32x4 dov = live ? k.dov : zero;
        f32x4 v4;
        if constexpr (BF16)
            v4 = v_chunk(make_uint2(k.v[0], k.v[1]));
        else
            v4 = (f32x4){__uint_as_float(k.v[0]), __uint_as_float(k.v[1]), __uint_as_float(k.v[2]),
                         __uint_as_float(k.v[3])};
        // the read row: its output's gradient, then into G.  A slot listed
        // at several read positions of the token is updated once, by its
        // first position, with the sum of those positions' weights in list
        // order (two lanes storing to one address in one instruction would
        // lose a term).  The lists of all chunks are the same, so lane s
        // holds position s.
        const uint32_t roff0 = goff(jr, k.ri);
        const f32x4 gv = __builtin_amdgcn_raw_buffer_load_b128(Grs, roff0, 0, 0);
        uint64_t later = 0;   // lanes whose slot is also at an earlier position
#pragma unroll
        for (int s = 0; s + 1 < Q; ++s) {
            if (s + 1 >= R) break;   // uniform
            const int32_t ss = __builtin_amdgcn_readlane(k.ri, s);
            later |= __builtin_amdgcn_ballot_w64(jr && j > s && k.ri == ss);
        }
        float rw = jr ? k.rw : 0.f;
        if (later != 0) {   // uniform, and rare: repeated read slots
            float sum = 0.f;
            for (int s = 0; s < R; ++s) {
                const int32_t ss = __builtin_amdgcn_readlane(k.ri, s);
                const float ws = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(k.rw), s));
                if (k.ri == ss) sum += ws;
            }
            rw = jr ? sum : 0.f;
        }
        const uint32_t roff = ((later >> lane) & 1u) ? kOOB : roff0;
        __builtin_amdgcn_raw_buffer_store_b128(
            (f32x4){__builtin_fmaf(rw, dov.x, gv.x), __builtin_fmaf(rw, dov.y, gv.y), __builtin_fmaf(rw, dov.z, gv.z),
                    __builtin_fmaf(rw, dov.w, gv.w)},
            Grs, roff, 0, 0);
        asm volatile("" ::: "memory");
        float drp = (jr && live) ? dot4(dov, k.z) : 0.f;
        // the write row
        const uint32_t woff = goff(jw, k.wi);
        const f32x4 dy = __builtin_amdgcn_raw_buffer_load_b128(Grs, woff, 0, 0);   // zeros when idle
        const float ww = jw ? k.ww : 0.f;
        const f32x4 x = (jw && live) ? k.x : zero;
        const f32x4 p = weighted_rows<Q>(ww, x);
        const f32x4 du = mul4(k.b, weighted_rows<Q>(ww, dy));
        const f32x4 u = {__builtin_fmaf(-k.a, p.x, v4.x), __builtin_fmaf(-k.a, p.y, v4.y),
                         __builtin_fmaf(-k.a, p.z, v4.z), __builtin_fmaf(-k.a, p.w, v4.w)};
        const f32x4 dp = mul4(-k.a, du);
        __builtin_amdgcn_raw_buffer_store_b128(
            (f32x4){__builtin_fmaf(k.a, dy.x, ww * dp.x), __builtin_fmaf(k.a, dy.y, ww * dp.y),
                    __builtin_fmaf(k.a, dy.z, ww * dp.z), __builtin_fmaf(k.a, dy.w, ww * dp.w)},
            Grs, woff, 0, 0);
        asm volatile("" ::: "memory");
        if (j == 0 && live) *reinterpret_cast<f32x4 *>(A.dv + row * d_v + col) = du;
        const float yu = dot4(dy, u);
        float dwp = jw ? __builtin_fmaf(k.b, yu, dot4(dp, x)) : 0.f;
        float sa = dot4(dy, x) - ((j == 0 && live) ? dot4(p, du) : 0.f);
        float sb = ww * yu;
        // sums over the chunks of the wave (lanes j, j + Q, ...), then of the whole wave for da, db
        auto across = [&](auto jc) {
            constexpr int J = decltype(jc)::value;
            if constexpr (J >= Q && J < kWave) {
                dwp += __uint_as_float(lane_xor<J>(__float_as_uint(dwp)));
                drp += __uint_as_float(lane_xor<J>(__float_as_uint(drp)));
            }
        };
        across(std::integral_constant<int, 4>{});
        across(std::integral_constant<int, 8>{});
        across(std::integral_constant<int, 16>{});
        across(std::integral_constant<int, 32>{});
        sa = wave_sum_f32(sa);
        sb = wave_sum_f32(sb);
        if (cl == 0) {
            part[buf][wave][j] = dwp;
            part[buf][wave][kWave + j] = drp;
        }
        if (lane == 0) {
            part[buf][wave][2 * kWave] = sa;
            part[buf][wave][2 * kWave + 1] = sb;
        }
        __syncthreads();
        if (wave == 0) {
            float sw = 0.f, sr = 0.f;
            for (int w = 0; w < nwaves; ++w) {
                sw += part[buf][w][lane];
                sr += part[buf][w][kWave + lane];
            }
            if (lane < W) A.dw[row * W + lane] = sw;
            if (lane < R) A.dr[row * R + lane] = sr;
            if (lane == 0) {
                float ta = 0.f, tb = 0.f;
                for (int w = 0; w < nwaves; ++w) {
                    ta += part[buf][w][2 * kWave];
                    tb += part[buf][w][2 * kWave + 1];
                }
                A.da[row] = ta;
                A.db[row] = tb;
            }
        }
    };

    BwdTok<Q, BF16> k0, k1;
    load_tok(T - 1, k0);
    for (int64_t t = T - 1;;) {
        load_tok(t - 1, k1);
        step(k0, t);
        if (--t < 0) break;
        load_tok(t - 1, k0);
        step(k1, t);
        if (--t < 0) break;
    }
}

// the lane layout fits when one workgroup of at most 16 waves holds a chain
static bool rows_layout_fits(int d_v, int W, int R, int &q)
{
    q = 4;
    while (q < W || q < R) q *= 2;
    const int cpw = 64 / q;
    const int nwaves = (d_v / 4 + cpw - 1) / cpw;
    return nwaves <= 16;
}

hipError_t launch_scan_backward(const BwdArgs &A, bool bf16, hipStream_t stream)
{
    if (A.B * A.H == 0 || A.T == 0) return hipSuccess;
    int q = 0;
    if (rows_layout_fits(A.d_v, A.W, A.R, q)) {
        const int cpw = 64 / q;
        const int nwaves = (A.d_v / 4 + cpw - 1) / cpw;
        const dim3 grid((unsigned)(A.B * A.H)), block(64 * nwaves);
#define SDM_BWD_ROWS(QV)                                                                                  \
    case QV:                                                                                              \
        if (bf16)                                                                                         \
            hipLaunchKernelGGL((sdm_scan_backward_rows_kernel<QV, true>), grid, block, 0, stream, A);     \
        else                                                                                              \
            hipLaunchKernelGGL((sdm_scan_backward_rows_kernel<QV, false>), grid, block, 0, stream, A);    \
        break;
        switch (q) {
            SDM_BWD_ROWS(4)
            SDM_BWD_ROWS(8)
            SDM_BWD_ROWS(16)
            SDM_BWD_ROWS(32)
            SDM_BWD_ROWS(64)
        default: return hipErrorInvalidValue;
        }
#undef SDM_BWD_ROWS
        return hipGetLastError();
    }
    return launch_scan_backward_chunks(A, bf16, stream);
}

hipError_t launch_scan_backward_chunks(const BwdArgs &A, bool bf16, hipStream_t stream)
{
    const int64_t chains = A.B * A.H;
    if (chains == 0 || A.T == 0) return hipSuccess;
    int qc = 1;
    while (qc < A.d_v / 4) qc *= 2;
    const int64_t cpb = 256 / qc;
    const dim3 grid((unsigned)((chains + cpb - 1) / cpb)), block(256);
#define SDM_BWD(Q)                                                                                  \
    case Q:                                                                                         \
        if (bf16)                                                                                   \
            hipLaunchKernelGGL((sdm_scan_backward_kernel<Q, true>), grid, block, 0, stream, A);     \
        else                                                                                        \
            hipLaunchKernelGGL((sdm_scan_backward_kernel<Q, false>), grid, block, 0, stream, A);    \
        break;
    switch (qc) {
        SDM_BWD(8)
        SDM_BWD(16)
        SDM_BWD(32)
        SDM_BWD(64)
    default: return hipErrorInvalidValue;
    }
#undef SDM_BWD
    return hipGetLastError();
}

}  // namespace sdm
