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
    const float *X = A.xsave + chain * T * W * d_v + col;
    const float *Z = A.zsave + chain * T * R * d_v + col;
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
            const f32x4 z = live ? ld4(Z + (t * R + i) * d_v) : zero;
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
            const f32x4 x = live ? ld4(X + (t * W + j) * d_v) : zero;
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
            const f32x4 x = live ? ld4(X + (t * W + j) * d_v) : zero;
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

hipError_t launch_scan_backward(const BwdArgs &A, bool bf16, hipStream_t stream)
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
