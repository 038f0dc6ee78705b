// sdm_gdn_dense.hip -- the dense Gated DeltaNet recurrence, the rule that the
// sparse memory reduces to when every slot is selected with a dense key.
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 2 Eq. 2 (Gated DeltaNet) and Sec. 3.1 "Connection to GDN":
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t.
// The state is stored transposed, like the sparse memory with N = d_k slots:
// S [B,H,d_k,d_v], row j for key dimension j.
//
// Every column c of the state (one value feature) is an independent
// recurrence over a d_k-vector s = S[:, c]:
//     p = k . s;  s <- a s + b (v_c - a p) k;  o_c = q . s
// so a column lives in the registers of an aligned group of 16 lanes, EPL =
// d_k / 16 entries per lane, for the whole sequence; a wave holds 4 columns
// of one (sequence, head) and a workgroup 16.  Per token a lane reads its
// EPL entries of k and q (the other groups of the workgroup read the same
// bytes, from L1), v_c, and the two gates, which are uniform across the
// workgroup.  The two dot products are per-lane FMA chains followed by a
// 16-lane butterfly, so every lane of the group holds the same sum.  The
// inputs of the next PF tokens are loaded while the current ones compute.
// Bound: the VALU (about 3 d_k FMAs and 8 lane exchanges per column and token).
#include "device_common.h"
#include "kernels.h"

namespace sdm {

namespace {

constexpr int kGdnLanes = 16;   // lanes per state column
constexpr int kGdnCols = 16;    // columns per workgroup (4 waves)
constexpr int kGdnPf = 4;       // tokens of input loaded ahead

// One token's inputs for one lane, as loaded (bf16 pairs or fp32): EPL
// entries of k and q, v_c and the two gates.  Converted to fp32 where used,
// so that the registers a load writes are not copied before it completes.
template <int EPL, bool BF16>
struct GdnTok {
    static constexpr int NW = BF16 ? (EPL + 1) / 2 : EPL;   // 32-bit words per vector
    uint32_t k[NW], q[NW];
    float v, a, b;
};

// the NW words of a lane's vector entries, starting at element e
template <int EPL, bool BF16>
__device__ __forceinline__ void load_words(const void *p, int64_t e, uint32_t (&w)[GdnTok<EPL, BF16>::NW])
{
    constexpr int NW = GdnTok<EPL, BF16>::NW;
    const unsigned char *s = static_cast<const unsigned char *>(p) + e * (BF16 ? 2 : 4);
    if constexpr (BF16 && EPL == 1) {
        w[0] = *reinterpret_cast<const uint16_t *>(s);
    } else if constexpr (NW == 1) {
        w[0] = *reinterpret_cast<const uint32_t *>(s);
    } else if constexpr (NW == 2) {
        const uint2 r = *reinterpret_cast<const uint2 *>(s);
        w[0] = r.x; w[1] = r.y;
    } else {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const uint4 r = reinterpret_cast<const uint4 *>(s)[i];
            w[4 * i] = r.x; w[4 * i + 1] = r.y; w[4 * i + 2] = r.z; w[4 * i + 3] = r.w;
        }
    }
}

// entry i of a vector held as NW words
template <int EPL, bool BF16>
__device__ __forceinline__ float word_entry(const uint32_t *w, int i)
{
    if constexpr (BF16)
        return __uint_as_float((i & 1) ? (w[i / 2] & 0xffff0000u) : (w[i / 2] << 16));
    else
        return __uint_as_float(w[i]);
}

template <bool BF16>
__device__ __forceinline__ float load_one(const void *p, int64_t e)
{
    if constexpr (BF16)
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[e] << 16);
    else
        return static_cast<const float *>(p)[e];
}

// sum over the aligned group of 16 lanes, the same bits in every lane
__device__ __forceinline__ float sum16(float x)
{
    x += __uint_as_float(lane_xor<1>(__float_as_uint(x)));
    x += __uint_as_float(lane_xor<2>(__float_as_uint(x)));
    x += __uint_as_float(lane_xor<4>(__float_as_uint(x)));
    x += __uint_as_float(lane_xor<8>(__float_as_uint(x)));
    return x;
}

}  // namespace

template <int EPL, bool BF16>
__global__ void __launch_bounds__(64 * kGdnCols / 4) sdm_gdn_dense_kernel(GdnArgs A)
{
    const int ncb = (A.d_v + kGdnCols - 1) / kGdnCols;     // column blocks per (b, h)
    const int64_t bh = blockIdx.x / ncb;
    const int cb = (int)(blockIdx.x - bh * ncb);
    const int64_t bb = bh / A.H;
    const int h = (int)(bh - bb * A.H);
    const int lane16 = threadIdx.x % kGdnLanes;
    const int col0 = cb * kGdnCols + (int)(threadIdx.x / kGdnLanes);
    const bool live = col0 < A.d_v;
    const int col = live ? col0 : A.d_v - 1;                // dead groups compute a valid column, store nothing
    const int d_k = EPL * kGdnLanes, d_v = A.d_v;
    const int j0 = lane16 * EPL;                           // this lane's rows of the column

    float *Sc = A.S + bh * (int64_t)d_k * d_v;
    float s[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) s[e] = Sc[(int64_t)(j0 + e) * d_v + col];

    const int64_t T = A.T;
    // the inputs of token t (a valid token past the end; those are never used)
    auto load_tok = [&](int64_t t, GdnTok<EPL, BF16> &x) {
        const int64_t tt = t < T ? t : T - 1;
        const int64_t row = (bb * T + tt) * A.H + h;
        load_words<EPL, BF16>(A.k, row * d_k + j0, x.k);
        load_words<EPL, BF16>(A.q, row * d_k + j0, x.q);
        x.v = load_one<BF16>(A.v, row * d_v + col);
        x.a = A.a[row];
        x.b = A.b[row];
    };
    auto step = [&](const GdnTok<EPL, BF16> &x, int64_t t) {
        float pp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) pp = __builtin_fmaf(word_entry<EPL, BF16>(x.k, e), s[e], pp);
        const float p = sum16(pp);
        const float u = __builtin_fmaf(-x.a, p, x.v);   // v_c - a p
        const float bu = x.b * u;
        float oo = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            s[e] = __builtin_fmaf(x.a, s[e], bu * word_entry<EPL, BF16>(x.k, e));
            oo = __builtin_fmaf(word_entry<EPL, BF16>(x.q, e), s[e], oo);
        }
        const float o = sum16(oo);
        if (live && lane16 == 0) A.o[((bb * T + t) * A.H + h) * d_v + col] = o;
    };

    // groups of PF tokens in two register sets: the next group's loads are in
    // flight while the current group computes (T >= 1 here)
    GdnTok<EPL, BF16> g0[kGdnPf], g1[kGdnPf];
#pragma unroll
    for (int i = 0; i < kGdnPf; ++i) load_tok(i, g0[i]);
    for (int64_t t = 0;;) {
#pragma unroll
        for (int i = 0; i < kGdnPf; ++i) load_tok(t + kGdnPf + i, g1[i]);
#pragma unroll
        for (int i = 0; i < kGdnPf; ++i)
            if (t + i < T) step(g0[i], t + i);
        t += kGdnPf;
        if (t >= T) break;
#pragma unroll
        for (int i = 0; i < kGdnPf; ++i) load_tok(t + kGdnPf + i, g0[i]);
#pragma unroll
        for (int i = 0; i < kGdnPf; ++i)
            if (t + i < T) step(g1[i], t + i);
        t += kGdnPf;
        if (t >= T) break;
    }
    if (live) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) Sc[(int64_t)(j0 + e) * d_v + col] = s[e];
    }
}

hipError_t launch_gdn_dense(const GdnArgs &A, bool bf16, hipStream_t stream)
{
    const int64_t ncb = (A.d_v + kGdnCols - 1) / kGdnCols;
    const int64_t blocks = A.B * A.H * ncb;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(64 * kGdnCols / 4);
#define SDM_GDN_LAUNCH(E, BF) hipLaunchKernelGGL((sdm_gdn_dense_kernel<E, BF>), grid, block, 0, stream, A)
    const int epl = A.d_k / kGdnLanes;
    if (bf16) {
        switch (epl) {
        case 1: SDM_GDN_LAUNCH(1, true); break;
        case 2: SDM_GDN_LAUNCH(2, true); break;
        case 4: SDM_GDN_LAUNCH(4, true); break;
        case 8: SDM_GDN_LAUNCH(8, true); break;
        case 16: SDM_GDN_LAUNCH(16, true); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (epl) {
        case 1: SDM_GDN_LAUNCH(1, false); break;
        case 2: SDM_GDN_LAUNCH(2, false); break;
        case 4: SDM_GDN_LAUNCH(4, false); break;
        case 8: SDM_GDN_LAUNCH(8, false); break;
        case 16: SDM_GDN_LAUNCH(16, false); break;
        default: return hipErrorInvalidValue;
        }
    }
#undef SDM_GDN_LAUNCH
    return hipGetLastError();
}

}  // namespace sdm
