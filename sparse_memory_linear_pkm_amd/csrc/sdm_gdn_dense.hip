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
// so columns live in the registers of an aligned group of 16 lanes, EPL =
// d_k / 16 entries of each per lane, for the whole sequence: a group holds
// CPL = 2 columns (they share the loads and bf16 conversions of k and q), a
// wave 8 columns of one (sequence, head), a workgroup 32.  Per token a lane
// reads its EPL entries of k and q (the other groups of the workgroup read
// the same bytes, from L1), its v_c, and the two gates.  The two dot products
// are per-lane FMA chains followed by a 16-lane butterfly of DPP adds, so
// every lane of the group holds the same sum.  The inputs of the next tokens
// are loaded while the current ones compute.
// Bound: the VALU.  Per token and column about 32 multiply-adds (half the
// VALU instructions issued; the rest are the bf16 conversions, the
// butterflies and addressing); packed fp32 math is not used.
#include "device_common.h"
#include "kernels.h"

namespace sdm {

namespace {

constexpr int kGdnLanes = 16;   // lanes per state column
constexpr int kGdnCpl = 2;      // state columns per lane group
constexpr int kGdnGroups = 16;  // lane groups per workgroup (4 waves)
constexpr int kGdnPf = 2;       // tokens of input loaded ahead (per register set)

// One token's inputs for one lane, as loaded (bf16 pairs or fp32): EPL
// entries of k and q, v_c and the two gates.  Converted to fp32 where used,
// so that the registers a load writes are not copied before it completes.
template <int EPL, int CPL, bool BF16>
struct GdnTok {
    static constexpr int NW = BF16 ? (EPL + 1) / 2 : EPL;   // 32-bit words per vector
    uint32_t k[NW], q[NW];
    float v[CPL], a, b;
};

// the NW words of a lane's vector entries, starting at element e
template <int EPL, bool BF16>
__device__ __forceinline__ void load_words(const void *p, int64_t e, uint32_t (&w)[BF16 ? (EPL + 1) / 2 : EPL])
{
    constexpr int NW = BF16 ? (EPL + 1) / 2 : EPL;
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

template <int C>
__device__ __forceinline__ float add_dpp1(float x)
{
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), C, 0xF, 0xF, true));
}

// sum over the aligned group of 16 lanes, the same bits in every lane: each
// stage adds two partial sums of disjoint lane blocks (lane ^ 1, lane ^ 2,
// then the mirrors within 8 and within 16), one DPP add each
__device__ __forceinline__ float sum16(float x)
{
    x = add_dpp1<0xB1>(x);    // quad_perm [1,0,3,2]
    x = add_dpp1<0x4E>(x);    // quad_perm [2,3,0,1]
    x = add_dpp1<0x141>(x);   // row_half_mirror
    x = add_dpp1<0x140>(x);   // row_mirror
    return x;
}

}  // namespace

// CPL columns per lane group (they share the loads and conversions of k and
// q), GROUPS lane groups per workgroup.
template <int EPL, int CPL, int GROUPS, bool BF16>
__global__ void __launch_bounds__(kGdnLanes * GROUPS) sdm_gdn_dense_kernel(GdnArgs A)
{
    constexpr int kColsWg = GROUPS * CPL;
    const int ncb = (A.d_v + kColsWg - 1) / kColsWg;        // column blocks per (b, h)
    const int64_t bh = blockIdx.x / ncb;
    const int cb = (int)(blockIdx.x - bh * ncb);
    const int64_t bb = bh / A.H;
    const int h = (int)(bh - bb * A.H);
    const int lane16 = threadIdx.x % kGdnLanes;
    const int colg = cb * kColsWg + (int)(threadIdx.x / kGdnLanes) * CPL;   // the group's first column
    const int d_k = EPL * kGdnLanes, d_v = A.d_v;
    const int j0 = lane16 * EPL;                           // this lane's rows of its columns
    bool live[CPL];
    int col[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        live[c] = colg + c < d_v;
        col[c] = live[c] ? colg + c : d_v - 1;             // dead columns compute a valid one, store nothing
    }

    float *Sc = A.S + bh * (int64_t)d_k * d_v;
    float s[CPL][EPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < EPL; ++e) s[c][e] = Sc[(int64_t)(j0 + e) * d_v + col[c]];

    const int64_t T = A.T;
    // the inputs of token t (a valid token past the end; those are never used)
    auto load_tok = [&](int64_t t, GdnTok<EPL, CPL, BF16> &x) {
        const int64_t tt = t < T ? t : T - 1;
        const int64_t row = (bb * T + tt) * A.H + h;
        load_words<EPL, BF16>(A.k, row * d_k + j0, x.k);
        load_words<EPL, BF16>(A.q, row * d_k + j0, x.q);
#pragma unroll
        for (int c = 0; c < CPL; ++c) x.v[c] = load_one<BF16>(A.v, row * d_v + col[c]);
        x.a = A.a[row];
        x.b = A.b[row];
    };
    auto step = [&](const GdnTok<EPL, CPL, BF16> &x, int64_t t) {
        float kf[EPL], pp[CPL], oo[CPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) kf[e] = word_entry<EPL, BF16>(x.k, e);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            pp[c] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) pp[c] = __builtin_fmaf(kf[e], s[c][e], pp[c]);
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) pp[c] = sum16(pp[c]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float u = __builtin_fmaf(-x.a, pp[c], x.v[c]);   // v_c - a p
            const float bu = x.b * u;
            oo[c] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                s[c][e] = __builtin_fmaf(x.a, s[c][e], bu * kf[e]);
                oo[c] = __builtin_fmaf(word_entry<EPL, BF16>(x.q, e), s[c][e], oo[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) oo[c] = sum16(oo[c]);
        if (lane16 == 0) {
            float *orow = A.o + ((bb * T + t) * A.H + h) * d_v;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                if (live[c]) orow[col[c]] = oo[c];
        }
    };

    // groups of PF tokens in two register sets: the next group's loads are in
    // flight while the current group computes (T >= 1 here)
    GdnTok<EPL, CPL, BF16> g0[kGdnPf], g1[kGdnPf];
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
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        if (live[c]) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) Sc[(int64_t)(j0 + e) * d_v + col[c]] = s[c][e];
        }
}

template <int EPL, bool BF16>
static void launch_gdn_epl(const GdnArgs &A, hipStream_t stream)
{
    constexpr int CPL = kGdnCpl, GROUPS = kGdnGroups;
    const int64_t ncb = (A.d_v + GROUPS * CPL - 1) / (GROUPS * CPL);
    const dim3 grid((unsigned)(A.B * A.H * ncb)), block(kGdnLanes * GROUPS);
    hipLaunchKernelGGL((sdm_gdn_dense_kernel<EPL, CPL, GROUPS, BF16>), grid, block, 0, stream, A);
}

hipError_t launch_gdn_dense(const GdnArgs &A, bool bf16, hipStream_t stream)
{
    if (A.B * A.H == 0 || A.T == 0) return hipSuccess;
    const int epl = A.d_k / kGdnLanes;
    if (bf16) {
        switch (epl) {
        case 1: launch_gdn_epl<1, true>(A, stream); break;
        case 2: launch_gdn_epl<2, true>(A, stream); break;
        case 4: launch_gdn_epl<4, true>(A, stream); break;
        case 8: launch_gdn_epl<8, true>(A, stream); break;
        case 16: launch_gdn_epl<16, true>(A, stream); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (epl) {
        case 1: launch_gdn_epl<1, false>(A, stream); break;
        case 2: launch_gdn_epl<2, false>(A, stream); break;
        case 4: launch_gdn_epl<4, false>(A, stream); break;
        case 8: launch_gdn_epl<8, false>(A, stream); break;
        case 16: launch_gdn_epl<16, false>(A, stream); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace sdm
