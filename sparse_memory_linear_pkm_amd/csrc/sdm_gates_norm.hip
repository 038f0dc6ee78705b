// sdm_gates_norm.hip -- the element-wise steps either side of the path:
// the forget and input gates that the scan consumes, and the read-out's RMS
// norm with its output gate, which feeds the head-mixing projection.
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 step 2 (per-head forget gate a_t with a learnable decay A, input
// gate b_t), Sec. 3.1 step 4 (RMS-Norm, element-wise output gate) and Sec. 4
// (the decay and the time-step bias follow the Gated DeltaNet conventions).
//
// Both are streaming kernels bound by HBM bandwidth: every input element is
// read once and every output element written once, with coalesced accesses.
#include "device_common.h"
#include "kernels.h"

namespace sdm {

// 1 / (1 + e^-x) in the form whose exponential cannot overflow (so that
// very negative x give their subnormal values rather than 0)
__device__ __forceinline__ float sigmoid(float x)
{
    const float e = expf(-fabsf(x));
    return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// a = exp(-A[h] softplus(a_raw + dt_bias[h])), b = sigmoid(b_raw); one
// token-head per thread.  a may be the same buffer as a_raw and b the same
// as b_raw: each thread reads its element before writing it.
__global__ void __launch_bounds__(256) sdm_gates_kernel(GateArgs G)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= G.n) return;
    const int h = (int)(i % G.H);
    const float z = G.a_raw[i] + G.dt_bias[h];
    const float braw = G.b_raw[i];
    // ln(1 + e^z) in the form whose exponential cannot overflow
    const float sp = z > 0.f ? z + log1pf(expf(-z)) : log1pf(expf(z));
    G.a[i] = expf(-G.A[h] * sp);
    G.b[i] = sigmoid(braw);
}

hipError_t launch_gates(const GateArgs &G, hipStream_t stream)
{
    if (G.n == 0) return hipSuccess;
    const int64_t blocks = (G.n + 255) / 256;
    hipLaunchKernelGGL(sdm_gates_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, G);
    return hipGetLastError();
}

namespace {

// four consecutive elements of g as fp32
template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void *p, int64_t e)
{
    if constexpr (BF16) {
        const uint2 r = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + e);
        return (f32x4){__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
    } else {
        return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + e);
    }
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_rne(float x)
{
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <bool BF16>
__device__ __forceinline__ void store4(void *p, int64_t e, f32x4 y)
{
    if constexpr (BF16) {
        const uint2 r = {bf16_rne(y.x) | (bf16_rne(y.y) << 16), bf16_rne(y.z) | (bf16_rne(y.w) << 16)};
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p) + e) = r;
    } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(p) + e) = y;
    }
}

__device__ __forceinline__ float silu(float g) { return g * sigmoid(g); }

__device__ __forceinline__ f32x4 norm_gate4(f32x4 x, float inv, f32x4 gm, f32x4 g)
{
    return (f32x4){x.x * inv * gm.x * silu(g.x), x.y * inv * gm.y * silu(g.y), x.z * inv * gm.z * silu(g.z),
                   x.w * inv * gm.w * silu(g.w)};
}

}  // namespace

// y = o / sqrt(mean(o^2) + eps) * gamma * silu(g) per token-head row of d_v
// features.  An aligned group of 8 lanes takes one row: lane l holds the
// 4-column chunks l, l + 8, ... (each group access is 128 contiguous bytes of
// o), sums its squares and the group adds the 8 partial sums with a
// butterfly, so every lane of the group has the same sum.  NC = d_v / 32
// chunks per lane kept in registers (1, 2 or 4); NC = 0 reads o again for
// the output pass (other d_v).
template <bool BF16, int NC>
__global__ void __launch_bounds__(256) sdm_out_norm_gate_kernel(NormArgs A)
{
    const int gl = threadIdx.x & 7;
    const int64_t row0 = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const bool live = row0 < A.rows;
    const int64_t row = live ? row0 : A.rows - 1;   // groups past the end load a valid row, store nothing
    const int d_v = A.d_v;
    const int nc = NC > 0 ? NC : d_v / 32;
    const float *orow = A.o + row * d_v;
    const int64_t base = row * d_v;
    float ss = 0.f;
    f32x4 ov[NC > 0 ? NC : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int k = 0; k < NC; ++k) ov[k] = *reinterpret_cast<const f32x4 *>(orow + (gl + 8 * k) * 4);
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            ss = __builtin_fmaf(ov[k].x, ov[k].x, ss);
            ss = __builtin_fmaf(ov[k].y, ov[k].y, ss);
            ss = __builtin_fmaf(ov[k].z, ov[k].z, ss);
            ss = __builtin_fmaf(ov[k].w, ov[k].w, ss);
        }
    } else {
        for (int k = 0; k < nc; ++k) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(orow + (gl + 8 * k) * 4);
            ss = __builtin_fmaf(x.x, x.x, ss);
            ss = __builtin_fmaf(x.y, x.y, ss);
            ss = __builtin_fmaf(x.z, x.z, ss);
            ss = __builtin_fmaf(x.w, x.w, ss);
        }
    }
    ss += __uint_as_float(lane_xor<1>(__float_as_uint(ss)));
    ss += __uint_as_float(lane_xor<2>(__float_as_uint(ss)));
    ss += __uint_as_float(lane_xor<4>(__float_as_uint(ss)));
    const float inv = 1.f / sqrtf(ss / (float)d_v + A.eps);
    if constexpr (NC > 0) {
        f32x4 gv[NC], gm[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int col = (gl + 8 * k) * 4;
            gv[k] = load4<BF16>(A.g, base + col);
            gm[k] = *reinterpret_cast<const f32x4 *>(A.gamma + col);
        }
        if (live) {
#pragma unroll
            for (int k = 0; k < NC; ++k)
                store4<BF16>(A.y, base + (gl + 8 * k) * 4, norm_gate4(ov[k], inv, gm[k], gv[k]));
        }
    } else {
        for (int k = 0; k < nc; ++k) {
            const int col = (gl + 8 * k) * 4;
            const f32x4 x = *reinterpret_cast<const f32x4 *>(orow + col);
            const f32x4 gv = load4<BF16>(A.g, base + col);
            const f32x4 gm = *reinterpret_cast<const f32x4 *>(A.gamma + col);
            if (live) store4<BF16>(A.y, base + col, norm_gate4(x, inv, gm, gv));
        }
    }
}

hipError_t launch_out_norm_gate(const NormArgs &A, bool bf16, hipStream_t stream)
{
    if (A.rows == 0) return hipSuccess;
    const int64_t blocks = (A.rows + 31) / 32;
    const dim3 grid((unsigned)blocks), block(256);
    const int nc = A.d_v / 32;
#define SDM_NORM_LAUNCH(B, N) hipLaunchKernelGGL((sdm_out_norm_gate_kernel<B, N>), grid, block, 0, stream, A)
    if (bf16) {
        if (nc == 1) SDM_NORM_LAUNCH(true, 1);
        else if (nc == 2) SDM_NORM_LAUNCH(true, 2);
        else if (nc == 4) SDM_NORM_LAUNCH(true, 4);
        else SDM_NORM_LAUNCH(true, 0);
    } else {
        if (nc == 1) SDM_NORM_LAUNCH(false, 1);
        else if (nc == 2) SDM_NORM_LAUNCH(false, 2);
        else if (nc == 4) SDM_NORM_LAUNCH(false, 4);
        else SDM_NORM_LAUNCH(false, 0);
    }
#undef SDM_NORM_LAUNCH
    return hipGetLastError();
}

}  // namespace sdm
