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
#include "gates_math.h"
#include "kernels.h"

namespace sdm {

__device__ __forceinline__ float sigmoid(float x) { return gate_sigmoid(x); }

// a = exp(-A[h] softplus(a_raw + dt_bias[h])), b = sigmoid(b_raw); one
// token-head per thread.  a may be the same buffer as a_raw and b the same
// as b_raw: each thread reads its element before writing it.
__global__ void __launch_bounds__(256) sdm_gates_kernel(GateArgs G)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= G.n) return;
    const int h = (int)(i % G.H);
    const float araw = G.a_raw[i], braw = G.b_raw[i];
    G.a[i] = gate_decay(araw, G.dt_bias[h], G.A[h]);
    G.b[i] = gate_sigmoid(braw);
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

// ---------------------------------------------------------------------------
// Gradients (reverse mode of the two functions above).  The sums over tokens
// (the per-head dA and ddt_bias, the per-feature dgamma) are taken in a fixed
// order that depends on the shape only, never on timing, so every result is
// the same bit for bit from run to run.

namespace {

struct GateGrad {
    float da_raw, tA;   // dL/da_raw, and this token-head's term of dL/dA
};

// a = exp(-A softplus(z)), z = a_raw + dt_bias:
//   da/dz = -A a sigmoid(z),  da/dA = -softplus(z) a
__device__ __forceinline__ GateGrad gate_grad(const GateBwdArgs &G, int64_t i, int h)
{
    const float z = G.a_raw[i] + G.dt_bias[h];
    const float sp = z > 0.f ? z + log1pf(expf(-z)) : log1pf(expf(z));
    const float a = expf(-G.A[h] * sp);
    const float da = G.da[i];
    return {da * a * (-G.A[h]) * sigmoid(z), da * a * (-sp)};
}

// sum of 256 per-thread values by a fixed LDS tree; every thread gets it
__device__ float block_sum256(float v, float *red)
{
    red[threadIdx.x] = v;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

}  // namespace

// Layout of the gates' backward: a workgroup of 256 threads is ROWS tokens
// x HP heads (HP the power of two >= H, at most 256), so that each step
// of its loop reads ROWS * HP consecutive elements; grid (ceil(H / HP),
// parts), part p taking a contiguous range of tokens.
GateBwdLayout gates_bwd_layout(int64_t bt, int64_t H)
{
    GateBwdLayout L;
    L.hp = 1;
    while (L.hp < H && L.hp < 256) L.hp *= 2;
    const int64_t rows = 256 / L.hp;
    const int64_t p = (bt + rows * 4 - 1) / (rows * 4);   // at least 4 loop steps per workgroup
    L.parts = (int)(p < 1 ? 1 : p > kGateBwdParts ? kGateBwdParts : p);
    L.chunk = (bt + L.parts - 1) / L.parts;
    L.hblocks = (int)((H + L.hp - 1) / L.hp);
    return L;
}

// Every token-head once: da_raw and db_raw, and this workgroup's partial
// sums of dA and ddt_bias per head (each thread sums its tokens in order,
// then the rows are added in row order).  b = sigmoid(b_raw) gives
// db_raw = db b (1 - b), taken as db e / (1 + e)^2 with e = exp(-|b_raw|):
// the same value, without the cancellation of 1 - b when b is near 1.
__global__ void __launch_bounds__(256) sdm_gates_bwd_kernel(GateBwdArgs G, GateBwdLayout L)
{
    __shared__ float red[2][256];
    const int hl = threadIdx.x % L.hp, r = threadIdx.x / L.hp, rows = 256 / L.hp;
    const int64_t h = (int64_t)blockIdx.x * L.hp + hl;
    const int64_t bt = G.n / G.H;
    const int64_t t0 = (int64_t)blockIdx.y * L.chunk;
    const int64_t t1 = t0 + L.chunk < bt ? t0 + L.chunk : bt;
    float sa = 0.f, sd = 0.f;
    if (h < G.H) {
        for (int64_t t = t0 + r; t < t1; t += rows) {
            const int64_t i = t * G.H + h;
            const GateGrad g = gate_grad(G, i, (int)h);
            G.da_raw[i] = g.da_raw;
            sa += g.tA;
            sd += g.da_raw;
            const float e = expf(-fabsf(G.b_raw[i]));
            const float rc = 1.f / (1.f + e);
            G.db_raw[i] = G.db[i] * (e * rc) * rc;
        }
    }
    red[0][threadIdx.x] = sa;
    red[1][threadIdx.x] = sd;
    __syncthreads();
    if (r == 0 && h < G.H) {
        for (int k = 1; k < rows; ++k) {
            sa += red[0][k * L.hp + hl];
            sd += red[1][k * L.hp + hl];
        }
        G.part[(int64_t)blockIdx.y * G.H + h] = sa;
        G.part[((int64_t)L.parts + blockIdx.y) * G.H + h] = sd;
    }
}

// one workgroup per head: dA[h] and ddt_bias[h] from the parts (thread l
// takes parts l, l + 256, ... in order, then a fixed tree)
__global__ void __launch_bounds__(256) sdm_gates_bwd_reduce_kernel(GateBwdArgs G, int parts)
{
    __shared__ float red[256];
    const int64_t h = blockIdx.x;
    float sa = 0.f, sd = 0.f;
    for (int p = threadIdx.x; p < parts; p += blockDim.x) {
        sa += G.part[(int64_t)p * G.H + h];
        sd += G.part[((int64_t)parts + p) * G.H + h];
    }
    sa = block_sum256(sa, red);
    sd = block_sum256(sd, red);
    if (threadIdx.x == 0) {
        G.dA[h] = sa;
        G.ddt[h] = sd;
    }
}

hipError_t launch_gates_backward(const GateBwdArgs &G, hipStream_t stream)
{
    if (G.n == 0) return hipSuccess;
    const GateBwdLayout L = gates_bwd_layout(G.n / G.H, G.H);
    hipLaunchKernelGGL(sdm_gates_bwd_kernel, dim3((unsigned)L.hblocks, (unsigned)L.parts), dim3(256), 0, stream, G,
                       L);
    hipLaunchKernelGGL(sdm_gates_bwd_reduce_kernel, dim3((unsigned)G.H), dim3(256), 0, stream, G, L.parts);
    return hipGetLastError();
}

// Workgroups of the norm's backward: a fixed number, each taking the 32-row
// tiles blockIdx.x, blockIdx.x + grid, ... so that the dgamma partial sums
// have a fixed count and order.
int norm_bwd_blocks(int64_t rows)
{
    const int64_t tiles = (rows + 31) / 32;
    return (int)(tiles < kNormBwdBlocks ? tiles : kNormBwdBlocks);
}

// With n = o inv (inv = 1/sqrt(mean(o^2) + eps)), s = sigmoid(g) and
// q = dy gamma g s, the gradients of y = n gamma g s are
//   do     = inv (q - n <q, n> / d_v)
//   dg     = dy gamma n s (1 + g (1 - s))
//   dgamma = sum over rows of dy n g s.
// An aligned group of 8 lanes takes one row, as in the forward (the same
// chunk layout and butterfly).  NC = d_v / 32 chunks per lane held in
// registers (1, 2 or 4); NC = 0 reads the row again for the output pass.
// Each group adds its rows' dgamma terms into its own LDS row slot (so the
// order is fixed); at the end the 32 slots are added in slot order, into
// the workgroup's partial row of the workspace.
template <bool BF16, int NC>
__global__ void __launch_bounds__(256) sdm_out_norm_gate_bwd_kernel(NormBwdArgs A)
{
    extern __shared__ __align__(16) float slot[];   // [32][d_v] dgamma terms
    const int gl = threadIdx.x & 7, rl = threadIdx.x >> 3;
    const int d_v = A.d_v;
    const int nc = NC > 0 ? NC : d_v / 32;
    float *myslot = slot + rl * d_v;
    for (int k = 0; k < nc; ++k) *reinterpret_cast<f32x4 *>(myslot + (gl + 8 * k) * 4) = (f32x4){0.f, 0.f, 0.f, 0.f};
    f32x4 gm[NC > 0 ? NC : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int k = 0; k < NC; ++k) gm[k] = *reinterpret_cast<const f32x4 *>(A.gamma + (gl + 8 * k) * 4);
    }
    const int64_t tiles = (A.rows + 31) / 32;
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int64_t row0 = tile * 32 + rl;
        const bool live = row0 < A.rows;
        const int64_t base = (live ? row0 : A.rows - 1) * d_v;   // groups past the end read a valid row
        f32x4 xv[NC > 0 ? NC : 1], gv[NC > 0 ? NC : 1], dyv[NC > 0 ? NC : 1];
        float ss = 0.f, qn = 0.f;
        auto row_terms = [&](f32x4 x, f32x4 g, f32x4 gmk, f32x4 dy) {
            ss = __builtin_fmaf(x.x, x.x, ss);
            ss = __builtin_fmaf(x.y, x.y, ss);
            ss = __builtin_fmaf(x.z, x.z, ss);
            ss = __builtin_fmaf(x.w, x.w, ss);
            // <q, o>: scaled by inv once the row's norm is known
            qn = __builtin_fmaf(dy.x * gmk.x * silu(g.x), x.x, qn);
            qn = __builtin_fmaf(dy.y * gmk.y * silu(g.y), x.y, qn);
            qn = __builtin_fmaf(dy.z * gmk.z * silu(g.z), x.z, qn);
            qn = __builtin_fmaf(dy.w * gmk.w * silu(g.w), x.w, qn);
        };
        if constexpr (NC > 0) {
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                const int col = (gl + 8 * k) * 4;
                xv[k] = *reinterpret_cast<const f32x4 *>(A.o + base + col);
                gv[k] = load4<BF16>(A.g, base + col);
                dyv[k] = *reinterpret_cast<const f32x4 *>(A.dy + base + col);
            }
#pragma unroll
            for (int k = 0; k < NC; ++k) row_terms(xv[k], gv[k], gm[k], dyv[k]);
        } else {
            for (int k = 0; k < nc; ++k) {
                const int col = (gl + 8 * k) * 4;
                row_terms(*reinterpret_cast<const f32x4 *>(A.o + base + col), load4<BF16>(A.g, base + col),
                          *reinterpret_cast<const f32x4 *>(A.gamma + col),
                          *reinterpret_cast<const f32x4 *>(A.dy + base + col));
            }
        }
        ss += __uint_as_float(lane_xor<1>(__float_as_uint(ss)));
        ss += __uint_as_float(lane_xor<2>(__float_as_uint(ss)));
        ss += __uint_as_float(lane_xor<4>(__float_as_uint(ss)));
        qn += __uint_as_float(lane_xor<1>(__float_as_uint(qn)));
        qn += __uint_as_float(lane_xor<2>(__float_as_uint(qn)));
        qn += __uint_as_float(lane_xor<4>(__float_as_uint(qn)));
        const float inv = 1.f / sqrtf(ss / (float)d_v + A.eps);
        const float mqn = qn * inv / (float)d_v;   // <q, n> / d_v
        auto out = [&](int col, f32x4 x, f32x4 g, f32x4 gmk, f32x4 dy) {
            f32x4 dov, dgv, tg;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float n = x[e] * inv, sg = sigmoid(g[e]), si = g[e] * sg;
                dov[e] = inv * __builtin_fmaf(-n, mqn, dy[e] * gmk[e] * si);
                dgv[e] = dy[e] * gmk[e] * n * sg * __builtin_fmaf(g[e], 1.f - sg, 1.f);
                tg[e] = dy[e] * n * si;
            }
            if (live) {
                *reinterpret_cast<f32x4 *>(A.dout + base + col) = dov;
                *reinterpret_cast<f32x4 *>(A.dg + base + col) = dgv;
                f32x4 *acc = reinterpret_cast<f32x4 *>(myslot + col);
                *acc = *acc + tg;
            }
        };
        if constexpr (NC > 0) {
#pragma unroll
            for (int k = 0; k < NC; ++k) out((gl + 8 * k) * 4, xv[k], gv[k], gm[k], dyv[k]);
        } else {
            for (int k = 0; k < nc; ++k) {
                const int col = (gl + 8 * k) * 4;
                out(col, *reinterpret_cast<const f32x4 *>(A.o + base + col), load4<BF16>(A.g, base + col),
                    *reinterpret_cast<const f32x4 *>(A.gamma + col), *reinterpret_cast<const f32x4 *>(A.dy + base + col));
            }
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < d_v; c += blockDim.x) {
        float acc = 0.f;
        for (int r = 0; r < 32; ++r) acc += slot[r * d_v + c];
        A.part[(int64_t)blockIdx.x * d_v + c] = acc;
    }
}

// one workgroup per feature: dgamma[c] = sum of the workgroups' partial rows
// (thread l takes parts l, l + 256, ... in order, then a fixed tree)
__global__ void __launch_bounds__(256) sdm_out_norm_gate_bwd_reduce_kernel(NormBwdArgs A, int nparts)
{
    __shared__ float red[256];
    const int c = blockIdx.x;
    float s = 0.f;
    for (int p = threadIdx.x; p < nparts; p += blockDim.x) s += A.part[(int64_t)p * A.d_v + c];
    s = block_sum256(s, red);
    if (threadIdx.x == 0) A.dgamma[c] = s;
}

hipError_t launch_out_norm_gate_backward(const NormBwdArgs &A, bool bf16, hipStream_t stream)
{
    if (A.rows == 0) return hipSuccess;
    const int nblk = norm_bwd_blocks(A.rows);
    const size_t smem = sizeof(float) * 32 * (size_t)A.d_v;
    const int nc = A.d_v / 32;
    const void *fn;
#define SDM_NBWD_FN(B)                                                                          \
    (nc == 1 ? (const void *)sdm_out_norm_gate_bwd_kernel<B, 1>                                 \
     : nc == 2 ? (const void *)sdm_out_norm_gate_bwd_kernel<B, 2>                               \
     : nc == 4 ? (const void *)sdm_out_norm_gate_bwd_kernel<B, 4>                               \
               : (const void *)sdm_out_norm_gate_bwd_kernel<B, 0>)
    fn = bf16 ? SDM_NBWD_FN(true) : SDM_NBWD_FN(false);
#undef SDM_NBWD_FN
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)nblk), block(256);
#define SDM_NBWD_LAUNCH(B, N) hipLaunchKernelGGL((sdm_out_norm_gate_bwd_kernel<B, N>), grid, block, smem, stream, A)
    if (bf16) {
        if (nc == 1) SDM_NBWD_LAUNCH(true, 1);
        else if (nc == 2) SDM_NBWD_LAUNCH(true, 2);
        else if (nc == 4) SDM_NBWD_LAUNCH(true, 4);
        else SDM_NBWD_LAUNCH(true, 0);
    } else {
        if (nc == 1) SDM_NBWD_LAUNCH(false, 1);
        else if (nc == 2) SDM_NBWD_LAUNCH(false, 2);
        else if (nc == 4) SDM_NBWD_LAUNCH(false, 4);
        else SDM_NBWD_LAUNCH(false, 0);
    }
#undef SDM_NBWD_LAUNCH
    hipLaunchKernelGGL(sdm_out_norm_gate_bwd_reduce_kernel, dim3((unsigned)A.d_v), dim3(256), 0, stream, A, nblk);
    return hipGetLastError();
}

}  // namespace sdm
