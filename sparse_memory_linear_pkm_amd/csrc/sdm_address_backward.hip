// sdm_address_backward.hip -- gradients of the PKM addressing with the
// selected slots held fixed (the selection is piecewise constant).
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 2 (a slot's score is the sum of its two half scores, each a dot
// product with a sub-key) and Sec. 4 (softmax over the selected scores):
//     dsc_j = w_j (dw_j - sum_k w_k dw_k)
//     dx_c += dsc_j C[h][c][i_c(j)]          (i_0 = slot / n_sub, i_1 = slot % n_sub)
//     dC[h][c][i_c(j)] += dsc_j x_c          (summed over every token)
// for each kind (write: x = k against C_w, read: x = q against C_r).
//
// Three launches, every sum in a fixed order (deterministic):
//   1. one wave per (token-head, kind): the softmax backward (dsc, kept in
//      the workspace) and dx, summed over the list in order;
//   2. one wave per (kind, head, half, range of 8 sub-keys, part of the
//      tokens): the wave's lanes scan 64 list entries at a time for those
//      that select a sub-key of its range, and adds dsc * x for each, in
//      token and list order, into the 8 rows held in registers (each lane
//      owns columns); the part's rows go to the workspace;
//   3. the parts summed in order (and the two kinds together when the
//      caller passes one codebook-gradient buffer for both).
#include "device_common.h"
#include "kernels.h"

namespace sdm {

namespace {

constexpr int kAbRows = 8;                 // sub-key rows per wave, in registers
constexpr int64_t kAbWaves = 16384;        // target number of waves for the codebook gradient

template <bool BF16>
__device__ __forceinline__ float ld_in(const void *p, int64_t e)
{
    if constexpr (BF16)
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[e] << 16);
    else
        return static_cast<const float *>(p)[e];
}

}  // namespace

// token parts: enough waves to fill the chip, at least one token per part
int address_bwd_parts(int64_t BT, int64_t H, int n_sub)
{
    const int64_t units = 2 * H * 2 * ((n_sub + kAbRows - 1) / kAbRows);
    int64_t p = (kAbWaves + units - 1) / units;
    if (p > BT) p = BT;
    return (int)(p < 1 ? 1 : p);
}

size_t address_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int n_sub, int half)
{
    const int P = address_bwd_parts(B * T, H, n_sub);
    const size_t dsc = sizeof(float) * (size_t)(B * T * H * (W + R));
    const size_t parts = sizeof(float) * (size_t)(2 * H * 2 * P) * (size_t)n_sub * half;
    return ((dsc + 255) & ~(size_t)255) + parts;
}

// 1. softmax backward and dx: one wave per (row, kind); lanes over the list
// for dsc, over the features for dx
template <bool BF16, int NM>
__global__ void __launch_bounds__(256) sdm_address_bwd_dx_kernel(AddrBwdArgs A, float *dsc_ws)
{
    const int64_t rows = A.rows;
    const int64_t gw = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (gw >= 2 * rows) return;                 // whole waves
    const int kind = (int)(gw / rows);
    const int64_t r = gw - (int64_t)kind * rows;
    const int lane = lane_id();
    const int n = kind ? A.R : A.W;
    const int32_t *idx = (kind ? A.ridx : A.widx) + r * n;
    const float *wt = (kind ? A.rwt : A.wwt) + r * n;
    const float *dwt = (kind ? A.dr : A.dw) + r * n;
    const void *C = kind ? A.C_r : A.C_w;
    const int h = (int)(r % A.H);
    const int ns = A.n_sub, half = A.d_k / 2;
    const int jl = lane < n ? lane : 0;   // unconditional loads, masked after
    const float wl = wt[jl], gl = dwt[jl];
    const int32_t sl = idx[jl];
    const float w = lane < n ? wl : 0.f, g = lane < n ? gl : 0.f;
    const float mean = wave_sum_f32(w * g);
    const float ds = w * (g - mean);
    const int32_t s = lane < n ? sl : 0;
    if (lane < n) dsc_ws[(kind ? rows * A.W : 0) + r * n + lane] = ds;
    // NM = ceil(d_k / 64) features per lane
    float acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = 0.f;
    // eight list entries at a time, their codebook loads issued together;
    // entries past the list (dsc 0, slot 0) and slots outside the memory
    // (dsc forced to 0) add exactly nothing
    constexpr int kJ = 8;
    for (int j0 = 0; j0 < n; j0 += kJ) {
        float cv[kJ][NM], dj[kJ];
#pragma unroll
        for (int jj = 0; jj < kJ; ++jj) {
            const int j = min(j0 + jj, kWave - 1);
            int32_t sj = __builtin_amdgcn_readlane(s, j);
            dj[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ds), j));
            const bool ok = j0 + jj < n && sj >= 0 && sj < ns * ns;
            dj[jj] = ok ? dj[jj] : 0.f;
            sj = ok ? sj : 0;
            const int64_t row0 = ((int64_t)(h * 2 + 0) * ns + sj / ns) * half;
            const int64_t row1 = ((int64_t)(h * 2 + 1) * ns + sj % ns) * half;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int e = lane + kWave * m;
                const int ec = e < A.d_k ? e : 0;
                const float cl = ld_in<BF16>(C, ec < half ? row0 + ec : row1 + (ec - half));
                cv[jj][m] = e < A.d_k ? cl : 0.f;
            }
        }
#pragma unroll
        for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[m] = __builtin_fmaf(dj[jj], cv[jj][m], acc[m]);
    }
    float *dx = (kind ? A.dq : A.dk) + r * A.d_k;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int e = lane + kWave * m;
        if (e < A.d_k) dx[e] = acc[m];
    }
}

// 2. codebook-gradient parts: one wave per (kind, head, half, range of
// kAbRows sub-keys, token part); HM = ceil(half / 64) columns per lane
template <bool BF16, int HM>
__global__ void __launch_bounds__(256) sdm_address_bwd_dc_kernel(AddrBwdArgs A, const float *dsc_ws, float *parts,
                                                                 int P)
{
    const int half = A.d_k / 2, ns = A.n_sub, N = ns * ns;
    const int nrg = (ns + kAbRows - 1) / kAbRows;
    const int64_t units = (int64_t)2 * A.H * 2 * nrg * P;
    const int64_t unit = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (unit >= units) return;                  // whole waves
    int64_t id = unit;
    const int part = (int)(id % P); id /= P;
    const int rg = (int)(id % nrg); id /= nrg;
    const int c = (int)(id % 2); id /= 2;
    const int h = (int)(id % A.H); id /= A.H;
    const int kind = (int)id;
    const int lane = lane_id();
    const int u0 = rg * kAbRows;
    const int n = kind ? A.R : A.W;
    const int64_t bt_all = A.rows / A.H;
    const int64_t per = (bt_all + P - 1) / P;
    const int64_t bt0 = min(bt_all, (int64_t)part * per), bt1 = min(bt_all, bt0 + per);
    const int32_t *idx = kind ? A.ridx : A.widx;
    const float *dsc = dsc_ws + (kind ? A.rows * A.W : 0);
    const void *X = kind ? A.q : A.k;
    float acc[kAbRows][HM];
#pragma unroll
    for (int rr = 0; rr < kAbRows; ++rr)
#pragma unroll
        for (int m = 0; m < HM; ++m) acc[rr][m] = 0.f;
    const int64_t f1 = bt1 * n;
    for (int64_t f0 = bt0 * n; f0 < f1; f0 += kWave) {
        // 64 list entries, one per lane, in token-then-list order
        const int64_t f = f0 + lane < f1 ? f0 + lane : f0;
        const int64_t bt = f / n;
        const int j = (int)(f - bt * n);
        const int64_t r = bt * A.H + h;
        const int32_t sl = idx[r * n + j];
        const float dl = dsc[r * n + j];
        const bool ok = f0 + lane < f1 && sl >= 0 && sl < N;
        const int u = ok ? (c ? sl % ns : sl / ns) - u0 : -1;
        uint64_t hit = __builtin_amdgcn_ballot_w64(ok && u >= 0 && u < kAbRows);
        while (hit) {
            // up to four hits at a time: their input rows are loaded together
            int kk[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                kk[q] = hit ? __builtin_ctzll(hit) : -1;
                hit &= hit ? hit - 1 : 0;
            }
            float xv[4][HM], dq[4];
            int uq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = kk[q] < 0 ? kk[0] : kk[q];
                const int64_t rk = (int64_t)__builtin_amdgcn_readlane((int)(r & 0x7fffffff), k) |
                                   ((int64_t)__builtin_amdgcn_readlane((int)(r >> 31), k) << 31);
                dq[q] = kk[q] < 0 ? 0.f : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dl), k));
                uq[q] = __builtin_amdgcn_readlane(u, k);
#pragma unroll
                for (int m = 0; m < HM; ++m) {
                    const int e = lane + kWave * m;
                    const float xl = ld_in<BF16>(X, rk * A.d_k + c * half + (e < half ? e : 0));
                    xv[q][m] = e < half ? xl : 0.f;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int rr = 0; rr < kAbRows; ++rr)
#pragma unroll
                    for (int m = 0; m < HM; ++m) {
                        const float t = __builtin_fmaf(dq[q], xv[q][m], acc[rr][m]);
                        acc[rr][m] = uq[q] == rr ? t : acc[rr][m];
                    }
        }
    }
    float *out = parts + ((((size_t)kind * A.H + h) * 2 + c) * P + part) * (size_t)ns * half;
#pragma unroll
    for (int rr = 0; rr < kAbRows; ++rr)
#pragma unroll
        for (int m = 0; m < HM; ++m) {
            const int e = lane + kWave * m;
            if (u0 + rr < ns && e < half) out[(size_t)(u0 + rr) * half + e] = acc[rr][m];
        }
}

// 3. the parts summed in order, into dC_w and dC_r (or one buffer for both)
__global__ void __launch_bounds__(256) sdm_address_bwd_reduce_kernel(AddrBwdArgs A, const float *parts, int P)
{
    const int half = A.d_k / 2, ns = A.n_sub;
    const int64_t per_hc = (int64_t)ns * half;
    const int64_t per_kind = (int64_t)A.H * 2 * per_hc;   // elements of one codebook gradient
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool shared = A.dC_w == A.dC_r;
    if (i >= (shared ? 1 : 2) * per_kind) return;
    const int kind0 = shared ? 0 : (int)(i / per_kind);
    const int64_t e = shared ? i : i - kind0 * per_kind;
    const int64_t hc = e / per_hc, w = e - hc * per_hc;    // (h, c) and the element within
    float s = 0.f;
    for (int kind = kind0; kind <= (shared ? 1 : kind0); ++kind) {
        const float *p0 = parts + ((size_t)kind * A.H * 2 + hc) * P * per_hc + w;
        for (int p = 0; p < P; ++p) s += p0[(size_t)p * per_hc];
    }
    (kind0 ? A.dC_r : A.dC_w)[e] = s;
}

hipError_t launch_address_backward(const AddrBwdArgs &A, bool bf16, void *ws, hipStream_t stream)
{
    if (A.rows == 0) return hipSuccess;
    const int half = A.d_k / 2;
    const int P = address_bwd_parts(A.rows / A.H, A.H, A.n_sub);
    float *dsc = static_cast<float *>(ws);
    const size_t dsc_bytes = sizeof(float) * (size_t)(A.rows * (A.W + A.R));
    float *parts = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) + ((dsc_bytes + 255) & ~(size_t)255));
    const int64_t b1 = (2 * A.rows + 3) / 4;
    const int64_t units = 2 * (int64_t)A.H * 2 * ((A.n_sub + kAbRows - 1) / kAbRows) * P;
    const int64_t b2 = (units + 3) / 4;
    const int64_t per_kind = (int64_t)A.H * 2 * A.n_sub * half;
    const int64_t b3 = ((A.dC_w == A.dC_r ? 1 : 2) * per_kind + 255) / 256;
    const int nm = (A.d_k + kWave - 1) / kWave, hm = (half + kWave - 1) / kWave;
#define SDM_AB_DX(BF, M)                                                                                      \
    hipLaunchKernelGGL((sdm_address_bwd_dx_kernel<BF, M>), dim3((unsigned)b1), dim3(256), 0, stream, A, dsc)
#define SDM_AB_DC(BF, M)                                                                                      \
    hipLaunchKernelGGL((sdm_address_bwd_dc_kernel<BF, M>), dim3((unsigned)b2), dim3(256), 0, stream, A, dsc, parts, P)
    if (bf16) {
        if (nm <= 1) SDM_AB_DX(true, 1);
        else if (nm <= 2) SDM_AB_DX(true, 2);
        else if (nm <= 4) SDM_AB_DX(true, 4);
        else SDM_AB_DX(true, 8);
        if (hm <= 1) SDM_AB_DC(true, 1);
        else if (hm <= 2) SDM_AB_DC(true, 2);
        else SDM_AB_DC(true, 4);
    } else {
        if (nm <= 1) SDM_AB_DX(false, 1);
        else if (nm <= 2) SDM_AB_DX(false, 2);
        else if (nm <= 4) SDM_AB_DX(false, 4);
        else SDM_AB_DX(false, 8);
        if (hm <= 1) SDM_AB_DC(false, 1);
        else if (hm <= 2) SDM_AB_DC(false, 2);
        else SDM_AB_DC(false, 4);
    }
#undef SDM_AB_DX
#undef SDM_AB_DC
    hipLaunchKernelGGL(sdm_address_bwd_reduce_kernel, dim3((unsigned)b3), dim3(256), 0, stream, A, parts, P);
    return hipGetLastError();
}

}  // namespace sdm
