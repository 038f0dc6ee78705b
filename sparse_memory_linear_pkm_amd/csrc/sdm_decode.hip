// sdm_decode.hip -- one new token for each of B sequences: PKM addressing and
// one step of the sparse gated delta rule fused in a single launch.
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 steps 1-3 for a single token.
//
// One workgroup (4 waves) per (b, h):
//   A. the four half-score vectors (write/read x half 0/1) on bf16 MFMA, with
//      the same tile code as the prefill addressing (so the scores, and hence
//      the selected slots, are bit-identical to a prefill of the same token);
//   B. wave w selects the top-k' of list w;
//   C. waves 0 and 1 merge and softmax the write and read lists;
//   D. the write and the read in the lane layout of the prefill scan (lane
//      (i, j) of a wave: column chunk i of the pass, write row j and read row
//      j), with the same arithmetic, so a decode step reproduces the prefill
//      scan of the same token bit for bit.  The read rows are loaded after
//      the stores of the write (same wave, so they see the new rows).
#include "kernels.h"
#include "pkm_address.h"
#include "scan_lanes.h"

namespace sdm {

struct DecodeLds {
    // byte offsets into dynamic LDS
    size_t S, L, scratch, stair, fidx, fwt, total;
};

__host__ __device__ inline DecodeLds decode_lds_layout(int n_sub, int kp)
{
    DecodeLds o;
    o.S = 0;                                                      // float [4][n_sub]
    o.L = o.S + sizeof(float) * 4 * (size_t)n_sub;                // HalfEntry [4][kp]
    o.scratch = o.L + sizeof(HalfEntry) * 4 * (size_t)kp;         // u64 [4][64]
    o.stair = o.scratch + sizeof(uint64_t) * 4 * kWave;           // u16 [2][kMaxStair]
    o.fidx = o.stair + sizeof(uint16_t) * 2 * kMaxStair;          // int32 [2][64]
    o.fwt = o.fidx + sizeof(int32_t) * 2 * kWave;                 // float [2][64]
    o.total = o.fwt + sizeof(float) * 2 * kWave;
    return o;
}

template <int Q, bool BF16>
__global__ void __launch_bounds__(256) sdm_decode_kernel(DecodeArgs A)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int bh = blockIdx.x;
    const int bb = bh / A.H, h = bh - bb * A.H;
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const int n_sub = A.n_sub, half = A.d_k / 2, kp = A.k_prime;
    const size_t esz = BF16 ? 2 : 4;

    const DecodeLds lay = decode_lds_layout(n_sub, kp);
    uint32_t *S = reinterpret_cast<uint32_t *>(smem + lay.S);                 // [4][n_sub]
    HalfEntry *L = reinterpret_cast<HalfEntry *>(smem + lay.L);         // [4][kp]
    uint64_t *wscr = reinterpret_cast<uint64_t *>(smem + lay.scratch) + wave * kWave;
    uint16_t *stair = reinterpret_cast<uint16_t *>(smem + lay.stair);   // [2][kMaxStair]
    int32_t *fidx = reinterpret_cast<int32_t *>(smem + lay.fidx);       // [2][64]
    float *fwt = reinterpret_cast<float *>(smem + lay.fwt);             // [2][64]

    // A. scores (row 0 of a 16-row tile is this token; the others are zero)
#pragma unroll
    for (int kind = 0; kind < 2; ++kind) {
        const void *x = kind ? A.q : A.k;
        const void *C = kind ? A.C_r : A.C_w;
        const unsigned char *xb = static_cast<const unsigned char *>(x) + (size_t)bh * A.d_k * esz;
        const unsigned char *Cb = static_cast<const unsigned char *>(C) +
                                  (size_t)h * 2 * n_sub * half * esz;
        for (int c = 0; c < 2; ++c)
            score_half_tile<BF16>(xb, A.d_k, 1, 1, Cb + (size_t)c * n_sub * half * esz, c, half,
                                  n_sub, S + (kind * 2 + c) * n_sub);
    }
    load_staircase(A.stair[0], stair);
    load_staircase(A.stair[1], stair + kMaxStair);
    __syncthreads();
    // B. per-half top-k': wave w takes list w (kind w / 2, half w % 2)
    {
        const int rows[1] = {wave};
        uint64_t key[1];
        half_topk<1>(S, rows, n_sub, kp, wscr, key);
        if (lane < kp) {
            HalfEntry e;
            e.score = __float_as_uint(key_score(key[0]));
            e.index = key_index(key[0]);
            L[wave * kp + lane] = e;
        }
    }
    __syncthreads();
    // C. merge + softmax
    if (wave < 2) {
        const int kind = wave;
        const int n = kind ? (int)A.R : (int)A.W;
        const HalfEntry *const L0[1] = {L + (kind * 2) * kp};
        const HalfEntry *const L1[1] = {L + (kind * 2 + 1) * kp};
        int slot[1];
        float wt[1];
        merge_softmax<1>(L0, L1, kp, n_sub, n, stair + kind * kMaxStair, A.stair[kind].count, wscr, slot, wt);
        fidx[kind * kWave + lane] = slot[0];
        fwt[kind * kWave + lane] = wt[0];
        int32_t *out = kind ? A.ridx_out : A.widx_out;
        if (out && lane < n) out[(size_t)bh * n + lane] = slot[0];
    }
    __syncthreads();
    // D. the write and the read
    constexpr int K = kWave / Q;
    constexpr uint32_t kOOB = 0x80000000u;
    constexpr uint32_t vbytes = BF16 ? 8u : 16u;   // one 4-column chunk of v
    const int i = lane / Q, j = lane % Q;
    const uint32_t d_v = (uint32_t)A.d_v;
    const int nchunk = A.d_v / 4;
    const __amdgpu_buffer_rsrc_t Mrs =
        make_rsrc(A.M + (size_t)bh * A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
    const __amdgpu_buffer_rsrc_t Vrs =
        make_rsrc(static_cast<const unsigned char *>(A.v) + (size_t)bh * d_v * esz, d_v * (uint32_t)esz);
    const __amdgpu_buffer_rsrc_t Ors = make_rsrc(A.o + (size_t)bh * d_v, d_v * 4u);
    const float at = A.a[bh], bt = A.b[bh];
    const float wj = j < A.W ? fwt[j] : 0.f;
    const float rj = j < A.R ? fwt[kWave + j] : 0.f;
    for (int c0 = wave * K; c0 < nchunk; c0 += 4 * K) {
        const int chunk = c0 + i;
        const bool live = chunk < nchunk;
        const uint32_t col4 = (uint32_t)chunk * 16u;
        const uint32_t offw = (live && j < A.W) ? (uint32_t)fidx[j] * d_v * 4u + col4 : kOOB;
        const uint32_t offr = (live && j < A.R) ? (uint32_t)fidx[kWave + j] * d_v * 4u + col4 : kOOB;
        const f32x4 xw = __builtin_amdgcn_raw_buffer_load_b128(Mrs, offw, 0, 0);
        f32x4 v4;
        if constexpr (BF16) {
            const auto raw = __builtin_amdgcn_raw_buffer_load_b64(Vrs, live ? (uint32_t)chunk * vbytes : kOOB, 0, 0);
            v4 = v_chunk((uint2){raw[0], raw[1]});
        } else {
            v4 = __builtin_amdgcn_raw_buffer_load_b128(Vrs, live ? (uint32_t)chunk * vbytes : kOOB, 0, 0);
        }
        const f32x4 p = weighted_rows<Q>(wj, xw);
        const f32x4 nm = written_row(xw, at, bt * wj, v4, p);
        __builtin_amdgcn_raw_buffer_store_b128(nm, Mrs, offw, 0, 0);
        const f32x4 xr = __builtin_amdgcn_raw_buffer_load_b128(Mrs, offr, 0, 0);
        const f32x4 o = weighted_rows<Q>(rj, xr);
        __builtin_amdgcn_raw_buffer_store_b128(o, Ors, (live && j == 0) ? col4 : kOOB, 0, 0);
    }
}

size_t decode_smem_bytes(int n_sub, int k_prime) { return decode_lds_layout(n_sub, k_prime).total; }

template <int Q>
static hipError_t launch_decode_q(const DecodeArgs &A, bool bf16, hipStream_t stream)
{
    const int64_t blocks = (int64_t)A.B * A.H;
    const size_t smem = decode_smem_bytes(A.n_sub, A.k_prime);
    const void *fn = bf16 ? (const void *)sdm_decode_kernel<Q, true> : (const void *)sdm_decode_kernel<Q, false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    if (bf16)
        hipLaunchKernelGGL((sdm_decode_kernel<Q, true>), dim3((unsigned)blocks), dim3(256), smem, stream, A);
    else
        hipLaunchKernelGGL((sdm_decode_kernel<Q, false>), dim3((unsigned)blocks), dim3(256), smem, stream, A);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &A, bool bf16, hipStream_t stream)
{
    if ((int64_t)A.B * A.H == 0) return hipSuccess;
    int q = 4;   // the lane group of the prefill scan: power of two >= W, R
    while (q < A.W || q < A.R) q *= 2;
    switch (q) {
    case 4: return launch_decode_q<4>(A, bf16, stream);
    case 8: return launch_decode_q<8>(A, bf16, stream);
    case 16: return launch_decode_q<16>(A, bf16, stream);
    case 32: return launch_decode_q<32>(A, bf16, stream);
    case 64: return launch_decode_q<64>(A, bf16, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sdm
