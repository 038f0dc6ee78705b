// sdm_decode.hip -- one new token for each of B sequences: PKM addressing and
// one step of the sparse gated delta rule fused in a single launch.
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 steps 1-3 for a single token.
//
// One workgroup (12 waves) per (head h, tile of TS consecutive sequences):
// the sequences of a tile share the head's codebooks, so the tile reads them
// once (the 16-row MFMA tile has TS real rows).
//   A. the 4*TS half-score vectors (write/read x half 0/1 x sequence) on bf16
//      MFMA, with the tile code of the prefill addressing (every score is
//      bit-identical to a prefill of the same token);
//   B. one wave per (list, sequence) selects the top-k';
//   C. one wave per (kind, sequence) merges and softmaxes; the read rows that
//      are also written by the token are matched to their write positions;
//   D. the write and the read in the lane layout of the prefill scan (lane
//      (i, j) of a wave: unit i = (sequence, 4-column chunk), write row j and
//      read row j), with the same arithmetic, so a decode step reproduces the
//      prefill scan of the same token bit for bit.  Write and read rows are
//      gathered together; a read row the token also writes takes the new
//      value from the lane that computed it.
#include "kernels.h"
#include "pkm_address.h"
#include "scan_lanes.h"

namespace sdm {

// 12 waves: at 16 the 128-register limit per lane made the kernel spill
// inside the scoring loop (scratch reloads that drained the loads in flight)
constexpr int kDecWaves = 12;

struct DecodeLds {
    // byte offsets into dynamic LDS
    size_t S, L, scratch, stair, lidx, lwt, mpos, lbit, total;
};

__host__ __device__ inline DecodeLds decode_lds_layout(int n_sub, int kp, int ts)
{
    DecodeLds o;
    o.S = 0;                                                          // u32 [4][ts][n_sub]
    o.L = o.S + sizeof(uint32_t) * 4 * (size_t)ts * n_sub;            // HalfEntry [4][ts][kp]
    o.scratch = o.L + sizeof(HalfEntry) * 4 * (size_t)ts * kp;        // u64 [16][64]
    o.stair = o.scratch + sizeof(uint64_t) * kDecWaves * kWave;       // u16 [2][kMaxStair]
    o.lidx = o.stair + sizeof(uint16_t) * 2 * kMaxStair;              // int32 [2][ts][64]
    o.lwt = o.lidx + sizeof(int32_t) * 2 * (size_t)ts * kWave;        // float [2][ts][64]
    o.mpos = o.lwt + sizeof(float) * 2 * (size_t)ts * kWave;          // int32 [ts][64]
    o.lbit = o.mpos + sizeof(int32_t) * (size_t)ts * kWave;           // int32 [2][ts][64] (copy-on-write)
    o.total = o.lbit + sizeof(int32_t) * 2 * (size_t)ts * kWave;
    return o;
}

// 16-byte lane exchange within the wave (ds_bpermute: all lanes take part)
__device__ __forceinline__ f32x4 lane_fetch(f32x4 x, int src)
{
    const int a = src << 2;
    return (f32x4){__int_as_float(__builtin_amdgcn_ds_bpermute(a, __float_as_int(x.x))),
                   __int_as_float(__builtin_amdgcn_ds_bpermute(a, __float_as_int(x.y))),
                   __int_as_float(__builtin_amdgcn_ds_bpermute(a, __float_as_int(x.z))),
                   __int_as_float(__builtin_amdgcn_ds_bpermute(a, __float_as_int(x.w)))};
}

// Half scores of the tile for both halves of NKIND kinds (keys, then
// queries) against one codebook, every codebook and input load of this wave
// issued before the first MFMA: the decode step is a chain of dependent
// phases, so each phase should cost one memory round trip, and when both
// kinds use the same codebook each fragment is loaded once for both.  Same
// MFMA sequence per score as score_half_tile (k-steps in order), so the
// scores are bit-identical to the prefill's.  For d_k <= 128 (at most two
// k-steps); larger keys take score_half_tile.
//   x[kind]: the tile's first input row of that kind; S[kind]: its two
//   half-score lists ([c][srows][n_sub]).
template <int NKIND, int NB, int NK>
__device__ __forceinline__ void score_batched(const uint16_t *const (&x)[NKIND], int64_t row_stride, int nrows,
                                              int srows, const uint16_t *C, int half, int n_sub,
                                              uint32_t *const (&S)[NKIND])
{
    static_assert(NK == 1 || NK == 2, "one or two k-steps (d_k = 64 * NK)");
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
    const int r = lane & 15, kg = lane >> 4;
    // the input fragments are the same for every sub-key tile: loaded once,
    // by the lanes of live rows only (the others hold zeros)
    const bf16x8 zero = (bf16x8){};
    bf16x8 av[NKIND][2][NK];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
            for (int q = 0; q < NKIND; ++q) av[q][c][kk] = zero;
    if (r < nrows) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
#pragma unroll
                for (int q = 0; q < NKIND; ++q)
                    av[q][c][kk] =
                        *reinterpret_cast<const bf16x8 *>(x[q] + (int64_t)r * row_stride + c * half + kk * 32 + kg * 8);
    }
    // codebook fragments as in score_half_tile: contiguous loads, then a
    // lane exchange (codebook_tile_load / codebook_tile_frag); sub-keys past
    // n_sub load a valid neighbour and are zeroed
    for (int st0 = wave * NB; st0 * 16 < n_sub; st0 += nwaves * NB) {
        i32x4 raw[2][NB][NK];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
#pragma unroll
                for (int t = 0; t < NB; ++t)
                    raw[c][t][kk] = codebook_tile_load<false>(C + (int64_t)c * n_sub * half + kk * 32, half, n_sub, st0 + t);
        bf16x8 bv[2][NB][NK];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
#pragma unroll
                for (int t = 0; t < NB; ++t) bv[c][t][kk] = codebook_tile_frag(raw[c][t][kk]);
#pragma unroll
        for (int q = 0; q < NKIND; ++q) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int t = 0; t < NB; ++t) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q][c][kk], bv[c][t][kk], acc, 0, 0, 0);
                    const int u = (st0 + t) * 16 + r;
                    if (u < n_sub) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = 4 * kg + e;
                            if (row < srows) S[q][((size_t)c * srows + row) * n_sub + u] = score_bits(acc[e]);
                        }
                    }
                }
            }
        }
    }
}

// COW: the state is copy-on-write over M0 (A.touched): the merge waves look
// up the bit of each selected slot (in LDS for phase D), each gathered row
// is then loaded from M where the sequence has written it and from M0
// elsewhere, and the rows the step writes are marked once every bit has been
// read (after the barrier before phase D).
template <int Q, bool BF16, bool COW>
__global__ void __launch_bounds__(64 * kDecWaves) sdm_decode_kernel(DecodeArgs A, int TS)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int ntile = (A.B + TS - 1) / TS;
    const int h = blockIdx.x / ntile, b0 = (blockIdx.x - h * ntile) * TS;
    const int nb = min(TS, A.B - b0);            // live sequences of the tile
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int lane = lane_id();
    const int n_sub = A.n_sub, half = A.d_k / 2, kp = A.k_prime;
    const size_t esz = BF16 ? 2 : 4;

    const DecodeLds lay = decode_lds_layout(n_sub, kp, TS);
    uint32_t *S = reinterpret_cast<uint32_t *>(smem + lay.S);              // [list][row][n_sub]
    HalfEntry *L = reinterpret_cast<HalfEntry *>(smem + lay.L);         // [list][row][kp]
    uint64_t *wscr = reinterpret_cast<uint64_t *>(smem + lay.scratch) + wave * kWave;
    uint16_t *stair = reinterpret_cast<uint16_t *>(smem + lay.stair);   // [kind][kMaxStair]
    int32_t *lidx = reinterpret_cast<int32_t *>(smem + lay.lidx);       // [kind][row][64]
    float *lwt = reinterpret_cast<float *>(smem + lay.lwt);             // [kind][row][64]
    int32_t *mpos = reinterpret_cast<int32_t *>(smem + lay.mpos);       // [row][64]
    int32_t *lbit = reinterpret_cast<int32_t *>(smem + lay.lbit);       // [kind][row][64]
    const size_t wpb = ((size_t)A.N + 31) / 32;   // bitmap words per (b, h)

    // A. scores: list l = kind * 2 + c; row r of the tile = sequence b0 + r
    // (rows past the live ones are scored as zero vectors)
    {
        const size_t xoff = ((size_t)b0 * A.H + h) * A.d_k * esz, coff = (size_t)h * 2 * n_sub * half * esz;
        const unsigned char *xk = static_cast<const unsigned char *>(A.k) + xoff;
        const unsigned char *xq = static_cast<const unsigned char *>(A.q) + xoff;
        const unsigned char *Cw = static_cast<const unsigned char *>(A.C_w) + coff;
        const unsigned char *Cr = static_cast<const unsigned char *>(A.C_r) + coff;
        const int64_t rs = (int64_t)A.H * A.d_k;
        if (BF16 && (half == 32 || half == 64) && A.C_w == A.C_r) {
            const uint16_t *const xs[2] = {reinterpret_cast<const uint16_t *>(xk), reinterpret_cast<const uint16_t *>(xq)};
            uint32_t *const Ss[2] = {S, S + (size_t)2 * TS * n_sub};
            if (half == 64)
                score_batched<2, 2, 2>(xs, rs, nb, TS, reinterpret_cast<const uint16_t *>(Cw), half, n_sub, Ss);
            else
                score_batched<2, 2, 1>(xs, rs, nb, TS, reinterpret_cast<const uint16_t *>(Cw), half, n_sub, Ss);
        } else if (BF16 && (half == 32 || half == 64)) {
            for (int kind = 0; kind < 2; ++kind) {
                const uint16_t *const xs[1] = {reinterpret_cast<const uint16_t *>(kind ? xq : xk)};
                uint32_t *const Ss[1] = {S + (size_t)kind * 2 * TS * n_sub};
                const uint16_t *Ck = reinterpret_cast<const uint16_t *>(kind ? Cr : Cw);
                if (half == 64)
                    score_batched<1, 4, 2>(xs, rs, nb, TS, Ck, half, n_sub, Ss);
                else
                    score_batched<1, 4, 1>(xs, rs, nb, TS, Ck, half, n_sub, Ss);
            }
        } else {
            for (int l = 0; l < 4; ++l) {
                const int kind = l >> 1, c = l & 1;
                score_half_tile<BF16, 4>(kind ? xq : xk, rs, nb, TS, (kind ? Cr : Cw) + (size_t)c * n_sub * half * esz,
                                         c, half, n_sub, S + (size_t)l * TS * n_sub);
            }
        }
    }
    load_staircase(A.stair[0], stair);
    load_staircase(A.stair[1], stair + kMaxStair);
    __syncthreads();
    // B. per-half top-k': wave w takes (list, row) pairs w, w + 16, ...
    for (int lr = wave; lr < 4 * TS; lr += kDecWaves) {
        const int l = lr / TS, r = lr - l * TS;
        const int rows[1] = {r};
        uint64_t key[1];
        half_topk<1>(S + (size_t)l * TS * n_sub, rows, n_sub, kp, wscr, key);
        if (lane < kp) {
            HalfEntry e;
            e.score = __float_as_uint(key_score(key[0]));
            e.index = key_index(key[0]);
            L[((size_t)l * TS + r) * kp + lane] = e;
        }
    }
    __syncthreads();
    // C. merge + softmax: wave w takes (kind, row) pairs w, w + 16, ...
    for (int kr = wave; kr < 2 * TS; kr += kDecWaves) {
        const int kind = kr / TS, r = kr - kind * TS;
        const int n = kind ? (int)A.R : (int)A.W;
        const HalfEntry *const L0[1] = {L + ((size_t)(kind * 2) * TS + r) * kp};
        const HalfEntry *const L1[1] = {L + ((size_t)(kind * 2 + 1) * TS + r) * kp};
        int slot[1];
        float wt[1];
        merge_softmax<1>(L0, L1, kp, n_sub, n, stair + kind * kMaxStair, A.stair[kind].count, wscr, slot, wt);
        lidx[(kind * TS + r) * kWave + lane] = lane < n ? slot[0] : -1;
        lwt[(kind * TS + r) * kWave + lane] = lane < n ? wt[0] : 0.f;
        if constexpr (COW) {
            // whether the sequence has written the slot before this step (a
            // valid word for idle lanes and rows past the live ones)
            const int rr = r < nb ? r : 0;
            const uint32_t s = (uint32_t)(lane < n ? slot[0] : 0);
            const uint32_t word = A.touched[((size_t)(b0 + rr) * A.H + h) * wpb + (s >> 5)];
            lbit[(kind * TS + r) * kWave + lane] = (int32_t)((word >> (s & 31)) & 1u);
        }
        int32_t *out = kind ? A.ridx_out : A.widx_out;
        if (out && r < nb && lane < n) out[((size_t)(b0 + r) * A.H + h) * n + lane] = slot[0];
    }
    __syncthreads();
    // D. the write and the read
    constexpr int K = kWave / Q;
    constexpr uint32_t kOOB = 0x80000000u;
    constexpr uint32_t vbytes = BF16 ? 8u : 16u;   // one 4-column chunk of v
    const int i = lane / Q, j = lane % Q;
    const uint32_t d_v = (uint32_t)A.d_v;
    const int nchunk = A.d_v / 4;
    const int npr = (nchunk + K - 1) / K;           // passes per row (K chunks each)
    const int npass = nb * npr;
    // PB passes of a wave at a time, all their loads issued first; one row
    // (sequence) per pass, so the buffer resources are uniform
    constexpr int PB = 4;
    // The update's loads of one round of PB passes per wave.  The first
    // round is issued before the matching of read to write positions below,
    // so that its latency overlaps that phase and its barrier; a read row
    // the token also writes is loaded all the same (its value is then taken
    // from the lane that computes the new row, not from memory).
    f32x4 xw[PB], xr[PB], v4[PB];
    auto load_round = [&](int p0) {
#pragma unroll
        for (int t = 0; t < PB; ++t) {
            // passes past the last are neither loaded nor used (uniform)
            if (p0 + t * kDecWaves >= npass) break;
            const int pass = p0 + t * kDecWaves;
            const int r = pass / npr;
            const int chunk = (pass - r * npr) * K + i;
            const bool live = chunk < nchunk;
            const size_t bh = (size_t)(b0 + r) * A.H + h;
            const __amdgpu_buffer_rsrc_t Mrs =
                make_rsrc(A.M + bh * A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
            const uint32_t col4 = (uint32_t)chunk * 16u;
            const int sw = lidx[r * kWave + j], sr = lidx[(TS + r) * kWave + j];
            const uint32_t offw = (live && j < A.W) ? (uint32_t)sw * d_v * 4u + col4 : kOOB;
            const uint32_t offr = (live && j < A.R) ? (uint32_t)sr * d_v * 4u + col4 : kOOB;
            if constexpr (COW) {
                // each row from M if the sequence has written it, else from M0
                // (the other load is out of range: no memory access, zeros)
                const __amdgpu_buffer_rsrc_t M0rs =
                    make_rsrc(A.M0 + (size_t)h * A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
                const bool bwt = lbit[r * kWave + j] != 0, brd = lbit[(TS + r) * kWave + j] != 0;
                const f32x4 wm = __builtin_amdgcn_raw_buffer_load_b128(Mrs, bwt ? offw : kOOB, 0, 0);
                const f32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(M0rs, bwt ? kOOB : offw, 0, 0);
                const f32x4 rm = __builtin_amdgcn_raw_buffer_load_b128(Mrs, brd ? offr : kOOB, 0, 0);
                const f32x4 r0 = __builtin_amdgcn_raw_buffer_load_b128(M0rs, brd ? kOOB : offr, 0, 0);
                xw[t] = bwt ? wm : w0;
                xr[t] = brd ? rm : r0;
            } else {
                xw[t] = __builtin_amdgcn_raw_buffer_load_b128(Mrs, offw, 0, 0);
                xr[t] = __builtin_amdgcn_raw_buffer_load_b128(Mrs, offr, 0, 0);
            }
            const __amdgpu_buffer_rsrc_t Vrs =
                make_rsrc(static_cast<const unsigned char *>(A.v) + bh * d_v * esz, d_v * (uint32_t)esz);
            if constexpr (BF16) {
                const auto raw =
                    __builtin_amdgcn_raw_buffer_load_b64(Vrs, live ? (uint32_t)chunk * vbytes : kOOB, 0, 0);
                v4[t] = v_chunk((uint2){raw[0], raw[1]});
            } else {
                v4[t] = __builtin_amdgcn_raw_buffer_load_b128(Vrs, live ? (uint32_t)chunk * vbytes : kOOB, 0, 0);
            }
        }
    };
    load_round(wave);
    // read position j of row r is also written by the token at write
    // position mpos (the lists hold distinct slots), else -1
    for (int r = wave; r < TS; r += kDecWaves) {
        const int s = lidx[(TS + r) * kWave + lane];
        const i32x4 *wl = reinterpret_cast<const i32x4 *>(lidx + r * kWave);   // the write list, 4 at a time
        int m = -1;
        for (int jw = 0; jw < A.W; jw += 4) {
            const i32x4 w4 = wl[jw / 4];
#pragma unroll
            for (int e = 0; e < 4; ++e) m = (s >= 0 && w4[e] == s) ? jw + e : m;
        }
        mpos[r * kWave + lane] = m;
    }
    __syncthreads();

    if constexpr (COW) {
        // every bit this step reads was taken before the last barrier: mark
        // the rows the step writes
        for (int r = wave; r < nb; r += kDecWaves) {
            const int s = lidx[r * kWave + lane];
            if (lane < A.W && s >= 0 && s < A.N)
                atomicOr(A.touched + ((size_t)(b0 + r) * A.H + h) * wpb + ((uint32_t)s >> 5), 1u << (s & 31));
        }
    }
    for (int p0 = wave; p0 < npass; p0 += kDecWaves * PB) {
        if (p0 != wave) load_round(p0);
        int mm[PB];
#pragma unroll
        for (int t = 0; t < PB; ++t) {
            const int pass = min(p0 + t * kDecWaves, npass - 1);
            mm[t] = mpos[(pass / npr) * kWave + j];
        }
#pragma unroll
        for (int t = 0; t < PB; ++t) {
            if (p0 + t * kDecWaves >= npass) break;
            const int pass = p0 + t * kDecWaves;
            const int r = pass / npr;
            const int chunk = (pass - r * npr) * K + i;
            const bool live = chunk < nchunk;
            const size_t bh = (size_t)(b0 + r) * A.H + h;
            const __amdgpu_buffer_rsrc_t Mrs =
                make_rsrc(A.M + bh * A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
            const uint32_t col4 = (uint32_t)chunk * 16u;
            const int sw = lidx[r * kWave + j];
            const float wj = lwt[r * kWave + j], rj = lwt[(TS + r) * kWave + j];
            const uint32_t offw = (live && j < A.W) ? (uint32_t)sw * d_v * 4u + col4 : kOOB;
            const float at = A.a[bh], bt = A.b[bh];

            const f32x4 p = weighted_rows<Q>(wj, xw[t]);
            const f32x4 nm = written_row(xw[t], at, bt * wj, v4[t], p);
            __builtin_amdgcn_raw_buffer_store_b128(nm, Mrs, offw, 0, 0);
            const f32x4 own = lane_fetch(nm, i * Q + (mm[t] < 0 ? 0 : mm[t]));
            const f32x4 x2 = mm[t] >= 0 ? own : xr[t];
            const f32x4 o = weighted_rows<Q>(rj, x2);
            const __amdgpu_buffer_rsrc_t Ors = make_rsrc(A.o + bh * d_v, d_v * 4u);
            __builtin_amdgcn_raw_buffer_store_b128(o, Ors, (live && j == 0) ? col4 : kOOB, 0, 0);
        }
    }
}

// copy-on-write state: clear every sequence's bitmap (no row written yet)
__global__ void __launch_bounds__(256) sdm_cow_reset_kernel(CowArgs A)
{
    const int64_t n = A.B * A.H * ((A.N + 31) / 32);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        A.touched[i] = 0u;
}

// copy-on-write state made plain: the rows not yet written take M0's values
// (one 16-byte chunk per thread)
__global__ void __launch_bounds__(256) sdm_cow_materialize_kernel(CowArgs A)
{
    const int64_t cpr = A.d_v / 4;                      // chunks per row
    const int64_t n = A.B * A.H * A.N * cpr;
    const int64_t wpb = (A.N + 31) / 32;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / cpr, c = i - row * cpr;     // row of [B*H][N]
        const int64_t bh = row / A.N, slot = row - bh * A.N;
        const uint32_t word = A.touched[bh * wpb + (slot >> 5)];
        if (((word >> (slot & 31)) & 1u) == 0u) {
            const int64_t h = bh % A.H;
            const f32x4 x = *reinterpret_cast<const f32x4 *>(A.M0 + (h * A.N + slot) * A.d_v + c * 4);
            *reinterpret_cast<f32x4 *>(A.M + row * A.d_v + c * 4) = x;
        }
    }
}

// ... and then every row marked as written
__global__ void __launch_bounds__(256) sdm_cow_mark_all_kernel(CowArgs A)
{
    const int64_t n = A.B * A.H * ((A.N + 31) / 32);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        A.touched[i] = ~0u;
}

static unsigned grid_for(int64_t n)
{
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 1 ? 1 : b > (1 << 20) ? (1 << 20) : b);
}

hipError_t launch_cow_reset(const CowArgs &A, hipStream_t stream)
{
    const int64_t n = A.B * A.H * ((A.N + 31) / 32);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(sdm_cow_reset_kernel, dim3(grid_for(n)), dim3(256), 0, stream, A);
    return hipGetLastError();
}

hipError_t launch_cow_materialize(const CowArgs &A, hipStream_t stream)
{
    const int64_t n = A.B * A.H * A.N * (A.d_v / 4);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(sdm_cow_materialize_kernel, dim3(grid_for(n)), dim3(256), 0, stream, A);
    hipLaunchKernelGGL(sdm_cow_mark_all_kernel, dim3(grid_for(A.B * A.H * ((A.N + 31) / 32))), dim3(256), 0, stream,
                       A);
    return hipGetLastError();
}

// Sequences per workgroup: the most (up to 4) whose LDS fits and that still
// leave a workgroup for every CU.  A tile saves only codebook reads, which
// mostly hit in L2, while a chip that is not full loses whole CUs: one
// sequence per workgroup is fastest until B * H reaches the CU count
// (32 x 8 heads, n_sub = 1024: 24 us per step against 31 us at 4).
static int decode_tile_rows(int64_t B, int64_t H, int n_sub, int k_prime)
{
    constexpr int64_t kCUs = 256;
    for (int ts = 4; ts >= 1; ts /= 2)
        if (decode_lds_layout(n_sub, k_prime, ts).total <= 160 * 1024 && (ts == 1 || H * ((B + ts - 1) / ts) >= kCUs))
            return ts;
    return 0;
}

template <int Q>
static hipError_t launch_decode_q(const DecodeArgs &A, bool bf16, hipStream_t stream)
{
    const int ts = decode_tile_rows(A.B, A.H, A.n_sub, A.k_prime);
    if (ts == 0) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)A.H * ((A.B + ts - 1) / ts);
    const size_t smem = decode_lds_layout(A.n_sub, A.k_prime, ts).total;
    const bool cow = A.touched != nullptr;
    const void *fn = bf16 ? (cow ? (const void *)sdm_decode_kernel<Q, true, true> : (const void *)sdm_decode_kernel<Q, true, false>)
                          : (cow ? (const void *)sdm_decode_kernel<Q, false, true> : (const void *)sdm_decode_kernel<Q, false, false>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
#define SDM_DEC_LAUNCH(BF, CW) \
    hipLaunchKernelGGL((sdm_decode_kernel<Q, BF, CW>), dim3((unsigned)blocks), dim3(64 * kDecWaves), smem, stream, A, ts)
    if (bf16) {
        if (cow) SDM_DEC_LAUNCH(true, true);
        else SDM_DEC_LAUNCH(true, false);
    } else {
        if (cow) SDM_DEC_LAUNCH(false, true);
        else SDM_DEC_LAUNCH(false, false);
    }
#undef SDM_DEC_LAUNCH
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
