// sdm_scan_pipe.hip -- software-pipelined prefill scan.
//
// The recurrence is the sparse gated delta rule of "Sparse Delta Memory:
// Scaling the State of Linear RNNs through Sparsity", Sec. 3.1 steps 2-3
// (Eq. 4): per token, gather the W write rows and R read rows of the
// (sequence, head) memory, p = sum w_j M[s_j], write
// M[s_j] = a M[s_j] + b w_j (v - a p), then o = sum r_j M[s'_j] after the write.
//
// One wave per (b, h, 32-column slice), tokens in order.  The latency of the
// random row gathers is hidden by issuing the gathers of token t+D right
// after the stores of token t, straight into an LDS ring of D token slots
// (buffer loads with the LDS destination bit, 1 KB = 8 row segments per
// instruction).  Their completion is awaited with s_waitcnt vmcnt(K), where K
// is the exact number of vector-memory instructions issued after them, known
// at compile time from the fixed instruction schedule of a token step.  A gather
// issued that early misses the writes of the D-1 tokens in between (and, for
// read rows, the token's own write); those rows are replaced from an LDS ring
// holding the rows written by the last D tokens, following exact per-position
// forwarding codes computed beforehand (scan_hazard.hip).  Same-wave stores
// are ordered before later loads of the same address, so every other gather
// sees the current value.
//
// Per-token metadata (slot lists, weights, v, gates, codes) is fetched in
// blocks of 16 tokens with 16-byte loads into registers and written to LDS one
// block later, so waiting for it never stalls the gather pipeline.
//
// Every vector-memory access in the token loop is unconditional: lanes or
// tokens that must not touch memory use an offset beyond the buffer range, so
// the hardware bounds check returns zeros for loads and drops stores.  The
// number of vector-memory instructions per step is therefore fixed, which is
// what makes the compile-time wait counts exact.
#include <type_traits>

#include "kernels.h"
#include "scan_step.h"

namespace sdm {

constexpr int kMB = 16;                    // tokens per metadata block
constexpr uint32_t kOOB = 0x80000000u;     // beyond every buffer range used here (all < 2 GiB)

// Fixed per-step vector-memory schedule of the token loop (program order):
//   s == 0 only: the metadata loads of block blk + 2        (NMETA)
//   wait for the gathers of this token
//   the W row stores of this token                           (WK)
//   (s & 7) == 7 only: one store of 8 tokens' outputs        (1)
//   the gathers of token t + D                               (G = WK + RK)
// The gathers of token t were issued at the end of step t - D, so the number
// of instructions issued after them when step s waits is fixed.
constexpr int pipe_step_ops(int j, int WK, int G, int NMETA)
{
    const int s = ((j % kMB) + kMB) % kMB;
    return (s == 0 ? NMETA : 0) + WK + ((s & 7) == 7 ? 1 : 0) + G;
}

// younger instructions at the wait of step s in a steady-state block
constexpr int pipe_wait_steady(int s, int D, int WK, int G, int NMETA)
{
    int k = (s == 0 ? NMETA : 0);
    for (int j = s - D + 1; j <= s - 1; ++j) k += pipe_step_ops(j, WK, G, NMETA);
    return k;
}

// the same in the first block, where the D prologue gathers precede step 0
// (only prologue gathers, no stores, stand in for the steps before 0)
constexpr int pipe_wait_first(int s, int D, int WK, int G, int NMETA)
{
    if (s >= D) return pipe_wait_steady(s, D, WK, G, NMETA);
    int k = (D - 1 - s) * G + (s == 0 ? NMETA : 0);
    for (int j = 0; j <= s - 1; ++j) k += pipe_step_ops(j, WK, G, NMETA);
    return k;
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 (compile-time indices).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Reads this lane's 16 bytes of G consecutive 1 KB rows of the gather ring
// and its v entry (VB bytes) in one asm block that also waits for them: the
// compiler would otherwise wait for every outstanding LDS-destination gather
// before such reads.  The caller has already waited (vmcnt) for the gathers
// of this slot.  Outputs are early-clobber: the reads of one block are in
// flight together, so no output may share a register with the addresses.
#define SDM_RD(i) "ds_read_b128 %" #i ", %[a] offset:" #i "*1024\n\t"
template <int G, class VT>
__device__ __forceinline__ void read_gathered(f32x4 (&x)[G], uint32_t addr, VT &v, uint32_t vaddr)
{
    static_assert(G == 2 || G == 4 || G == 8 || G == 16, "unsupported gather count");
    static_assert(sizeof(VT) == 8 || sizeof(VT) == 16, "v entry is 8 or 16 bytes");
#define SDM_RDV (sizeof(VT) == 8 ? "ds_read_b64 %[v], %[va]\n\ts_waitcnt lgkmcnt(0)" \
                                 : "ds_read_b128 %[v], %[va]\n\ts_waitcnt lgkmcnt(0)")
    if constexpr (G == 2) {
        if constexpr (sizeof(VT) == 8)
            asm volatile(SDM_RD(0) SDM_RD(1) "ds_read_b64 %[v], %[va]\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(x[0]), "=&v"(x[1]), [v] "=&v"(v) : [a] "v"(addr), [va] "v"(vaddr) : "memory");
        else
            asm volatile(SDM_RD(0) SDM_RD(1) "ds_read_b128 %[v], %[va]\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(x[0]), "=&v"(x[1]), [v] "=&v"(v) : [a] "v"(addr), [va] "v"(vaddr) : "memory");
    } else if constexpr (G == 4) {
        if constexpr (sizeof(VT) == 8)
            asm volatile(SDM_RD(0) SDM_RD(1) SDM_RD(2) SDM_RD(3) "ds_read_b64 %[v], %[va]\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), [v] "=&v"(v)
                         : [a] "v"(addr), [va] "v"(vaddr)
                         : "memory");
        else
            asm volatile(SDM_RD(0) SDM_RD(1) SDM_RD(2) SDM_RD(3) "ds_read_b128 %[v], %[va]\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), [v] "=&v"(v)
                         : [a] "v"(addr), [va] "v"(vaddr)
                         : "memory");
    } else if constexpr (G == 8) {
        if constexpr (sizeof(VT) == 8)
            asm volatile(SDM_RD(0) SDM_RD(1) SDM_RD(2) SDM_RD(3) SDM_RD(4) SDM_RD(5) SDM_RD(6) SDM_RD(7)
                         "ds_read_b64 %[v], %[va]\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
                           "=&v"(x[7]), [v] "=&v"(v)
                         : [a] "v"(addr), [va] "v"(vaddr)
                         : "memory");
        else
            asm volatile(SDM_RD(0) SDM_RD(1) SDM_RD(2) SDM_RD(3) SDM_RD(4) SDM_RD(5) SDM_RD(6) SDM_RD(7)
                         "ds_read_b128 %[v], %[va]\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
                           "=&v"(x[7]), [v] "=&v"(v)
                         : [a] "v"(addr), [va] "v"(vaddr)
                         : "memory");
    } else {
        f32x4(&lo)[8] = *reinterpret_cast<f32x4(*)[8]>(&x[0]);
        f32x4(&hi)[8] = *reinterpret_cast<f32x4(*)[8]>(&x[8]);
        VT dummy;
        read_gathered<8>(lo, addr, v, vaddr);
        read_gathered<8>(hi, addr + 8192u, dummy, vaddr);
    }
#undef SDM_RDV
}
#undef SDM_RD

// 32-bit LDS byte address of a __shared__ object (for inline-asm ds_* reads).
template <class T>
__device__ __forceinline__ uint32_t lds_addr(const T *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T *)p;
}

template <int K>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(K >= 0 && K <= 63, "vmcnt out of range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
}

__device__ __forceinline__ i32x4 bload4(__amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
}

__device__ __forceinline__ uint32_t bload1(__amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
}

template <int WK, int RK, bool BF16>
struct PipeLds {
    static constexpr int WM = 8 * WK, RM = 8 * RK, PM = WM + RM;
    int32_t widx[2][kMB][WM];
    float wwt[2][kMB][WM];
    int32_t ridx[2][kMB][RM];
    float rwt[2][kMB][RM];
    uint32_t codes[2][kMB][PM / 2];   // pairs of 16-bit forwarding codes
    // the slice's 32 values of v per token, in the lane's 4-column groups
    typename std::conditional<BF16, uint2, f32x4>::type v[2][kMB][8];
    float ab[2][kMB][2];
    uint32_t flag[2][kMB];
};

// Loads NC 16-byte chunks of one metadata block: chunk ci belongs to token
// ci / cpt and covers bytes (ci % cpt) * 16 of that token's record; token
// records are tstride bytes apart.  Chunks past the block read zeros.
template <int NC>
__device__ __forceinline__ void load_chunks(i32x4 (&r)[NC], __amdgpu_buffer_rsrc_t rs, uint32_t tstride,
                                            int cpt)
{
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int ci = lane + i * kWave;
        const int tok = ci / cpt, part = ci - tok * cpt;
        const uint32_t off = tok < kMB ? (uint32_t)tok * tstride + (uint32_t)part * 16u : kOOB;
        r[i] = bload4(rs, off);
    }
}

template <int NC>
__device__ __forceinline__ void store_chunks(const i32x4 (&r)[NC], unsigned char *lds, int lds_tok_bytes,
                                             int cpt)
{
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int ci = lane + i * kWave;
        const int tok = ci / cpt, part = ci - tok * cpt;
        if (tok < kMB) *reinterpret_cast<i32x4 *>(lds + tok * lds_tok_bytes + part * 16) = r[i];
    }
}

// Buffer resource over the records of tokens [t0, t0 + ntok) of one chain:
// the record of token t0 + i starts at base + i * tstride and is rec bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void *base, int64_t ntok, uint32_t tstride,
                                                             uint32_t rec)
{
    const uint32_t bytes = ntok > 0 ? (uint32_t)(ntok - 1) * tstride + rec : 0u;
    return make_rsrc(base, bytes);
}

template <int WK, int RK, int D, bool BF16>
__global__ void __launch_bounds__(64) sdm_scan_pipe_kernel(ScanArgs A, const uint16_t *__restrict__ codes,
                                                           const uint32_t *__restrict__ flags)
{
    // gfx950-only body; the host pass only needs the signature for the launch stub
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(kMB % D == 0, "D must divide the metadata block");
    constexpr int WM = 8 * WK, RM = 8 * RK, PM = WM + RM;
    constexpr int NCW = (kMB * WM / 4 + kWave - 1) / kWave;
    constexpr int NCR = (kMB * RM / 4 + kWave - 1) / kWave;
    constexpr int NCC = (kMB * PM / 8 + kWave - 1) / kWave;
    constexpr int VB = BF16 ? 64 : 128;  // bytes of the slice's v per token
    constexpr int NCV = (kMB * VB / 16 + kWave - 1) / kWave;
    constexpr int G = WK + RK;
    constexpr int NMETA = 2 * NCW + 2 * NCR + NCC + NCV + 3;
    __shared__ PipeLds<WK, RK, BF16> L;
    __shared__ f32x4 ring[D][WM][8];   // rows written by the last D tokens (this slice)
    __shared__ f32x4 gath[D][G][64];   // gathered rows of the D tokens in flight, lane order

    const int nslice = A.d_v / 32;
    const int unit = blockIdx.x;
    const int slice = unit % nslice;
    const int ch = unit / nslice;
    const int bb = ch / A.H, h = ch - bb * A.H;
    const int lane = lane_id();
    const int rsub = lane >> 3, c4 = lane & 7;
    const int col = slice * 32 + 4 * c4;
    const int W = A.W, R = A.R;     // W <= WM, R <= RM, multiples of 4, (W + R) % 8 == 0
    const int P = W + R;
    const int64_t T = A.T;
    const int64_t H = A.H;
    const int d_v = A.d_v;
    const __amdgpu_buffer_rsrc_t Mrs =
        make_rsrc(A.M + (size_t)ch * A.N * d_v, (uint32_t)((uint64_t)A.N * d_v * 4u));
    const int64_t row0 = (int64_t)bb * T * H + h;  // row of token t: row0 + t*H
    const uint32_t vesz = BF16 ? 2 : 4;

    i32x4 gw[NCW], gwt[NCW], gr[NCR], grt[NCR], gc[NCC], gv[NCV];
    uint32_t gab = 0, gfl = 0;
    const int64_t nblk = (T + kMB - 1) / kMB;

    // metadata block -> registers (all loads unconditional; past T they read zeros)
#define SDM_LOAD_BLOCK(blk_)                                                                              \
    do {                                                                                                  \
        const int64_t t0_ = (int64_t)(blk_) * kMB;                                                        \
        const int64_t nt_ = t0_ < T ? (T - t0_ < kMB ? T - t0_ : kMB) : 0;                                \
        const int64_t r0_ = row0 + t0_ * H;                                                               \
        load_chunks(gw, block_rsrc(A.widx + r0_ * W, nt_, (uint32_t)(H * W * 4), W * 4), H * W * 4, W / 4); \
        load_chunks(gwt, block_rsrc(A.wwt + r0_ * W, nt_, (uint32_t)(H * W * 4), W * 4), H * W * 4, W / 4); \
        load_chunks(gr, block_rsrc(A.ridx + r0_ * R, nt_, (uint32_t)(H * R * 4), R * 4), H * R * 4, R / 4); \
        load_chunks(grt, block_rsrc(A.rwt + r0_ * R, nt_, (uint32_t)(H * R * 4), R * 4), H * R * 4, R / 4); \
        load_chunks(gc, block_rsrc(codes + r0_ * P, nt_, (uint32_t)(H * P * 2), P * 2), H * P * 2, P / 8); \
        load_chunks(gv,                                                                                   \
                    block_rsrc(static_cast<const unsigned char *>(A.v) + (r0_ * d_v + slice * 32) * vesz,  \
                               nt_, (uint32_t)(H * d_v * vesz), VB),                                      \
                    (uint32_t)(H * d_v * vesz), VB / 16);                                                 \
        const uint32_t tofs_ = (uint32_t)((lane & 15) * H * 4);                                           \
        const uint32_t ga_ = bload1(block_rsrc(A.a + r0_, nt_, (uint32_t)(H * 4), 4), lane < 16 ? tofs_ : kOOB); \
        const uint32_t gb_ = bload1(block_rsrc(A.b + r0_, nt_, (uint32_t)(H * 4), 4),                     \
                                    (lane >= 16 && lane < 32) ? tofs_ : kOOB);                            \
        gab = lane < 16 ? ga_ : gb_;                                                                      \
        gfl = bload1(block_rsrc(flags + r0_, nt_, (uint32_t)(H * 4), 4), lane < 16 ? tofs_ : kOOB);       \
    } while (0)

#define SDM_STORE_BLOCK(buf_)                                                                             \
    do {                                                                                                  \
        store_chunks(gw, reinterpret_cast<unsigned char *>(&L.widx[buf_][0][0]), WM * 4, W / 4);          \
        store_chunks(gwt, reinterpret_cast<unsigned char *>(&L.wwt[buf_][0][0]), WM * 4, W / 4);          \
        store_chunks(gr, reinterpret_cast<unsigned char *>(&L.ridx[buf_][0][0]), RM * 4, R / 4);          \
        store_chunks(grt, reinterpret_cast<unsigned char *>(&L.rwt[buf_][0][0]), RM * 4, R / 4);          \
        store_chunks(gc, reinterpret_cast<unsigned char *>(&L.codes[buf_][0][0]), PM * 2, P / 8);         \
        store_chunks(gv, reinterpret_cast<unsigned char *>(&L.v[buf_][0][0]), VB, VB / 16);               \
        if (lane < 32) L.ab[buf_][lane & 15][lane >> 4] = __uint_as_float(gab);                           \
        if (lane < 16) L.flag[buf_][lane] = gfl;                                                          \
    } while (0)

    // write offsets of the D tokens in flight (needed again at store time)
    uint32_t offw[D][WK];

#define SDM_ISSUE(rs_, tn_)                                                                               \
    do {                                                                                                  \
        const int64_t tn_m = (tn_);                                                                         \
        const int buf_m = (int)((tn_m / kMB) & 1), sn_m = (int)(tn_m % kMB);                                      \
        const bool live_m = tn_m < T;                                                                         \
        _Pragma("unroll") for (int k_m = 0; k_m < WK; ++k_m) {                                                  \
            const int j_m = rsub + 8 * k_m;                                                                   \
            const uint32_t slot_m = (uint32_t)L.widx[buf_m][sn_m][j_m];                                              \
            offw[rs_][k_m] = (live_m && j_m < W) ? (slot_m * (uint32_t)d_v + (uint32_t)col) * 4u : kOOB;             \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                     \
                Mrs, (__attribute__((address_space(3))) void *)&gath[rs_][k_m][0], 16, offw[rs_][k_m], 0, 0, 0); \
        }                                                                                                 \
        _Pragma("unroll") for (int k_m = 0; k_m < RK; ++k_m) {                                                  \
            const int j_m = rsub + 8 * k_m;                                                                   \
            const uint32_t slot_m = (uint32_t)L.ridx[buf_m][sn_m][j_m];                                              \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                     \
                Mrs, (__attribute__((address_space(3))) void *)&gath[rs_][WK + k_m][0], 16,                 \
                (live_m && j_m < R) ? (slot_m * (uint32_t)d_v + (uint32_t)col) * 4u : kOOB, 0, 0, 0);              \
        }                                                                                                 \
    } while (0)

    SDM_LOAD_BLOCK(0);
    SDM_STORE_BLOCK(0);
    SDM_LOAD_BLOCK(1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < D; ++s) SDM_ISSUE(s, s);
    // One full drain before the loop (vmcnt(0), known to the compiler): the
    // loop is entered with nothing pending, so the compiler's own waits inside
    // the loop see only the steady-state schedule.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");

    f32x4 obuf = {0.f, 0.f, 0.f, 0.f};
    // One block of 16 tokens.  The first block is peeled off the loop so that
    // the loop is always entered with a steady-state schedule behind it.
    auto do_block = [&](int64_t blk, auto first_c) __attribute__((always_inline)) {
        constexpr bool first = decltype(first_c)::value;
        const int cb = (int)(blk & 1);
        SDM_STORE_BLOCK(cb ^ 1);   // block blk + 1 (loaded one block ago)
        SDM_LOAD_BLOCK(blk + 2);
        const int64_t t0 = blk * kMB;
        const int64_t ntb = T - t0 < kMB ? T - t0 : kMB;
        const __amdgpu_buffer_rsrc_t Ors =
            block_rsrc(A.o + (row0 + t0 * H) * d_v, ntb, (uint32_t)(H * d_v * 4), (uint32_t)(d_v * 4));
        static_for<0, kMB>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            const int64_t t = t0 + s;
            constexpr int rs = s % D;
            // ---- wait for this token's gathers (exact count, see pipe_step_ops) ----
            if constexpr (first)
                wait_vmcnt<pipe_wait_first(s, D, WK, G, NMETA)>();
            else
                wait_vmcnt<pipe_wait_steady(s, D, WK, G, NMETA)>();
            f32x4 gx[G];
            typename std::conditional<BF16, uint2, f32x4>::type vraw;
            read_gathered<G>(gx, lds_addr(&gath[rs][0][lane]), vraw, lds_addr(&L.v[cb][s][c4]));
            const bool hz = __builtin_amdgcn_readfirstlane(L.flag[cb][s]) != 0;
            // ---- write: prediction, update, scatter ----
            float wv[WK];
            f32x4 xw[WK];
#pragma unroll
            for (int k = 0; k < WK; ++k) {
                const int j = rsub + 8 * k;
                wv[k] = j < W ? L.wwt[cb][s][j] : 0.f;
                xw[k] = gx[k];
            }
            if (hz) {
#pragma unroll
                for (int k = 0; k < WK; ++k) {
                    const int j = rsub + 8 * k;
                    const uint32_t code = j < W ? (L.codes[cb][s][j >> 1] >> (16 * (j & 1))) & 0xFFFFu : 0xFFFFu;
                    if (code != 0xFFFFu) {
                        const int dl = (int)(code >> 6), jp = (int)(code & 63);
                        xw[k] = ring[(s - dl + kMB) % D][jp][c4];
                    }
                }
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < WK; ++k) acc = fma4(wv[k], xw[k], acc);
            const f32x4 p = rowgroup_sum(acc);
            f32x4 vv;
            if constexpr (BF16) {
                vv.x = __uint_as_float(vraw.x << 16);
                vv.y = __uint_as_float(vraw.x & 0xffff0000u);
                vv.z = __uint_as_float(vraw.y << 16);
                vv.w = __uint_as_float(vraw.y & 0xffff0000u);
            } else {
                vv = vraw;
            }
            const float at = L.ab[cb][s][0], bt = L.ab[cb][s][1];
            f32x4 u;
            u.x = __builtin_fmaf(-at, p.x, vv.x);
            u.y = __builtin_fmaf(-at, p.y, vv.y);
            u.z = __builtin_fmaf(-at, p.z, vv.z);
            u.w = __builtin_fmaf(-at, p.w, vv.w);
#pragma unroll
            for (int k = 0; k < WK; ++k) {
                const float bw = bt * wv[k];
                f32x4 nm;
                nm.x = __builtin_fmaf(at, xw[k].x, bw * u.x);
                nm.y = __builtin_fmaf(at, xw[k].y, bw * u.y);
                nm.z = __builtin_fmaf(at, xw[k].z, bw * u.z);
                nm.w = __builtin_fmaf(at, xw[k].w, bw * u.w);
                mstore(Mrs, offw[rs][k], nm);   // out-of-range offset for masked lanes
                ring[rs][rsub + 8 * k][c4] = nm;
            }
            // ---- read (after this token's write) ----
            f32x4 xr[RK];
            float rv[RK];
#pragma unroll
            for (int k = 0; k < RK; ++k) {
                const int j = rsub + 8 * k;
                rv[k] = j < R ? L.rwt[cb][s][j] : 0.f;
                xr[k] = gx[WK + k];
            }
            if (hz) {
#pragma unroll
                for (int k = 0; k < RK; ++k) {
                    const int j = rsub + 8 * k;
                    const int p = W + j;
                    const uint32_t code = j < R ? (L.codes[cb][s][p >> 1] >> (16 * (p & 1))) & 0xFFFFu : 0xFFFFu;
                    if (code != 0xFFFFu) {
                        const int dl = (int)(code >> 6), jp = (int)(code & 63);
                        xr[k] = ring[(s - dl + kMB) % D][jp][c4];
                    }
                }
            }
            f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < RK; ++k) oacc = fma4(rv[k], xr[k], oacc);
            const f32x4 o = rowgroup_sum(oacc);
            if (rsub == (s & 7)) obuf = o;
            if constexpr ((s & 7) == 7) {
                const int tl = s - 7 + rsub;  // token (within the block) held by this lane
                __builtin_amdgcn_raw_buffer_store_b128(
                    obuf, Ors, (uint32_t)((int64_t)tl * H * d_v + col) * 4u, 0, 0);
            }
            // ---- gathers of token t + D (after this token's stores and after
            // every LDS read of the slot they overwrite) ----
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            SDM_ISSUE(rs, t + D);
            asm volatile("" ::: "memory");
        });
    };
    do_block(0, std::true_type{});
    for (int64_t blk = 1; blk < nblk; ++blk) do_block(blk, std::false_type{});
#undef SDM_ISSUE
#undef SDM_STORE_BLOCK
#undef SDM_LOAD_BLOCK
#endif  // __HIP_DEVICE_COMPILE__
}

template <int WK, int RK, int D, bool BF16>
static hipError_t launch_pipe(const ScanArgs &A, const uint16_t *codes, const uint32_t *flags, hipStream_t st)
{
    const int64_t units = A.B * A.H * (A.d_v / 32);
    hipLaunchKernelGGL((sdm_scan_pipe_kernel<WK, RK, D, BF16>), dim3((unsigned)units), dim3(64), 0, st, A,
                       codes, flags);
    return hipGetLastError();
}

// Pipeline depth used for a list length (0: no pipelined kernel for it).
int scan_pipe_depth(int W, int R)
{
    if (W != R) return 0;
    switch (W) {
    case 4: return 16;
    case 8: return 8;
    case 16: return 8;
    case 32: return 4;
    case 64: return 2;
    default: return 0;
    }
}

hipError_t launch_scan_pipe(const ScanArgs &A, bool bf16, const uint16_t *codes, const uint32_t *flags,
                            hipStream_t st)
{
#define SDM_PIPE_CASE(WV, WKV, DV)                                                    \
    case WV:                                                                          \
        return bf16 ? launch_pipe<WKV, WKV, DV, true>(A, codes, flags, st)            \
                    : launch_pipe<WKV, WKV, DV, false>(A, codes, flags, st);
    switch (A.W) {
        SDM_PIPE_CASE(4, 1, 16)
        SDM_PIPE_CASE(8, 1, 8)
        SDM_PIPE_CASE(16, 2, 8)
        SDM_PIPE_CASE(32, 4, 4)
        SDM_PIPE_CASE(64, 8, 2)
    default: return hipErrorInvalidValue;
    }
#undef SDM_PIPE_CASE
}

}  // namespace sdm
