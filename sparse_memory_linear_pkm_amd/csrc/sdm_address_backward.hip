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
// Every sum has a fixed order (deterministic), and nothing uses floating-
// point atomics:
//   1. one wave per (token-head, kind): the softmax backward (dsc, kept in
//      the workspace) and dx, summed over the list in order;
//   2. the codebook gradient: the list entries of each (kind, head, half)
//      are put in order of the sub-key they select by a stable counting
//      sort (integer counts per chunk of entries, their prefix sums, then a
//      scatter that keeps token-then-list order within a sub-key), as
//      (row, dsc) pairs, entries of one token that select the same sub-key
//      combined into one;
//   3. each sub-key's sorted entries are cut into pieces of at most
//      kAbPiece (so that a sub-key most tokens select does not serialise
//      one wave); one wave per piece adds dsc * x for its entries in order
//      into registers (each lane owns columns), every entry read once; then
//      one wave per (head, half, sub-key) [and kind, unless one buffer takes
//      both kinds' sums] adds its pieces in order.
#include "device_common.h"
#include "kernels.h"

namespace sdm {

namespace {

constexpr int64_t kAbChunk = 4096;         // list entries per chunk of the counting sort
constexpr int64_t kAbDxRows = 8;           // token-head rows per wave of the dx pass
constexpr int kAbPiece = 2048;             // sorted entries per wave of the sums pass at most

template <bool BF16>
__device__ __forceinline__ float ld_in(const void *p, int64_t e)
{
    if constexpr (BF16)
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[e] << 16);
    else
        return static_cast<const float *>(p)[e];
}

// lanes whose key equals this lane's: one ballot per key bit
__device__ __forceinline__ uint64_t same_key(int key, int key_bits)
{
    uint64_t eq = ~0ull;
    for (int b = 0; b < key_bits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t ones = __builtin_amdgcn_ballot_w64(bit);
        eq &= bit ? ones : ~ones;
    }
    return eq;
}

// sum of v over the lanes of mask g, in lane order (each lane its own g)
__device__ __forceinline__ float sum_in_lane_order(float v, uint64_t g)
{
    float s = 0.f;
    for (int l = 0; l < kWave; ++l) {
        const float x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
        s += ((g >> l) & 1) ? x : 0.f;
    }
    return s;
}

}  // namespace

// Workspace layout (each piece starting on a 256-byte boundary):
//   dsc     [rows][W] then [rows][R] fp32 (kind 0 then kind 1)
//   cnt     per kind k, [H][2][nch_k][n_sub] int32: entries of each chunk
//           per sub-key, then (in place) their offset within the sub-key
//   start   [2][H][2][n_sub + 1] int32: where each sub-key's entries begin
//   sorted  per kind k, [H][2][B*T*n_k] (row, dsc) pairs
//   pstart  [2][H][2][n_sub + 1] int32: each sub-key's first piece
//   pmap    [2][H][2][maxp] int32: the sub-key of each piece
//   part    [2][H][2][maxp][d_k / 2] fp32: each piece's sums
// where n_0 = W, n_1 = R and nch_k = ceil(B*T*n_k / kAbChunk).
AddrBwdLayout address_bwd_layout(int64_t BT, int64_t H, int W, int R, int n_sub, int half)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    AddrBwdLayout L;
    L.half = half;
    L.nch[0] = (BT * W + kAbChunk - 1) / kAbChunk;
    L.nch[1] = (BT * R + kAbChunk - 1) / kAbChunk;
    const int64_t rows = BT * H;
    L.off_cnt = up(sizeof(float) * (size_t)(rows * (W + R)));
    L.cnt1 = (size_t)(H * 2 * L.nch[0] * n_sub);
    L.off_start = L.off_cnt + up(sizeof(int32_t) * (L.cnt1 + (size_t)(H * 2 * L.nch[1] * n_sub)));
    L.off_sorted = L.off_start + up(sizeof(int32_t) * (size_t)(2 * H * 2 * (n_sub + 1)));
    L.sorted1 = (size_t)(H * 2 * BT * W);
    const int64_t segs = 2 * H * 2;
    // pieces of at most kAbPiece entries per (kind, head, half): at most
    // entries / kAbPiece + n_sub (one partial piece per sub-key)
    L.maxp = (BT * (W > R ? W : R) + kAbPiece - 1) / kAbPiece + n_sub;
    L.off_pstart = L.off_sorted + up(sizeof(int2) * (L.sorted1 + (size_t)(H * 2 * BT * R)));
    L.off_pmap = L.off_pstart + up(sizeof(int32_t) * (size_t)(segs * (n_sub + 1)));
    L.off_part = L.off_pmap + up(sizeof(int32_t) * (size_t)(segs * L.maxp));
    L.bytes = L.off_part + up(sizeof(float) * (size_t)(segs * L.maxp) * (size_t)half);
    return L;
}

size_t address_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int n_sub, int half)
{
    return address_bwd_layout(B * T, H, W, R, n_sub, half).bytes;
}

// 1. softmax backward and dx: one wave per kAbDxRows consecutive rows of one
// kind (the next row's list loaded while the current one is processed);
// lanes over the list for dsc, over the features for dx.  Each lane first
// turns its entry's slot into the element offsets of its two sub-key rows
// (the divisions by n_sub once per entry, in parallel), so that the loop
// over entries only reads them back (readlane) and loads.
template <bool BF16, int NM, int KJ>
__global__ void __launch_bounds__(256) sdm_address_bwd_dx_kernel(AddrBwdArgs A, float *dsc_ws)
{
    const int64_t rows = A.rows;
    const int64_t wpk = (rows + kAbDxRows - 1) / kAbDxRows;   // waves per kind
    // the wave's index, uniform (so that the codebook's buffer resource is scalar)
    const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    if (gw >= 2 * wpk) return;                 // whole waves
    const int kind = (int)(gw / wpk);
    const int64_t r0 = (gw - (int64_t)kind * wpk) * kAbDxRows;
    const int64_t r1 = min(rows, r0 + kAbDxRows);
    const int lane = lane_id();
    const int n = kind ? A.R : A.W;
    const int32_t *idx = kind ? A.ridx : A.widx;
    const float *wt = kind ? A.rwt : A.wwt;
    const float *dwt = kind ? A.dr : A.dw;
    const void *C = kind ? A.C_r : A.C_w;
    const int ns = A.n_sub, half = A.d_k / 2;
    const int jl = lane < n ? lane : 0;   // unconditional loads, masked after
    // feature e of a lane: e < half reads half 0 at e, else half 1 at e - half
    int32_t fe[NM];
    bool h1[NM], live[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int e = lane + kWave * m;
        live[m] = e < A.d_k;
        h1[m] = live[m] ? e >= half : true;
        fe[m] = live[m] ? e : half;   // a valid element of half 1 for dead features
    }
    float wl = wt[r0 * n + jl], gl = dwt[r0 * n + jl];
    int32_t sl = idx[r0 * n + jl];
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t rn = r + 1 < r1 ? r + 1 : r;
        const float wn = wt[rn * n + jl], gn = dwt[rn * n + jl];
        const int32_t sn = idx[rn * n + jl];
        const int h = (int)(r % A.H);
        const float w = lane < n ? wl : 0.f, g = lane < n ? gl : 0.f;
        const float mean = wave_sum_f32(w * g);
        const float ds = w * (g - mean);
        if (lane < n) dsc_ws[(kind ? rows * A.W : 0) + r * n + lane] = ds;
        // entries past the list and slots outside the memory add exactly nothing
        const bool ok = lane < n && sl >= 0 && sl < ns * ns;
        const float dsl = ok ? ds : 0.f;
        const int32_t s = ok ? sl : 0;
        // byte offsets (in the head's codebook) of this entry's rows of half 0
        // and half 1, the latter less half a row so that feature e adds e
        constexpr int esz = BF16 ? 2 : 4;
        const int32_t off0 = (s / ns) * half * esz;
        const int32_t off1 = ((ns + s % ns) * half - half) * esz;
        const __amdgpu_buffer_rsrc_t Crs = make_rsrc(static_cast<const unsigned char *>(C) +
                                                         (int64_t)h * 2 * ns * half * esz,
                                                     (uint32_t)(2 * ns * half * esz));
        float acc[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = 0.f;
        // KJ list entries at a time, their codebook loads issued together
        constexpr int kJ = KJ;
        for (int j0 = 0; j0 < n; j0 += kJ) {
            float cv[kJ][NM], dj[kJ];
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj) {
                const int j = min(j0 + jj, kWave - 1);
                const int32_t o0 = __builtin_amdgcn_readlane(off0, j);
                const int32_t o1 = __builtin_amdgcn_readlane(off1, j);
                dj[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dsl), j));
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const uint32_t off = (uint32_t)((h1[m] ? o1 : o0) + fe[m] * esz);
                    if constexpr (BF16)
                        cv[jj][m] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(Crs, off, 0, 0) << 16);
                    else
                        cv[jj][m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(Crs, off, 0, 0));
                }
            }
#pragma unroll
            for (int jj = 0; jj < kJ; ++jj)
#pragma unroll
                for (int m = 0; m < NM; ++m) acc[m] = __builtin_fmaf(dj[jj], cv[jj][m], acc[m]);
        }
        float *dx = (kind ? A.dq : A.dk) + r * A.d_k;
#pragma unroll
        for (int m = 0; m < NM; ++m)
            if (live[m]) dx[lane + kWave * m] = acc[m];
        wl = wn;
        gl = gn;
        sl = sn;
    }
}

// 1, wide form (when a 16-byte piece of a codebook row, 8 bf16 or 4 fp32
// features, never straddles the two halves and d_k / 8 resp. d_k / 4 is a
// power of two): each lane loads 16 bytes of a codebook row per list entry
// instead of one element.  Lane (g, f) = (lane / NF, lane % NF) takes feature
// piece f of list entries g, g + EG, g + 2 EG, ... (EG = 64 / NF; KB of them
// at most), summed in that order; the EG partial sums of a piece are then
// added by a fixed butterfly (every lane of the piece ends with the same
// bits).  The entries' offsets and dsc come from the lanes holding them
// (ds_bpermute).
template <bool BF16, int NF, int KB>
__global__ void __launch_bounds__(256) sdm_address_bwd_dx_wide_kernel(AddrBwdArgs A, float *dsc_ws)
{
    constexpr int FPL = BF16 ? 8 : 4;     // features per 16-byte piece
    constexpr int EG = kWave / NF;        // entry groups
    constexpr int esz = BF16 ? 2 : 4;
    const int64_t rows = A.rows;
    const int64_t wpk = (rows + kAbDxRows - 1) / kAbDxRows;   // waves per kind
    const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    if (gw >= 2 * wpk) return;                 // whole waves
    const int kind = (int)(gw / wpk);
    const int64_t r0 = (gw - (int64_t)kind * wpk) * kAbDxRows;
    const int64_t r1 = min(rows, r0 + kAbDxRows);
    const int lane = lane_id();
    const int n = kind ? A.R : A.W;
    const int32_t *idx = kind ? A.ridx : A.widx;
    const float *wt = kind ? A.rwt : A.wwt;
    const float *dwt = kind ? A.dr : A.dw;
    const void *C = kind ? A.C_r : A.C_w;
    const int ns = A.n_sub, half = A.d_k / 2;
    const int g = lane / NF, f = lane % NF;
    const int e0 = f * FPL;                    // this lane's first feature
    const bool hi = e0 >= half;
    const uint32_t col = (uint32_t)(hi ? e0 - half : e0) * esz;
    const int jl = lane < n ? lane : 0;
    float wl = wt[r0 * n + jl], gl = dwt[r0 * n + jl];
    int32_t sl = idx[r0 * n + jl];
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t rn = r + 1 < r1 ? r + 1 : r;
        const float wn = wt[rn * n + jl], gn = dwt[rn * n + jl];
        const int32_t sn = idx[rn * n + jl];
        const int h = (int)(r % A.H);
        const float w = lane < n ? wl : 0.f, gg = lane < n ? gl : 0.f;
        const float mean = wave_sum_f32(w * gg);
        const float ds = w * (gg - mean);
        if (lane < n) dsc_ws[(kind ? rows * A.W : 0) + r * n + lane] = ds;
        // entries past the list and slots outside the memory add exactly nothing
        const bool ok = lane < n && sl >= 0 && sl < ns * ns;
        const float dsl = ok ? ds : 0.f;
        const int32_t s = ok ? sl : 0;
        // byte offsets (in the head's codebook) of this entry's rows of half 0 and half 1
        const int32_t off0 = (s / ns) * half * esz;
        const int32_t off1 = (ns + s % ns) * half * esz;
        const __amdgpu_buffer_rsrc_t Crs = make_rsrc(static_cast<const unsigned char *>(C) +
                                                         (int64_t)h * 2 * ns * half * esz,
                                                     (uint32_t)(2 * ns * half * esz));
        uint4 raw[KB];
        float dj[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int j = k * EG + g;
            const int src = j < n ? j : 0;
            const int o0 = __builtin_amdgcn_ds_bpermute(src * 4, off0);
            const int o1 = __builtin_amdgcn_ds_bpermute(src * 4, off1);
            const float d = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(dsl)));
            dj[k] = j < n ? d : 0.f;
            const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(Crs, (uint32_t)(hi ? o1 : o0) + col, 0, 0);
            raw[k] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
        }
        float acc[FPL];
#pragma unroll
        for (int e = 0; e < FPL; ++e) acc[e] = 0.f;
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
            for (int e = 0; e < FPL; ++e) {
                float c;
                if constexpr (BF16)
                    c = __uint_as_float((e & 1) ? (wd[e >> 1] & 0xFFFF0000u) : (wd[e >> 1] << 16));
                else
                    c = __uint_as_float(wd[e]);
                acc[e] = __builtin_fmaf(dj[k], c, acc[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < FPL; ++e) {
            if constexpr (NF <= 1) acc[e] += __uint_as_float(lane_xor<1>(__float_as_uint(acc[e])));
            if constexpr (NF <= 2) acc[e] += __uint_as_float(lane_xor<2>(__float_as_uint(acc[e])));
            if constexpr (NF <= 4) acc[e] += __uint_as_float(lane_xor<4>(__float_as_uint(acc[e])));
            if constexpr (NF <= 8) acc[e] += __uint_as_float(lane_xor<8>(__float_as_uint(acc[e])));
            if constexpr (NF <= 16) acc[e] += __uint_as_float(lane_xor<16>(__float_as_uint(acc[e])));
            if constexpr (NF <= 32) acc[e] += __uint_as_float(lane_xor<32>(__float_as_uint(acc[e])));
        }
        if (g == 0) {
            float *dx = (kind ? A.dq : A.dk) + r * A.d_k + e0;
#pragma unroll
            for (int e = 0; e < FPL; e += 4)
                *reinterpret_cast<f32x4 *>(dx + e) = (f32x4){acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
        }
        wl = wn;
        gl = gn;
        sl = sn;
    }
}

namespace {

// the pieces of the workspace for one launch
struct AbWs {
    float *dsc;
    int32_t *cnt, *start;
    int2 *sorted;
    int32_t *pstart, *pmap;   // [seg][n_sub + 1] first piece of each sub-key; [seg][maxp] sub-key of each piece
    float *part;              // [seg][maxp][half] each piece's sums
    int64_t nch[2];
    size_t cnt1, sorted1;
    int64_t maxp;
};

// which (kind, head, chunk) a workgroup of the count and scatter passes takes
__device__ __forceinline__ void chunk_unit(const AddrBwdArgs &A, const AbWs &S, int &kind, int &h, int64_t &ch)
{
    int64_t id = blockIdx.x;
    kind = id >= (int64_t)A.H * S.nch[0] ? 1 : 0;
    if (kind) id -= (int64_t)A.H * S.nch[0];
    h = (int)(id / S.nch[kind]);
    ch = id - (int64_t)h * S.nch[kind];
}

__device__ __forceinline__ int32_t *cnt_row(const AddrBwdArgs &A, const AbWs &S, int kind, int h, int c, int64_t ch)
{
    return S.cnt + (kind ? S.cnt1 : 0) + ((int64_t)(h * 2 + c) * S.nch[kind] + ch) * A.n_sub;
}

}  // namespace

// The sort's entries: within each group of 64 consecutive list entries (in
// token-then-list order), those of one token that select the same sub-key
// of a half are combined into one entry (their dsc summed in list order),
// placed where the first of them is.  lanes of the token of this lane:
__device__ __forceinline__ uint64_t same_row(int64_t bt, int64_t fb, int n)
{
    const int64_t lo = bt * n - fb, hi = lo + n;   // the token's entries, relative to the group
    const uint64_t upto = hi >= kWave ? ~0ull : ((1ull << hi) - 1ull);
    const uint64_t from = lo <= 0 ? ~0ull : ~((1ull << lo) - 1ull);
    return upto & from;
}

// 2a. entries per sub-key in each chunk of kAbChunk list entries (integer
// counts: the order of the LDS atomics does not matter); four waves, each
// taking every fourth group of 64 entries
__global__ void __launch_bounds__(256) sdm_address_bwd_count_kernel(AddrBwdArgs A, AbWs S, int key_bits)
{
    extern __shared__ int32_t hist[];   // [2][n_sub]
    int kind, h;
    int64_t ch;
    chunk_unit(A, S, kind, h, ch);
    const int ns = A.n_sub, n = kind ? A.R : A.W;
    const int32_t N = ns * ns;
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < 2 * ns; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const int64_t total = A.rows / A.H * n;
    const int64_t f0 = ch * kAbChunk, f1 = min(total, f0 + kAbChunk);
    const int32_t *idx = kind ? A.ridx : A.widx;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t fb = f0 + wv * kWave; fb < f1; fb += 4 * kWave) {
        const bool in = fb + lane < f1;
        const int64_t f = in ? fb + lane : fb;
        const int64_t bt = f / n;
        const int32_t sl = idx[(bt * A.H + h) * n + (f - bt * n)];
        const bool ok = in && sl >= 0 && sl < N;
        const uint64_t valid = __builtin_amdgcn_ballot_w64(ok) & same_row(bt, fb, n);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int key = ok ? (c ? sl % ns : sl / ns) : 0;
            const uint64_t grp = same_key(key, key_bits) & valid;
            if (ok && (grp & below) == 0) atomicAdd(&hist[c * ns + key], 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * ns; i += blockDim.x) cnt_row(A, S, kind, h, i / ns, ch)[i % ns] = hist[i];
}

// 2b. per (kind, head, half) and sub-key: the counts of the chunks turned in
// place into their exclusive prefix sums (the chunk's offset within the
// sub-key), and the sub-key's total; one thread per sub-key
__global__ void __launch_bounds__(256) sdm_address_bwd_chunk_prefix_kernel(AddrBwdArgs A, AbWs S)
{
    const int nbb = (A.n_sub + 255) / 256;      // workgroups per segment
    const int seg = blockIdx.x / nbb;           // (kind * H + h) * 2 + c
    const int kind = seg / (2 * A.H), h = (seg / 2) % A.H, c = seg % 2;
    const int u = (blockIdx.x - seg * nbb) * blockDim.x + threadIdx.x;
    if (u >= A.n_sub) return;
    int32_t *col = cnt_row(A, S, kind, h, c, 0) + u;
    const int64_t nch = S.nch[kind];
    int32_t run = 0;
    int64_t k = 0;
    for (; k + 8 <= nch; k += 8) {
        int32_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = col[(k + i) * A.n_sub];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            col[(k + i) * A.n_sub] = run;
            run += v[i];
        }
    }
    for (; k < nch; ++k) {
        const int32_t v = col[k * A.n_sub];
        col[k * A.n_sub] = run;
        run += v;
    }
    S.start[(int64_t)seg * (A.n_sub + 1) + u] = run;   // the total, until 2c
}

// 2c. per (kind, head, half): exclusive prefix over the sub-keys' totals, in
// place, and the grand total after them
__global__ void __launch_bounds__(256) sdm_address_bwd_key_prefix_kernel(AddrBwdArgs A, AbWs S)
{
    __shared__ int32_t part[256];
    int32_t *st = S.start + (int64_t)blockIdx.x * (A.n_sub + 1);
    const int ns = A.n_sub;
    const int per = (ns + 255) / 256;
    const int b0 = min(ns, (int)threadIdx.x * per), b1 = min(ns, b0 + per);
    int32_t sum = 0;
    for (int u = b0; u < b1; ++u) sum += st[u];
    part[threadIdx.x] = sum;
    __syncthreads();
    // inclusive scan of the 256 partial sums (Hillis-Steele)
    for (int d = 1; d < 256; d <<= 1) {
        const int32_t add = (int)threadIdx.x >= d ? part[threadIdx.x - d] : 0;
        __syncthreads();
        part[threadIdx.x] += add;
        __syncthreads();
    }
    int32_t run = part[threadIdx.x] - sum;
    const int32_t total = part[255];
    // the sub-keys' pieces of at most kAbPiece entries (empty sub-keys have none)
    int32_t np = 0;
    for (int u = b0; u < b1; ++u) np += (st[u] + kAbPiece - 1) / kAbPiece;
    __syncthreads();   // every thread has read its scan results before part is reused
    part[threadIdx.x] = np;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int32_t add = (int)threadIdx.x >= d ? part[threadIdx.x - d] : 0;
        __syncthreads();
        part[threadIdx.x] += add;
        __syncthreads();
    }
    int32_t prun = part[threadIdx.x] - np;
    int32_t *ps = S.pstart + (int64_t)blockIdx.x * (ns + 1);
    int32_t *pm = S.pmap + (int64_t)blockIdx.x * S.maxp;
    for (int u = b0; u < b1; ++u) {
        const int32_t v = st[u];
        const int32_t pu = (v + kAbPiece - 1) / kAbPiece;
        st[u] = run;
        ps[u] = prun;
        for (int i = 0; i < pu; ++i) pm[prun + i] = u;
        run += v;
        prun += pu;
    }
    if (threadIdx.x == 255) {
        st[ns] = total;
        ps[ns] = part[255];
    }
}

// 2d. stable scatter: one workgroup per (kind, head, chunk) of one wave
// placing both halves' entries, or (when there are few chunks, so that the
// latency of each wave's dependent chain of running offsets is what counts)
// of two waves, wave c placing half c's (the halves' sorts are independent).
// A wave walks its entries 64 at a time in token-then-list order (the next 64
// loaded while the current ones are placed); the combined entries that select
// the same sub-key find each other with one ballot per key bit and take
// consecutive places after the sub-key's running offset (in LDS), in lane
// order.  A combined entry's dsc is its first member's plus the others' in
// lane order, read from LDS.
__global__ void __launch_bounds__(2 * kWave) sdm_address_bwd_scatter_kernel(AddrBwdArgs A, AbWs S, int key_bits)
{
    extern __shared__ int32_t ctr[];   // [2][n_sub]
    __shared__ float dsl_all[2][kWave];
    int kind, h;
    int64_t ch;
    chunk_unit(A, S, kind, h, ch);
    const int ns = A.n_sub, n = kind ? A.R : A.W;
    const int32_t N = ns * ns;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const bool split = blockDim.x > kWave;
    const int c0 = split ? wave : 0, c1 = split ? wave + 1 : 2;   // the halves this wave places
    float *dsl = dsl_all[wave];
    for (int c = c0; c < c1; ++c) {
        const int32_t *cr = cnt_row(A, S, kind, h, c, ch);
        const int32_t *st = S.start + (int64_t)((kind * A.H + h) * 2 + c) * (ns + 1);
        for (int u = lane; u < ns; u += kWave) ctr[c * ns + u] = st[u] + cr[u];
    }
    __syncthreads();
    const int64_t BT = A.rows / A.H, total = BT * n;
    const int64_t f0 = ch * kAbChunk, f1 = min(total, f0 + kAbChunk);
    const int32_t *idx = kind ? A.ridx : A.widx;
    const float *dsc = S.dsc + (kind ? A.rows * A.W : 0);
    int2 *out0 = S.sorted + (kind ? S.sorted1 : 0) + (int64_t)(h * 2) * total;
    const uint64_t below = (1ull << lane) - 1ull;
    // the list entry of this lane in the group of 64 starting at fb (a valid
    // entry past the end)
    auto entry = [&](int64_t fb) {
        const int64_t f = fb + lane < f1 ? fb + lane : f0;
        const int64_t bt = f / n;
        return (bt * A.H + h) * n + (f - bt * n);
    };
    int64_t e = entry(f0);
    int32_t sl = idx[e];
    float ds = dsc[e];
    for (int64_t fb = f0; fb < f1; fb += kWave) {
        const int64_t en = entry(fb + kWave);
        const int32_t sln = idx[en];
        const float dsn = dsc[en];
        const bool ok = fb + lane < f1 && sl >= 0 && sl < N;
        const int64_t bt = e / ((int64_t)A.H * n);
        const uint64_t valid = __builtin_amdgcn_ballot_w64(ok) & same_row(bt, fb, n);
        const int32_t row = (int32_t)(e / n);
        dsl[lane] = ds;
        for (int c = c0; c < c1; ++c) {
            const int key = ok ? (c ? sl % ns : sl / ns) : 0;
            const uint64_t eq = same_key(key, key_bits);
            const uint64_t grp = eq & valid;
            const bool lead = ok && (grp & below) == 0;
            float gs = ds;
            uint64_t rest = lead ? grp & ~(below | (1ull << lane)) : 0ull;
            while (rest) {
                gs += dsl[__builtin_ctzll(rest)];
                rest &= rest - 1;
            }
            const uint64_t peers = eq & __builtin_amdgcn_ballot_w64(lead);   // this step's entries of the key
            const int rank = __builtin_popcountll(peers & below);
            const int base = ctr[c * ns + key];
            if (lead) {
                out0[(int64_t)c * total + base + rank] = make_int2(row, __float_as_int(gs));
                if (rank == 0) ctr[c * ns + key] = base + __builtin_popcountll(peers);
            }
        }
        e = en;
        sl = sln;
        ds = dsn;
    }
}

// 3a. one wave per piece (at most kAbPiece consecutive sorted entries of one
// sub-key of one (kind, head, half)): dsc * x summed in order into registers
// (each lane owns columns), the entries 64 at a time with their input rows
// loaded eight at a time; HM = ceil(half / 64) columns per lane
template <bool BF16, int HM>
__global__ void __launch_bounds__(256) sdm_address_bwd_accum_kernel(AddrBwdArgs A, AbWs S)
{
    const int half = A.d_k / 2, ns = A.n_sub;
    const int64_t unit = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int64_t seg = unit / S.maxp, lp = unit - seg * S.maxp;
    if (seg >= 2 * A.H * 2) return;                     // whole waves
    const int32_t *ps = S.pstart + seg * (ns + 1);
    if (lp >= ps[ns]) return;
    const int u = S.pmap[seg * S.maxp + lp];
    const int kind = (int)(seg / (2 * A.H)), hc = (int)(seg - (int64_t)kind * 2 * A.H), c = hc % 2;
    const int lane = lane_id();
    const int64_t BT = A.rows / A.H;
    const int n = kind ? A.R : A.W;
    const int32_t *st = S.start + seg * (ns + 1);
    const int2 *ent = S.sorted + (kind ? S.sorted1 : 0) + (int64_t)hc * BT * n;
    const void *X = kind ? A.q : A.k;
    const int32_t s0 = st[u] + (int32_t)(lp - ps[u]) * kAbPiece;
    const int32_t s1 = min(s0 + kAbPiece, st[u + 1]);
    float acc[HM];
#pragma unroll
    for (int m = 0; m < HM; ++m) acc[m] = 0.f;
    for (int32_t e0 = s0; e0 < s1; e0 += kWave) {
        const int cnt = min(kWave, s1 - e0);
        const int2 me = ent[lane < cnt ? e0 + lane : e0];
        for (int q0 = 0; q0 < cnt; q0 += 8) {
            float xv[8][HM], dq[8];
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) {
                const int q = min(q0 + qq, kWave - 1);
                const int32_t r = __builtin_amdgcn_readlane(me.x, q);
                const float d = __int_as_float(__builtin_amdgcn_readlane(me.y, q));
                dq[qq] = q0 + qq < cnt ? d : 0.f;
#pragma unroll
                for (int m = 0; m < HM; ++m) {
                    const int e = lane + kWave * m;
                    const float xl = ld_in<BF16>(X, (int64_t)r * A.d_k + c * half + (e < half ? e : 0));
                    xv[qq][m] = e < half ? xl : 0.f;
                }
            }
#pragma unroll
            for (int qq = 0; qq < 8; ++qq)
#pragma unroll
                for (int m = 0; m < HM; ++m) acc[m] = __builtin_fmaf(dq[qq], xv[qq][m], acc[m]);
        }
    }
    float *out = S.part + (seg * S.maxp + lp) * half;
#pragma unroll
    for (int m = 0; m < HM; ++m) {
        const int e = lane + kWave * m;
        if (e < half) out[e] = acc[m];
    }
}

// 3b. one wave per (head, half, sub-key) and kind (or both kinds in order
// when one buffer takes both sums): the sub-key's pieces added in order
template <int HM>
__global__ void __launch_bounds__(256) sdm_address_bwd_pieces_kernel(AddrBwdArgs A, AbWs S)
{
    const int half = A.d_k / 2, ns = A.n_sub;
    const bool shared = A.dC_w == A.dC_r;
    const int64_t per_kind = (int64_t)A.H * 2 * ns;
    const int64_t unit = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    if (unit >= (shared ? 1 : 2) * per_kind) return;   // whole waves
    const int kind0 = (int)(unit / per_kind);
    const int64_t hcu = unit - kind0 * per_kind;        // (h * 2 + c) * ns + u
    const int hc = (int)(hcu / ns), u = (int)(hcu - (int64_t)hc * ns);
    const int lane = lane_id();
    float acc[HM];
#pragma unroll
    for (int m = 0; m < HM; ++m) acc[m] = 0.f;
    for (int kind = kind0; kind <= (shared ? 1 : kind0); ++kind) {
        const int64_t seg = (int64_t)kind * 2 * A.H + hc;
        const int32_t *ps = S.pstart + seg * (ns + 1);
        const int32_t p0 = ps[u], p1 = ps[u + 1];
        for (int32_t p = p0; p < p1; ++p) {
            const float *pr = S.part + (seg * S.maxp + p) * half;
#pragma unroll
            for (int m = 0; m < HM; ++m) {
                const int e = lane + kWave * m;
                const float v = pr[e < half ? e : 0];
                acc[m] += e < half ? v : 0.f;
            }
        }
    }
    float *out = (kind0 ? A.dC_r : A.dC_w) + hcu * half;
#pragma unroll
    for (int m = 0; m < HM; ++m) {
        const int e = lane + kWave * m;
        if (e < half) out[e] = acc[m];
    }
}

hipError_t launch_address_backward(const AddrBwdArgs &A, bool bf16, void *ws, hipStream_t stream)
{
    if (A.rows == 0) return hipSuccess;
    const int half = A.d_k / 2, ns = A.n_sub;
    const int64_t BT = A.rows / A.H;
    const AddrBwdLayout L = address_bwd_layout(BT, A.H, A.W, A.R, ns, half);
    unsigned char *base = static_cast<unsigned char *>(ws);
    AbWs S;
    S.dsc = reinterpret_cast<float *>(base);
    S.cnt = reinterpret_cast<int32_t *>(base + L.off_cnt);
    S.start = reinterpret_cast<int32_t *>(base + L.off_start);
    S.sorted = reinterpret_cast<int2 *>(base + L.off_sorted);
    S.pstart = reinterpret_cast<int32_t *>(base + L.off_pstart);
    S.pmap = reinterpret_cast<int32_t *>(base + L.off_pmap);
    S.part = reinterpret_cast<float *>(base + L.off_part);
    S.maxp = L.maxp;
    S.nch[0] = L.nch[0];
    S.nch[1] = L.nch[1];
    S.cnt1 = L.cnt1;
    S.sorted1 = L.sorted1;
    int key_bits = 0;
    while ((1 << key_bits) < ns) ++key_bits;
    const int64_t b1 = (2 * ((A.rows + kAbDxRows - 1) / kAbDxRows) + 3) / 4;
    const int64_t chunks = (int64_t)A.H * (L.nch[0] + L.nch[1]);
    const int segs = 2 * A.H * 2;
    const bool shared = A.dC_w == A.dC_r;
    const int64_t b4 = (segs * L.maxp + 3) / 4;
    const int64_t b5 = ((shared ? 1 : 2) * (int64_t)A.H * 2 * ns + 3) / 4;
    const size_t hist_bytes = sizeof(int32_t) * 2 * (size_t)ns;
    const int nm = (A.d_k + kWave - 1) / kWave, hm = (half + kWave - 1) / kWave;
    // list entries whose codebook loads are issued together: 8, or 16 for
    // longer lists (32 measured slower on the 1.4B layer: fewer waves fit)
    const int maxn = A.W > A.R ? A.W : A.R;
#define SDM_AB_DX(BF, M)                                                                                      \
    do {                                                                                                      \
        if (maxn <= 8)                                                                                        \
            hipLaunchKernelGGL((sdm_address_bwd_dx_kernel<BF, M, 8>), dim3((unsigned)b1), dim3(256), 0, stream, A, \
                               S.dsc);                                                                        \
        else                                                                                                  \
            hipLaunchKernelGGL((sdm_address_bwd_dx_kernel<BF, M, 16>), dim3((unsigned)b1), dim3(256), 0, stream, \
                               A, S.dsc);                                                                     \
    } while (0)
#define SDM_AB_ACC(BF, M)                                                                                     \
    hipLaunchKernelGGL((sdm_address_bwd_accum_kernel<BF, M>), dim3((unsigned)b4), dim3(256), 0, stream, A, S)
    // the wide dx form: 16-byte codebook pieces within one half, a power-of-two
    // number of pieces per row, 16-byte aligned codebooks and outputs
    const int fpl = bf16 ? 8 : 4, nf = A.d_k / fpl;
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    // entries per lane group: ceil(max(W, R) / (64 / nf)), held in registers (at most 8)
    const int epg = nf >= 1 ? (maxn + kWave / nf - 1) / (kWave / nf) : 0;
    const bool wide = A.d_k % fpl == 0 && half % fpl == 0 && nf >= 2 && nf <= kWave && (nf & (nf - 1)) == 0 &&
                      epg <= 8 && al16(A.C_w) && al16(A.C_r) && al16(A.dk) && al16(A.dq);
#define SDM_AB_DXW_KB(BF, F, KB)                                                                              \
    hipLaunchKernelGGL((sdm_address_bwd_dx_wide_kernel<BF, F, KB>), dim3((unsigned)b1), dim3(256), 0, stream, A, \
                       S.dsc)
#define SDM_AB_DXW(BF, F)                                                                                     \
    do {                                                                                                      \
        if (epg <= 1) SDM_AB_DXW_KB(BF, F, 1);                                                                \
        else if (epg <= 2) SDM_AB_DXW_KB(BF, F, 2);                                                           \
        else if (epg <= 4) SDM_AB_DXW_KB(BF, F, 4);                                                           \
        else SDM_AB_DXW_KB(BF, F, 8);                                                                         \
    } while (0)
    if (wide) {
        if (bf16) {
            if (nf == 8) SDM_AB_DXW(true, 8);
            else if (nf == 16) SDM_AB_DXW(true, 16);
            else if (nf == 32) SDM_AB_DXW(true, 32);
            else SDM_AB_DXW(true, 64);
        } else {
            if (nf == 2) SDM_AB_DXW(false, 2);
            else if (nf == 4) SDM_AB_DXW(false, 4);
            else if (nf == 8) SDM_AB_DXW(false, 8);
            else if (nf == 16) SDM_AB_DXW(false, 16);
            else if (nf == 32) SDM_AB_DXW(false, 32);
            else SDM_AB_DXW(false, 64);
        }
    } else if (bf16) {
        if (nm <= 1) SDM_AB_DX(true, 1);
        else if (nm <= 2) SDM_AB_DX(true, 2);
        else if (nm <= 4) SDM_AB_DX(true, 4);
        else SDM_AB_DX(true, 8);
    } else {
        if (nm <= 1) SDM_AB_DX(false, 1);
        else if (nm <= 2) SDM_AB_DX(false, 2);
        else if (nm <= 4) SDM_AB_DX(false, 4);
        else SDM_AB_DX(false, 8);
    }
    hipLaunchKernelGGL(sdm_address_bwd_count_kernel, dim3((unsigned)chunks), dim3(256), hist_bytes, stream, A, S,
                       key_bits);
    hipLaunchKernelGGL(sdm_address_bwd_chunk_prefix_kernel, dim3((unsigned)(((ns + 255) / 256) * segs)), dim3(256), 0,
                       stream, A, S);
    hipLaunchKernelGGL(sdm_address_bwd_key_prefix_kernel, dim3((unsigned)segs), dim3(256), 0, stream, A, S);
    // two waves per chunk (one per half) when the chunks are few: measured
    // 179 -> 111 us on the small layer (1,024 chunks), but 1.11 -> 1.22 ms on
    // the 1.4B layer (16,384 chunks), where more waves only add scattered stores
    const int scatter_threads = chunks < 2048 ? 2 * kWave : kWave;
    hipLaunchKernelGGL(sdm_address_bwd_scatter_kernel, dim3((unsigned)chunks), dim3(scatter_threads), hist_bytes,
                       stream, A, S, key_bits);
    if (bf16) {
        if (hm <= 1) SDM_AB_ACC(true, 1);
        else if (hm <= 2) SDM_AB_ACC(true, 2);
        else SDM_AB_ACC(true, 4);
    } else {
        if (hm <= 1) SDM_AB_ACC(false, 1);
        else if (hm <= 2) SDM_AB_ACC(false, 2);
        else SDM_AB_ACC(false, 4);
    }
    if (hm <= 1)
        hipLaunchKernelGGL(sdm_address_bwd_pieces_kernel<1>, dim3((unsigned)b5), dim3(256), 0, stream, A, S);
    else if (hm <= 2)
        hipLaunchKernelGGL(sdm_address_bwd_pieces_kernel<2>, dim3((unsigned)b5), dim3(256), 0, stream, A, S);
    else
        hipLaunchKernelGGL(sdm_address_bwd_pieces_kernel<4>, dim3((unsigned)b5), dim3(256), 0, stream, A, S);
#undef SDM_AB_DX
#undef SDM_AB_DXW
#undef SDM_AB_DXW_KB
#undef SDM_AB_ACC
    return hipGetLastError();
}

}  // namespace sdm
