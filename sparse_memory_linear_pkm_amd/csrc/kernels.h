// kernels.h -- launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sdm {

// The staircase of the k' x k' merge: pairs (a, b) of half-list ranks with
// (a + 1)(b + 1) <= n.  Each of the (a + 1)(b + 1) pairs (a' <= a, b' <= b)
// scores at least as high as (a, b) (fp32 addition is monotone), so outside
// ties the top n lie inside it.  Entries (a << 8 | b) grouped by a, b
// ascending; the count is >= n for every k', n <= 64.  It depends only on
// (k', n), so the host builds it once per call and passes it by value.
constexpr int kMaxStair = 288;   // >= max over k', n <= 64 of the staircase size (280)

struct Staircase {
    uint16_t e[kMaxStair];
    int count;
};

inline void make_staircase(int kp, int n, Staircase &st)
{
    int k = 0;
    for (int a = 0; a < kp; ++a) {
        const int cnt = n / (a + 1) < kp ? n / (a + 1) : kp;
        for (int b = 0; b < cnt; ++b) st.e[k++] = (uint16_t)((a << 8) | b);
    }
    st.count = k;
}

struct AddressKind {
    const void *x;   // [B*T*H, d_k] keys (write) or queries (read)
    const void *C;   // [H, 2, n_sub, d_k/2] codebook
    int32_t *idx;    // [B*T*H, n_out]
    float *wt;       // [B*T*H, n_out]
    int n_out;       // W or R
    Staircase stair; // merge candidates for (k', n_out)
};

struct AddressArgs {
    AddressKind kind[2];  // 0: write, 1: read
    int64_t BT;           // B*T token positions per head
    int H, d_k, n_sub, k_prime;
};

struct ScanArgs {
    float *M;
    const int32_t *widx;
    const float *wwt;
    const int32_t *ridx;
    const float *rwt;
    const void *v;
    const float *a;
    const float *b;
    float *o;
    int64_t B, T;
    int H, N, d_v, W, R;
    // optional (both or neither): the rows each token used, for the backward
    // pass: xsave [B,H,T,d_v/4,W,4] the write rows before the write, zsave
    // [B,H,T,d_v/4,R,4] the read rows after it (4-column chunks, the list
    // positions of a chunk adjacent)
    float *xsave = nullptr, *zsave = nullptr;
    // optional (both or neither): a and b hold the gates' pre-activations
    // a_raw, b_raw, and the preparation pass applies the gates with the
    // per-head decay A [H] and time-step bias dt_bias [H] (gates_math.h)
    const float *A_decay = nullptr, *dt_bias = nullptr;
};


// The per-(sequence, head) streams the lane-parallel scan reads (written by
// the preparation pass, scan_prep.hip).  Streams are ordered [chain][token]
// with chain = b * H + h, so one chain's records are contiguous.
struct ScanStreams {
    uint4 *lane;        // [chain][t][Q]: {~codes, w_j, r_j, biased write row offset}
    uint2 *gofs;        // [chain][t][Q]: biased byte offsets of write / read row j
    uint4 *tok;         // [chain][t][d_v / 4]: {a_t, v chunk, b_t} (bf16) | {a_t, b_t, 0, 0}{v chunk} (f32)
};

struct PrepArgs {
    const int32_t *widx, *ridx;
    const float *wwt, *rwt, *a, *b;
    const void *v;
    ScanStreams st;
    int64_t B, T, H;
    int W, R, Q, K, window, hash_log2, d_v, bf16;   // K = tokens per scan step
    int lookahead;   // D * K - 1: superseded writes are looked for up to the end of step + D - 1
    const float *A_decay = nullptr, *dt_bias = nullptr;   // non-null: a, b are pre-activations (ScanArgs)
};

struct DecodeArgs {
    float *M;
    const void *k, *q, *C_w, *C_r, *v;
    const float *a, *b;
    float *o;
    int32_t *widx_out, *ridx_out;
    // copy-on-write state: rows of (b, h) whose bit in touched is clear are
    // read from M0 [H,N,d_v] instead of M (nullptr: M holds every row)
    const float *M0;
    uint32_t *touched;    // [B][H][ceil(N / 32)]
    int B, H, d_k, n_sub, d_v, k_prime, W, R, N;
    Staircase stair[2];   // merge candidates for (k', W) and (k', R)
};

struct CowArgs {
    float *M;
    const float *M0;
    uint32_t *touched;
    int64_t B, H, N, d_v;
};
hipError_t launch_cow_reset(const CowArgs &A, hipStream_t stream);
hipError_t launch_cow_materialize(const CowArgs &A, hipStream_t stream);

struct InitArgs {
    float *M;
    const float *M0;
    int64_t B;
    int64_t per_seq;  // H*N*d_v floats
};

struct GateArgs {
    const float *a_raw, *b_raw;   // [B*T*H]
    const float *A, *dt_bias;     // [H]
    float *a, *b;                 // [B*T*H]
    int64_t n;                    // B*T*H
    int H;
};

struct NormArgs {
    const float *o;       // [rows, d_v] fp32
    const void *g;        // [rows, d_v] bf16 or fp32
    const float *gamma;   // [d_v]
    void *y;              // [rows, d_v] same dtype as g
    int64_t rows;         // B*T*H
    int d_v;              // a multiple of 32
    float eps;
};

struct GdnArgs {
    float *S;                   // [B,H,d_k,d_v] fp32, in/out
    const void *k, *q, *v;      // [B,T,H,d_k], [B,T,H,d_k], [B,T,H,d_v]
    const float *a, *b;         // [B,T,H]
    float *o;                   // [B,T,H,d_v]
    int64_t B, T;               // T >= 1
    int H, d_k, d_v;            // d_k in {16, 32, 64, 128, 256}
};

struct BwdArgs {
    float *dM;                         // [B,H,N,d_v]: dL/dM after the call in, before it out
    const int32_t *widx, *ridx;        // [B,T,H,W], [B,T,H,R]
    const float *wwt, *rwt;
    const void *v;                     // [B,T,H,d_v]
    const float *a, *b;                // [B,T,H]
    const float *dout;                 // [B,T,H,d_v]
    const float *xsave, *zsave;        // [B,H,T,d_v/4,W,4], [B,H,T,d_v/4,R,4] from the forward
    float *dv, *da, *db, *dw, *dr;     // [B,T,H,d_v], [B,T,H] x2, [B,T,H,W], [B,T,H,R]
    int64_t B, T;
    int H, N, d_v, W, R;               // d_v a multiple of 32, <= 256
};

struct AddrBwdArgs {
    const void *k, *q, *C_w, *C_r;     // as for the addressing
    const int32_t *widx, *ridx;        // [rows, W], [rows, R]
    const float *wwt, *rwt;            // the forward's weights
    const float *dw, *dr;              // dL/dwwt, dL/drwt
    float *dk, *dq;                    // [rows, d_k]
    float *dC_w, *dC_r;                // [H,2,n_sub,d_k/2]; may be the same buffer (summed)
    int64_t rows;                      // B*T*H
    int H, d_k, n_sub, W, R;
};

// the addressing backward's workspace (see address_bwd_layout)
struct AddrBwdLayout {
    int64_t nch[2];               // chunks of list entries per (kind, head, half)
    int64_t maxp;                 // pieces of the sums pass per (kind, head, half), at most
    int half;
    size_t off_cnt, off_start, off_sorted, off_pstart, off_pmap, off_part, bytes;   // byte offsets, total size
    size_t cnt1, sorted1;         // elements of kind 0's counts and sorted entries
};
AddrBwdLayout address_bwd_layout(int64_t BT, int64_t H, int W, int R, int n_sub, int half);
size_t address_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int n_sub, int half);
hipError_t launch_address_backward(const AddrBwdArgs &args, bool bf16, void *workspace, hipStream_t stream);
hipError_t launch_scan_backward(const BwdArgs &args, bool bf16, hipStream_t stream);

// The lane-parallel backward of the scan (sdm_scan_bwd_lanes.hip): its
// workspace (0 when the shape is outside that path; the token-serial kernels
// of sdm_scan_backward.hip then run without one) and its launch.
size_t scan_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int d_v, bool bf16);
hipError_t launch_scan_backward_lanes(const BwdArgs &args, bool bf16, void *workspace, hipStream_t stream);
hipError_t launch_gdn_dense(const GdnArgs &args, bool bf16, hipStream_t stream);
struct GateBwdArgs {
    const float *a_raw, *b_raw, *A, *dt_bias, *da, *db;
    float *da_raw, *db_raw, *dA, *ddt;
    float *part;                  // workspace [2][parts][H]: per-part sums of dA, ddt_bias
    int64_t n;                    // B*T*H
    int64_t H;
};

// grid of the gates' backward (see gates_bwd_layout)
struct GateBwdLayout {
    int hp, hblocks, parts;
    int64_t chunk;                // tokens per part
};
constexpr int kGateBwdParts = 512;
GateBwdLayout gates_bwd_layout(int64_t bt, int64_t H);

struct NormBwdArgs {
    const float *o;
    const void *g;
    const float *gamma, *dy;
    float *dout, *dg, *dgamma;
    float *part;                  // workspace [norm_bwd_blocks(rows)][d_v]
    int64_t rows;
    int d_v;
    float eps;
};

// workgroups (and dgamma partial rows) of the norm's backward
constexpr int kNormBwdBlocks = 1024;
int norm_bwd_blocks(int64_t rows);
hipError_t launch_gates_backward(const GateBwdArgs &args, hipStream_t stream);
hipError_t launch_out_norm_gate_backward(const NormBwdArgs &args, bool bf16, hipStream_t stream);
hipError_t launch_gates(const GateArgs &args, hipStream_t stream);
hipError_t launch_out_norm_gate(const NormArgs &args, bool bf16, hipStream_t stream);
// one_per_cu: launched so that a CU holds at most one of its workgroups
// (room for a concurrent scan on another stream); same results
hipError_t launch_pkm_address(const AddressArgs &args, bool bf16, hipStream_t stream, bool one_per_cu = false);
size_t address_smem_bytes(int n_sub, int k_prime);
hipError_t launch_scan(const ScanArgs &args, bool bf16, void *workspace, size_t ws_bytes,
                       hipStream_t stream);
size_t scan_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int d_v, bool bf16);
bool scan_chain_fits(int64_t T, int W, int R, int d_v, bool bf16);
hipError_t launch_scan_prep(const PrepArgs &args, hipStream_t stream);
int scan_prep_hash_log2(int W, int window, int lookahead);
hipError_t launch_scan_lanes(const ScanArgs &args, bool bf16, const ScanStreams &st, int Q, int G, int D,
                             hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &args, bool bf16, hipStream_t stream);
hipError_t launch_state_init(const InitArgs &args, hipStream_t stream);

}  // namespace sdm
