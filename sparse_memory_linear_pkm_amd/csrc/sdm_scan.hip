// sdm_scan.hip -- prefill scan: the sequence-serial sparse gated delta rule
// over T tokens for every (sequence, head), in place on the HBM-resident
// memory.  "Sparse Delta Memory: Scaling the State of Linear RNNs through
// Sparsity", Sec. 3.1 steps 2-3 (Eq. 4).
//
// Two launches on the caller's stream: the preparation pass (scan_prep.hip:
// forwarding codes and the repacked per-chain input streams) and the
// lane-parallel scan (sdm_scan_lanes.hip).
#include "kernels.h"

namespace sdm {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Lanes per token of the lane-parallel scan: the power of two >= max(W, R).
static int scan_lanes_q(int W, int R)
{
    int q = 4;
    while (q < W || q < R) q *= 2;
    return q;
}

// Shape of the lane-parallel scan: G waves per workgroup (one G*16-byte
// row segment each) and pipeline depth D (steps in flight).  The widest
// segment that still gives every CU a workgroup wins (whole 128-byte lines
// per access); a workgroup holds D * G * 4 KB of LDS (16 KB of gathered rows
// per step in flight and a ring of the rows written by the last 2D steps,
// per 8 waves), so D = 2 lets two 8-wave workgroups share a CU.  Narrower
// workgroups run one wave per SIMD, whose steps are long enough that D = 4
// hides the gathers; a deeper pipeline would only widen the forwarding
// window the preparation pass searches.
struct LanesShape {
    int G, D;
};

static LanesShape scan_lanes_shape(int64_t chunks)   // chunks = B * H * d_v / 4
{
    constexpr int64_t kCUs = 256;
    if (chunks / 8 >= 2 * kCUs) return {8, 2};
    if (chunks / 8 >= kCUs) return {8, 4};
    if (chunks / 4 >= kCUs) return {4, 4};
    return {2, 4};
}

// Workspace: the three streams of the preparation pass, each 256-byte
// aligned: lane records [B*H, T, Q] (16 bytes), row offsets [B*H, T, Q]
// (8 bytes) and token records [B*H, T, d_v/4] (16 bytes, 32 for fp32 v).
struct WsLayout {
    size_t lane, gofs, tok, total;
};

static WsLayout ws_layout(int64_t B, int64_t T, int64_t H, int W, int R, int d_v, bool bf16)
{
    const size_t rows = (size_t)(B * T * H);
    const size_t q = (size_t)scan_lanes_q(W, R);
    WsLayout L;
    L.lane = 0;
    L.gofs = L.lane + align256(rows * q * 16);
    L.tok = L.gofs + align256(rows * q * 8);
    L.total = L.tok + align256(rows * (size_t)(d_v / 4) * (bf16 ? 16 : 32));
    return L;
}

size_t scan_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int d_v, bool bf16)
{
    return ws_layout(B, T, H, W, R, d_v, bf16).total;
}

bool scan_chain_fits(int64_t T, int W, int R, int d_v, bool bf16)
{
    const uint64_t q = (uint64_t)scan_lanes_q(W, R);
    const uint64_t lim = 1ull << 31;
    return (uint64_t)T * q * 16 < lim && (uint64_t)T * (uint64_t)(d_v / 4) * (bf16 ? 16 : 32) < lim;
}

hipError_t launch_scan(const ScanArgs &A, bool bf16, void *ws, size_t, hipStream_t stream)
{
    const int64_t units = A.B * A.H * (A.d_v / 4);
    if (units == 0 || A.T == 0) return hipSuccess;
    const int Q = scan_lanes_q(A.W, A.R);
    const LanesShape sh = scan_lanes_shape(units);
    const int D = sh.D;
    const int K = 64 / Q;
    // rows written in the last 2D steps may not be visible to a gather yet
    const int window = 2 * D * K - 1;
    const WsLayout L = ws_layout(A.B, A.T, A.H, A.W, A.R, A.d_v, bf16);
    unsigned char *base = static_cast<unsigned char *>(ws);
    ScanStreams st{reinterpret_cast<uint4 *>(base + L.lane), reinterpret_cast<uint2 *>(base + L.gofs),
                   reinterpret_cast<uint4 *>(base + L.tok)};
    PrepArgs pa{A.widx, A.ridx, A.wwt, A.rwt, A.a, A.b, A.v, st, A.B, A.T, A.H,
                A.W, A.R, Q, K, window, scan_prep_hash_log2(A.W, window, D * K - 1), A.d_v, bf16 ? 1 : 0,
                D * K - 1, A.A_decay, A.dt_bias};
    hipError_t e = launch_scan_prep(pa, stream);
    if (e != hipSuccess) return e;
    return launch_scan_lanes(A, bf16, st, Q, sh.G, D, stream);
}

}  // namespace sdm
