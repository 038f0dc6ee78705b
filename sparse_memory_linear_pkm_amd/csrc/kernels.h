// kernels.h -- launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sdm {

struct AddressKind {
    const void *x;   // [B*T*H, d_k] keys (write) or queries (read)
    const void *C;   // [H, 2, n_sub, d_k/2] codebook
    int32_t *idx;    // [B*T*H, n_out]
    float *wt;       // [B*T*H, n_out]
    int n_out;       // W or R
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
};

struct HazardArgs {
    const int32_t *widx;
    const int32_t *ridx;
    uint16_t *codes;   // [B,T,H,W+R]
    uint32_t *flags;   // [B,T,H]
    int64_t B, T, H;
    int W, R, window;
};

struct DecodeArgs {
    float *M;
    const void *k, *q, *C_w, *C_r, *v;
    const float *a, *b;
    float *o;
    int32_t *widx_out, *ridx_out;
    int B, H, d_k, n_sub, d_v, k_prime, W, R, N;
};

struct InitArgs {
    float *M;
    const float *M0;
    int64_t B;
    int64_t per_seq;  // H*N*d_v floats
};

hipError_t launch_pkm_address(const AddressArgs &args, bool bf16, hipStream_t stream);
size_t address_smem_bytes(int n_sub, int k_prime);
hipError_t launch_scan(const ScanArgs &args, bool bf16, void *workspace, size_t ws_bytes,
                       hipStream_t stream);
size_t scan_workspace_bytes(int64_t B, int64_t T, int64_t H, int W, int R, int d_v);
hipError_t launch_scan_hazard(const HazardArgs &args, hipStream_t stream);
int scan_pipe_depth(int W, int R);
hipError_t launch_scan_pipe(const ScanArgs &args, bool bf16, const uint16_t *codes, const uint32_t *flags,
                            hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &args, bool bf16, hipStream_t stream);
size_t decode_smem_bytes(int n_sub, int k_prime);
hipError_t launch_state_init(const InitArgs &args, hipStream_t stream);

}  // namespace sdm
