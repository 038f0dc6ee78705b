// sdm_api.hip -- the C ABI declared in include/sdm.h: host-side validation,
// error reporting and kernel launches.  No device memory is allocated here
// and no pointer is kept after a call returns.
#include "../../include/sdm.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.h"

// Scratch of sdm_scan_forward_noalloc: the scan's preparation streams live
// here instead of in a caller workspace.  Each GPU the library runs on holds
// its own copy (SDM_NOALLOC_SCRATCH_BYTES) until the process ends.  In host
// code the name is only a host-side stand-in: kernels get the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SDM_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

sdm_status fail(sdm_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

sdm_status hip_fail(hipError_t e, const char *what)
{
    return fail(SDM_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

constexpr int64_t kMaxList = 64;      // W, R, k' per wave-level selection
constexpr int64_t kMaxNsub = 2048;    // 16 x n_sub fp32 score tile in LDS
constexpr int64_t kMaxDv = 1024;

// Checks shared by every call that uses the memory geometry.
sdm_status check_memory_dims(const sdm_dims *d)
{
    if (!d) return fail(SDM_ERR_INVALID_ARG, "dims is NULL");
    if (d->reserved != 0) return fail(SDM_ERR_INVALID_ARG, "dims.reserved must be 0");
    if (d->B < 0 || d->H < 1 || d->n_sub < 1 || d->d_v < 1)
        return fail(SDM_ERR_INVALID_ARG, "need B >= 0, H >= 1, n_sub >= 1, d_v >= 1 (got B=%lld H=%lld n_sub=%lld d_v=%lld)",
                    (long long)d->B, (long long)d->H, (long long)d->n_sub, (long long)d->d_v);
    if (d->n_sub > 46340) return fail(SDM_ERR_INVALID_ARG, "n_sub^2 must fit in int32");
    if (d->B > 0x7FFFFFFF) return fail(SDM_ERR_UNSUPPORTED, "B must be < 2^31 (got %lld)", (long long)d->B);
    if (d->d_v % 32 != 0 || d->d_v > kMaxDv)
        return fail(SDM_ERR_UNSUPPORTED, "d_v must be a multiple of 32 and <= %lld (got %lld)",
                    (long long)kMaxDv, (long long)d->d_v);
    const uint64_t row_bytes = (uint64_t)d->d_v * 4u;
    if ((uint64_t)d->n_sub * (uint64_t)d->n_sub * row_bytes > (1ull << 31))
        return fail(SDM_ERR_UNSUPPORTED, "one (sequence, head) memory must be <= 2 GiB");
    return SDM_OK;
}

sdm_status check_method_dims(const sdm_dims *d, bool need_T)
{
    sdm_status st = check_memory_dims(d);
    if (st != SDM_OK) return st;
    if (need_T && d->T < 0) return fail(SDM_ERR_INVALID_ARG, "T must be >= 0");
    if (d->in_dtype != SDM_F32 && d->in_dtype != SDM_BF16)
        return fail(SDM_ERR_INVALID_ARG, "in_dtype must be SDM_F32 or SDM_BF16");
    if (d->d_k < 2 || (d->d_k & 1)) return fail(SDM_ERR_INVALID_ARG, "d_k must be even and >= 2");
    if (d->k_prime < 1 || d->k_prime > d->n_sub)
        return fail(SDM_ERR_INVALID_ARG, "need 1 <= k_prime <= n_sub");
    if (d->W < 1 || d->R < 1 || d->W > d->k_prime * d->k_prime || d->R > d->k_prime * d->k_prime)
        return fail(SDM_ERR_INVALID_ARG, "need 1 <= W, R <= k_prime^2");
    if (d->W > kMaxList || d->R > kMaxList || d->k_prime > kMaxList)
        return fail(SDM_ERR_UNSUPPORTED, "W, R and k_prime must be <= %lld", (long long)kMaxList);
    if (d->n_sub > kMaxNsub) return fail(SDM_ERR_UNSUPPORTED, "n_sub must be <= %lld", (long long)kMaxNsub);
    if (d->d_k > 512) return fail(SDM_ERR_UNSUPPORTED, "d_k must be <= 512");
    if (d->in_dtype == SDM_BF16 && ((d->d_k / 2) % 32) != 0)
        return fail(SDM_ERR_UNSUPPORTED, "bf16 inputs need d_k/2 to be a multiple of 32 (MFMA K)");
    return SDM_OK;
}

hipStream_t as_stream(sdm_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

size_t in_size(const sdm_dims *d) { return d->in_dtype == SDM_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

const char *sdm_status_string(sdm_status st)
{
    switch (st) {
    case SDM_OK: return "ok";
    case SDM_ERR_INVALID_ARG: return "invalid argument";
    case SDM_ERR_UNSUPPORTED: return "unsupported by this implementation";
    case SDM_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *sdm_last_error(void) { return g_last_error.c_str(); }

int sdm_version(void) { return 1 * 10000 + 0 * 100 + 0; }

sdm_status sdm_state_init(float *M, const float *M0, const sdm_dims *d, sdm_stream_t stream)
{
    sdm_status st = check_memory_dims(d);
    if (st != SDM_OK) return st;
    if (d->B == 0) return SDM_OK;
    if (!M || !M0) return fail(SDM_ERR_INVALID_ARG, "M and M0 must be non-NULL");
    if (!aligned(M, 16) || !aligned(M0, 16)) return fail(SDM_ERR_INVALID_ARG, "M and M0 must be 16-byte aligned");
    const int64_t per_seq = d->H * d->n_sub * d->n_sub * d->d_v;
    if (overlap(M, sizeof(float) * per_seq * d->B, M0, sizeof(float) * per_seq))
        return fail(SDM_ERR_INVALID_ARG, "M and M0 overlap");
    sdm::InitArgs A{M, M0, d->B, per_seq};
    hipError_t e = sdm::launch_state_init(A, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_state_init launch");
}

static sdm_status address_impl(const void *k, const void *q, const void *C_w, const void *C_r, const sdm_dims *d,
                               int32_t *widx, float *wwt, int32_t *ridx, float *rwt, sdm_stream_t stream,
                               bool one_per_cu);

sdm_status sdm_pkm_address(const void *k, const void *q, const void *C_w, const void *C_r,
                           const sdm_dims *d, int32_t *widx, float *wwt, int32_t *ridx, float *rwt,
                           sdm_stream_t stream)
{
    return address_impl(k, q, C_w, C_r, d, widx, wwt, ridx, rwt, stream, false);
}

sdm_status sdm_pkm_address_overlapped(const void *k, const void *q, const void *C_w, const void *C_r,
                                      const sdm_dims *d, int32_t *widx, float *wwt, int32_t *ridx, float *rwt,
                                      sdm_stream_t stream)
{
    return address_impl(k, q, C_w, C_r, d, widx, wwt, ridx, rwt, stream, true);
}

static sdm_status address_impl(const void *k, const void *q, const void *C_w, const void *C_r, const sdm_dims *d,
                               int32_t *widx, float *wwt, int32_t *ridx, float *rwt, sdm_stream_t stream,
                               bool one_per_cu)
{
    sdm_status st = check_method_dims(d, true);
    if (st != SDM_OK) return st;
    if (d->B * d->T == 0) return SDM_OK;
    if (!k || !q || !C_w || !C_r || !widx || !wwt || !ridx || !rwt)
        return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    const size_t al = d->in_dtype == SDM_BF16 ? 16 : 4;
    if (!aligned(k, al) || !aligned(q, al) || !aligned(C_w, al) || !aligned(C_r, al))
        return fail(SDM_ERR_INVALID_ARG, "k, q, C_w, C_r must be %zu-byte aligned", al);
    if (!aligned(widx, 4) || !aligned(wwt, 4) || !aligned(ridx, 4) || !aligned(rwt, 4))
        return fail(SDM_ERR_INVALID_ARG, "slot and weight outputs must be 4-byte aligned");
    const int64_t rows = d->B * d->T * d->H;
    if (overlap(widx, 4 * rows * d->W, ridx, 4 * rows * d->R) ||
        overlap(wwt, 4 * rows * d->W, rwt, 4 * rows * d->R) ||
        overlap(widx, 4 * rows * d->W, wwt, 4 * rows * d->W) ||
        overlap(ridx, 4 * rows * d->R, rwt, 4 * rows * d->R))
        return fail(SDM_ERR_INVALID_ARG, "output buffers overlap");
    if (rows == 0) return SDM_OK;
    sdm::AddressArgs A{};
    A.kind[0] = {k, C_w, widx, wwt, (int)d->W, {}};
    A.kind[1] = {q, C_r, ridx, rwt, (int)d->R, {}};
    sdm::make_staircase((int)d->k_prime, (int)d->W, A.kind[0].stair);
    sdm::make_staircase((int)d->k_prime, (int)d->R, A.kind[1].stair);
    A.BT = d->B * d->T;
    A.H = (int)d->H;
    A.d_k = (int)d->d_k;
    A.n_sub = (int)d->n_sub;
    A.k_prime = (int)d->k_prime;
    hipError_t e = sdm::launch_pkm_address(A, d->in_dtype == SDM_BF16, as_stream(stream), one_per_cu);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_pkm_address launch");
}

size_t sdm_scan_workspace_size(const sdm_dims *d)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1 || d->W < 1 || d->R < 1 || d->d_v < 1 || d->W > kMaxList ||
        d->R > kMaxList)
        return 0;
    return sdm::scan_workspace_bytes(d->B, d->T, d->H, (int)d->W, (int)d->R, (int)d->d_v,
                                     d->in_dtype == SDM_BF16);
}

static sdm_status scan_forward_impl(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                                    const float *rwt, const void *v, const float *a, const float *b, float *o,
                                    float *xsave, float *zsave, void *workspace, size_t workspace_bytes,
                                    const sdm_dims *d, sdm_stream_t stream, bool noalloc = false,
                                    const float *A_decay = nullptr, const float *dt_bias = nullptr);

sdm_status sdm_scan_forward(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                            const float *rwt, const void *v, const float *a, const float *b,
                            float *o, void *workspace, size_t workspace_bytes, const sdm_dims *d,
                            sdm_stream_t stream)
{
    return scan_forward_impl(M, widx, wwt, ridx, rwt, v, a, b, o, nullptr, nullptr, workspace, workspace_bytes, d,
                             stream);
}

sdm_status sdm_scan_forward_gated(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                                  const float *rwt, const void *v, const float *a_raw, const float *b_raw,
                                  const float *A, const float *dt_bias, float *o, void *workspace,
                                  size_t workspace_bytes, const sdm_dims *d, sdm_stream_t stream)
{
    if (d && d->B * d->T > 0 && (!A || !dt_bias)) return fail(SDM_ERR_INVALID_ARG, "A and dt_bias must be non-NULL");
    if (d && d->B * d->T > 0 && (!aligned(A, 4) || !aligned(dt_bias, 4)))
        return fail(SDM_ERR_INVALID_ARG, "A and dt_bias must be 4-byte aligned");
    return scan_forward_impl(M, widx, wwt, ridx, rwt, v, a_raw, b_raw, o, nullptr, nullptr, workspace,
                             workspace_bytes, d, stream, false, A, dt_bias);
}

sdm_status sdm_scan_forward_noalloc(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                                    const float *rwt, const void *v, const float *a, const float *b, float *o,
                                    const sdm_dims *d, sdm_stream_t stream)
{
    return scan_forward_impl(M, widx, wwt, ridx, rwt, v, a, b, o, nullptr, nullptr, nullptr, 0, d, stream, true);
}

sdm_status sdm_scan_forward_save(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                                 const float *rwt, const void *v, const float *a, const float *b, float *o,
                                 float *xsave, float *zsave, void *workspace, size_t workspace_bytes,
                                 const sdm_dims *d, sdm_stream_t stream)
{
    if (d && d->B * d->T > 0 && (!xsave || !zsave))
        return fail(SDM_ERR_INVALID_ARG, "xsave and zsave must be non-NULL");
    if (!xsave || !zsave) return scan_forward_impl(M, widx, wwt, ridx, rwt, v, a, b, o, nullptr, nullptr, workspace,
                                                   workspace_bytes, d, stream);
    return scan_forward_impl(M, widx, wwt, ridx, rwt, v, a, b, o, xsave, zsave, workspace, workspace_bytes, d,
                             stream);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; later calls reuse it.
static sdm_status scratch_address(void **out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SDM_ERR_UNSUPPORTED, "device ordinal %d beyond the %d the static scratch tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(SDM_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        addr[dev] = p;
    }
    *out = addr[dev];
    return SDM_OK;
}

static sdm_status scan_forward_impl(float *M, const int32_t *widx, const float *wwt, const int32_t *ridx,
                                    const float *rwt, const void *v, const float *a, const float *b, float *o,
                                    float *xsave, float *zsave, void *workspace, size_t workspace_bytes,
                                    const sdm_dims *d, sdm_stream_t stream, bool noalloc, const float *A_decay,
                                    const float *dt_bias)
{
    sdm_status st = check_memory_dims(d);
    if (st != SDM_OK) return st;
    if (d->T < 0) return fail(SDM_ERR_INVALID_ARG, "T must be >= 0");
    if (d->in_dtype != SDM_F32 && d->in_dtype != SDM_BF16)
        return fail(SDM_ERR_INVALID_ARG, "in_dtype must be SDM_F32 or SDM_BF16");
    if (d->W < 1 || d->R < 1) return fail(SDM_ERR_INVALID_ARG, "need W, R >= 1");
    if (d->W > d->n_sub * d->n_sub || d->R > d->n_sub * d->n_sub)
        return fail(SDM_ERR_INVALID_ARG, "W and R must not exceed N");
    if (d->W > kMaxList || d->R > kMaxList)
        return fail(SDM_ERR_UNSUPPORTED, "W and R must be <= %lld", (long long)kMaxList);
    if (d->B * d->T == 0) return SDM_OK;
    if (!M || !widx || !wwt || !ridx || !rwt || !v || !a || !b || !o)
        return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(M, 16) || !aligned(o, 16)) return fail(SDM_ERR_INVALID_ARG, "M and o must be 16-byte aligned");
    if (!aligned(v, d->in_dtype == SDM_BF16 ? 8 : 16)) return fail(SDM_ERR_INVALID_ARG, "v is misaligned");
    if (!aligned(widx, 4) || !aligned(wwt, 4) || !aligned(ridx, 4) || !aligned(rwt, 4) ||
        !aligned(a, 4) || !aligned(b, 4))
        return fail(SDM_ERR_INVALID_ARG, "slot lists, weights and gates must be 4-byte aligned");
    const int64_t N = d->n_sub * d->n_sub;
    const int64_t rows = d->B * d->T * d->H;
    const size_t msz = sizeof(float) * (size_t)(d->B * d->H * N * d->d_v);
    const size_t osz = sizeof(float) * (size_t)(rows * d->d_v);
    if (overlap(o, osz, M, msz)) return fail(SDM_ERR_INVALID_ARG, "o overlaps M");
    if (overlap(o, osz, widx, 4 * rows * d->W) || overlap(o, osz, ridx, 4 * rows * d->R) ||
        overlap(o, osz, wwt, 4 * rows * d->W) || overlap(o, osz, rwt, 4 * rows * d->R))
        return fail(SDM_ERR_INVALID_ARG, "o overlaps a slot list or weight array");
    if (overlap(M, msz, widx, 4 * rows * d->W) || overlap(M, msz, ridx, 4 * rows * d->R) ||
        overlap(M, msz, wwt, 4 * rows * d->W) || overlap(M, msz, rwt, 4 * rows * d->R))
        return fail(SDM_ERR_INVALID_ARG, "M overlaps a slot list or weight array");
    if (!sdm::scan_chain_fits(d->T, (int)d->W, (int)d->R, (int)d->d_v, d->in_dtype == SDM_BF16))
        return fail(SDM_ERR_UNSUPPORTED, "T too large: one (sequence, head) stream of the scan must stay below 2 GiB");
    const size_t need = sdm::scan_workspace_bytes(d->B, d->T, d->H, (int)d->W, (int)d->R, (int)d->d_v,
                                                  d->in_dtype == SDM_BF16);
    if (noalloc) {
        if (need > (size_t)SDM_NOALLOC_SCRATCH_BYTES)
            return fail(SDM_ERR_UNSUPPORTED,
                        "sdm_scan_forward_noalloc: these dims need %zu bytes of scratch, the static scratch holds "
                        "%zu (split T or B, or call sdm_scan_forward with a workspace)",
                        need, (size_t)SDM_NOALLOC_SCRATCH_BYTES);
        // every byte the scan reads from the scratch is written first by its
        // preparation pass in the same call, so nothing needs clearing
        sdm_status sst = scratch_address(&workspace);
        if (sst != SDM_OK) return sst;
        workspace_bytes = (size_t)SDM_NOALLOC_SCRATCH_BYTES;
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(SDM_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (need > 0 && !aligned(workspace, 16)) return fail(SDM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    {
        const size_t vsz = (size_t)(rows * d->d_v) * (d->in_dtype == SDM_BF16 ? 2 : 4);
        if (overlap(workspace, need, M, msz) || overlap(workspace, need, o, osz) ||
            overlap(workspace, need, v, vsz) || overlap(workspace, need, widx, 4 * rows * d->W) ||
            overlap(workspace, need, ridx, 4 * rows * d->R) || overlap(workspace, need, wwt, 4 * rows * d->W) ||
            overlap(workspace, need, rwt, 4 * rows * d->R) || overlap(workspace, need, a, 4 * rows) ||
            overlap(workspace, need, b, 4 * rows))
            return fail(SDM_ERR_INVALID_ARG, "workspace overlaps an input or output");
    }
    if (xsave) {
        if (!aligned(xsave, 16) || !aligned(zsave, 16)) return fail(SDM_ERR_INVALID_ARG, "xsave and zsave must be 16-byte aligned");
        const uint64_t per = (uint64_t)d->T * (uint64_t)(d->W > d->R ? d->W : d->R) * (uint64_t)d->d_v * 4u;
        if (per >= (1ull << 31))
            return fail(SDM_ERR_UNSUPPORTED, "T too large to save: one (sequence, head) of xsave or zsave must stay below 2 GiB");
        const size_t xb = sizeof(float) * (size_t)(rows * d->W * d->d_v), zb = sizeof(float) * (size_t)(rows * d->R * d->d_v);
        if (overlap(xsave, xb, zsave, zb) || overlap(xsave, xb, M, msz) || overlap(zsave, zb, M, msz) ||
            overlap(xsave, xb, o, osz) || overlap(zsave, zb, o, osz) || overlap(xsave, xb, workspace, need) ||
            overlap(zsave, zb, workspace, need))
            return fail(SDM_ERR_INVALID_ARG, "xsave or zsave overlaps another buffer");
    }
    if (A_decay) {   // the gated form: A and dt_bias [H] are read while M, o and the workspace are written
        const size_t hb = sizeof(float) * (size_t)d->H;
        if (overlap(A_decay, hb, M, msz) || overlap(A_decay, hb, o, osz) || overlap(A_decay, hb, workspace, need) ||
            overlap(dt_bias, hb, M, msz) || overlap(dt_bias, hb, o, osz) || overlap(dt_bias, hb, workspace, need))
            return fail(SDM_ERR_INVALID_ARG, "A or dt_bias overlaps M, o or the workspace");
    }
    if (rows == 0) return SDM_OK;
    sdm::ScanArgs A{M, widx, wwt, ridx, rwt, v, a, b, o, d->B, d->T, (int)d->H, (int)N, (int)d->d_v,
                    (int)d->W, (int)d->R, xsave, zsave, A_decay, dt_bias};
    hipError_t e = sdm::launch_scan(A, d->in_dtype == SDM_BF16, workspace, workspace_bytes,
                                    as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_scan_forward launch");
}

static sdm_status decode_impl(float *M, const float *M0, uint32_t *touched, const void *k, const void *q,
                              const void *C_w, const void *C_r, const void *v, const float *a, const float *b,
                              float *o, int32_t *widx_out, int32_t *ridx_out, const sdm_dims *d, sdm_stream_t stream);

sdm_status sdm_decode_step(float *M, const void *k, const void *q, const void *C_w, const void *C_r,
                           const void *v, const float *a, const float *b, float *o, int32_t *widx_out,
                           int32_t *ridx_out, const sdm_dims *d, sdm_stream_t stream)
{
    return decode_impl(M, nullptr, nullptr, k, q, C_w, C_r, v, a, b, o, widx_out, ridx_out, d, stream);
}

size_t sdm_cow_bitmap_bytes(const sdm_dims *d)
{
    if (!d || d->B < 0 || d->H < 1 || d->n_sub < 1 || d->n_sub > 46340) return 0;
    return sizeof(uint32_t) * (size_t)(d->B * d->H) * (size_t)((d->n_sub * d->n_sub + 31) / 32);
}

// checks shared by the copy-on-write calls: M0, the bitmap, and their overlaps with M
static sdm_status check_cow(float *M, const float *M0, const uint32_t *touched, const sdm_dims *d)
{
    if (!M || !M0 || !touched) return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(M, 16) || !aligned(M0, 16) || !aligned(touched, 4))
        return fail(SDM_ERR_INVALID_ARG, "M and M0 must be 16-byte aligned, the bitmap 4-byte aligned");
    const int64_t N = d->n_sub * d->n_sub;
    const size_t msz = sizeof(float) * (size_t)(d->B * d->H * N * d->d_v);
    const size_t m0sz = sizeof(float) * (size_t)(d->H * N * d->d_v);
    const size_t tsz = sdm_cow_bitmap_bytes(d);
    if (overlap(M, msz, M0, m0sz) || overlap(touched, tsz, M, msz) || overlap(touched, tsz, M0, m0sz))
        return fail(SDM_ERR_INVALID_ARG, "M, M0 and the bitmap must not overlap");
    return SDM_OK;
}

sdm_status sdm_cow_reset(uint32_t *touched, const sdm_dims *d, sdm_stream_t stream)
{
    if (!d) return fail(SDM_ERR_INVALID_ARG, "dims is NULL");
    if (d->B < 0 || d->H < 1 || d->n_sub < 1) return fail(SDM_ERR_INVALID_ARG, "need B >= 0, H >= 1, n_sub >= 1");
    if (d->n_sub > 46340) return fail(SDM_ERR_INVALID_ARG, "n_sub^2 must fit in int32");
    if (d->B > 0x7FFFFFFF) return fail(SDM_ERR_UNSUPPORTED, "B must be < 2^31 (got %lld)", (long long)d->B);
    if (d->B == 0) return SDM_OK;
    if (!touched || !aligned(touched, 4)) return fail(SDM_ERR_INVALID_ARG, "NULL or misaligned bitmap");
    sdm::CowArgs A{nullptr, nullptr, touched, d->B, d->H, d->n_sub * d->n_sub, d->d_v};
    hipError_t e = sdm::launch_cow_reset(A, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_cow_reset launch");
}

sdm_status sdm_cow_materialize(float *M, const float *M0, uint32_t *touched, const sdm_dims *d,
                               sdm_stream_t stream)
{
    sdm_status st = check_memory_dims(d);
    if (st != SDM_OK) return st;
    if (d->B == 0) return SDM_OK;
    st = check_cow(M, M0, touched, d);
    if (st != SDM_OK) return st;
    sdm::CowArgs A{M, M0, touched, d->B, d->H, d->n_sub * d->n_sub, d->d_v};
    hipError_t e = sdm::launch_cow_materialize(A, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_cow_materialize launch");
}

sdm_status sdm_decode_step_cow(float *M, const float *M0, uint32_t *touched, const void *k, const void *q,
                               const void *C_w, const void *C_r, const void *v, const float *a, const float *b,
                               float *o, int32_t *widx_out, int32_t *ridx_out, const sdm_dims *d,
                               sdm_stream_t stream)
{
    if (d && d->B > 0) {
        if (!M0 || !touched) return fail(SDM_ERR_INVALID_ARG, "M0 and the bitmap must be non-NULL");
    }
    return decode_impl(M, M0, touched, k, q, C_w, C_r, v, a, b, o, widx_out, ridx_out, d, stream);
}

static sdm_status decode_impl(float *M, const float *M0, uint32_t *touched, const void *k, const void *q,
                              const void *C_w, const void *C_r, const void *v, const float *a, const float *b,
                              float *o, int32_t *widx_out, int32_t *ridx_out, const sdm_dims *d, sdm_stream_t stream)
{
    sdm_status st = check_method_dims(d, false);
    if (st != SDM_OK) return st;
    if (d->T != 1) return fail(SDM_ERR_INVALID_ARG, "sdm_decode_step needs dims.T == 1");
    if (d->B == 0) return SDM_OK;
    if (!M || !k || !q || !C_w || !C_r || !v || !a || !b || !o)
        return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    const size_t al = d->in_dtype == SDM_BF16 ? 16 : 4;
    if (!aligned(k, al) || !aligned(q, al) || !aligned(C_w, al) || !aligned(C_r, al))
        return fail(SDM_ERR_INVALID_ARG, "k, q, C_w, C_r must be %zu-byte aligned", al);
    if (!aligned(M, 16) || !aligned(o, 16)) return fail(SDM_ERR_INVALID_ARG, "M and o must be 16-byte aligned");
    if (!aligned(v, d->in_dtype == SDM_BF16 ? 8 : 16)) return fail(SDM_ERR_INVALID_ARG, "v is misaligned");
    if (!aligned(a, 4) || !aligned(b, 4) || !aligned(widx_out, 4) || !aligned(ridx_out, 4))
        return fail(SDM_ERR_INVALID_ARG, "gates and slot outputs must be 4-byte aligned");
    const int64_t N = d->n_sub * d->n_sub;
    const size_t msz = sizeof(float) * (size_t)(d->B * d->H * N * d->d_v);
    if (overlap(o, sizeof(float) * d->B * d->H * d->d_v, M, msz)) return fail(SDM_ERR_INVALID_ARG, "o overlaps M");
    if (d->B * d->H > 0x7fffffff) return fail(SDM_ERR_UNSUPPORTED, "B*H too large");
    if (d->B == 0) return SDM_OK;
    if (touched) {
        const sdm_status cs = check_cow(M, M0, touched, d);
        if (cs != SDM_OK) return cs;
        const size_t tsz = sdm_cow_bitmap_bytes(d);
        const size_t osz = sizeof(float) * (size_t)(d->B * d->H * d->d_v);
        if (overlap(touched, tsz, o, osz) || overlap(M0, sizeof(float) * (size_t)(d->H * N * d->d_v), o, osz))
            return fail(SDM_ERR_INVALID_ARG, "o overlaps M0 or the bitmap");
    }
    sdm::DecodeArgs A{};
    A.M = M; A.k = k; A.q = q; A.C_w = C_w; A.C_r = C_r; A.v = v; A.a = a; A.b = b; A.o = o;
    A.widx_out = widx_out; A.ridx_out = ridx_out;
    A.M0 = M0; A.touched = touched;
    A.B = (int)d->B; A.H = (int)d->H; A.d_k = (int)d->d_k; A.n_sub = (int)d->n_sub;
    A.d_v = (int)d->d_v; A.k_prime = (int)d->k_prime; A.W = (int)d->W; A.R = (int)d->R; A.N = (int)N;
    sdm::make_staircase(A.k_prime, A.W, A.stair[0]);
    sdm::make_staircase(A.k_prime, A.R, A.stair[1]);
    hipError_t e = sdm::launch_decode(A, d->in_dtype == SDM_BF16, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_decode_step launch");
}

sdm_status sdm_gates(const float *a_raw, const float *b_raw, const float *A, const float *dt_bias,
                     const sdm_dims *d, float *a, float *b, sdm_stream_t stream)
{
    if (!d) return fail(SDM_ERR_INVALID_ARG, "dims is NULL");
    if (d->reserved != 0) return fail(SDM_ERR_INVALID_ARG, "dims.reserved must be 0");
    if (d->B < 0 || d->T < 0 || d->H < 1)
        return fail(SDM_ERR_INVALID_ARG, "need B >= 0, T >= 0, H >= 1");
    if (d->H > 0x7fffffff) return fail(SDM_ERR_UNSUPPORTED, "H too large");
    if (d->B * d->T == 0) return SDM_OK;
    if (!a_raw || !b_raw || !A || !dt_bias || !a || !b) return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(a_raw, 4) || !aligned(b_raw, 4) || !aligned(A, 4) || !aligned(dt_bias, 4) || !aligned(a, 4) ||
        !aligned(b, 4))
        return fail(SDM_ERR_INVALID_ARG, "gate arrays must be 4-byte aligned");
    const int64_t n = d->B * d->T * d->H;
    const size_t nb = sizeof(float) * (size_t)n, hb = sizeof(float) * (size_t)d->H;
    // a may be a_raw and b may be b_raw (in place); any other overlap is an error
    if (overlap(a, nb, b, nb) || overlap(a, nb, b_raw, nb) || overlap(b, nb, a_raw, nb) ||
        (a != a_raw && overlap(a, nb, a_raw, nb)) || (b != b_raw && overlap(b, nb, b_raw, nb)))
        return fail(SDM_ERR_INVALID_ARG, "a and b may only alias a_raw and b_raw exactly");
    if (overlap(a, nb, A, hb) || overlap(a, nb, dt_bias, hb) || overlap(b, nb, A, hb) || overlap(b, nb, dt_bias, hb))
        return fail(SDM_ERR_INVALID_ARG, "a or b overlaps A or dt_bias");
    if (n == 0) return SDM_OK;
    if ((n + 255) / 256 > 0x7fffffff) return fail(SDM_ERR_UNSUPPORTED, "B*T*H too large for one launch");
    sdm::GateArgs G{a_raw, b_raw, A, dt_bias, a, b, n, (int)d->H};
    hipError_t e = sdm::launch_gates(G, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_gates launch");
}

sdm_status sdm_output_norm_gate(const float *o, const void *g, const float *gamma, float eps, const sdm_dims *d,
                                void *y, sdm_stream_t stream)
{
    if (!d) return fail(SDM_ERR_INVALID_ARG, "dims is NULL");
    if (d->reserved != 0) return fail(SDM_ERR_INVALID_ARG, "dims.reserved must be 0");
    if (d->B < 0 || d->T < 0 || d->H < 1 || d->d_v < 1)
        return fail(SDM_ERR_INVALID_ARG, "need B >= 0, T >= 0, H >= 1, d_v >= 1");
    if (d->in_dtype != SDM_F32 && d->in_dtype != SDM_BF16)
        return fail(SDM_ERR_INVALID_ARG, "in_dtype must be SDM_F32 or SDM_BF16");
    if (d->d_v % 32 != 0 || d->d_v > kMaxDv)
        return fail(SDM_ERR_UNSUPPORTED, "d_v must be a multiple of 32 and <= %lld", (long long)kMaxDv);
    if (!(eps >= 0.0f) || !(eps <= 3.4e38f)) return fail(SDM_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (d->B * d->T == 0) return SDM_OK;
    if (!o || !g || !gamma || !y) return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    const size_t gal = d->in_dtype == SDM_BF16 ? 8 : 16;
    if (!aligned(o, 16) || !aligned(gamma, 16) || !aligned(g, gal) || !aligned(y, gal))
        return fail(SDM_ERR_INVALID_ARG, "o and gamma must be 16-byte aligned, g and y %zu-byte aligned", gal);
    const int64_t rows = d->B * d->T * d->H;
    const size_t ob = sizeof(float) * (size_t)(rows * d->d_v), gb = in_size(d) * (size_t)(rows * d->d_v);
    if (overlap(y, gb, o, ob) || overlap(y, gb, g, gb) || overlap(y, gb, gamma, sizeof(float) * (size_t)d->d_v))
        return fail(SDM_ERR_INVALID_ARG, "y overlaps an input");
    if (rows == 0) return SDM_OK;
    if ((rows + 31) / 32 > 0x7fffffff) return fail(SDM_ERR_UNSUPPORTED, "B*T*H too large for one launch");
    sdm::NormArgs A{o, g, gamma, y, rows, (int)d->d_v, eps};
    hipError_t e = sdm::launch_out_norm_gate(A, d->in_dtype == SDM_BF16, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_output_norm_gate launch");
}

size_t sdm_gates_backward_workspace_size(const sdm_dims *d)
{
    if (!d || d->reserved != 0 || d->B < 0 || d->T < 0 || d->H < 1 || d->H > 0x7fffffff) return 0;
    const sdm::GateBwdLayout L = sdm::gates_bwd_layout(d->B * d->T, d->H);
    return d->B * d->T == 0 ? 0 : sizeof(float) * 2 * (size_t)L.parts * (size_t)d->H;
}

sdm_status sdm_gates_backward(const float *a_raw, const float *b_raw, const float *A, const float *dt_bias,
                              const float *da, const float *db, const sdm_dims *d, float *da_raw, float *db_raw,
                              float *dA, float *ddt_bias, void *workspace, size_t workspace_bytes,
                              sdm_stream_t stream)
{
    if (!d) return fail(SDM_ERR_INVALID_ARG, "dims is NULL");
    if (d->reserved != 0) return fail(SDM_ERR_INVALID_ARG, "dims.reserved must be 0");
    if (d->B < 0 || d->T < 0 || d->H < 1)
        return fail(SDM_ERR_INVALID_ARG, "need B >= 0, T >= 0, H >= 1");
    if (d->H > 0x7fffffff) return fail(SDM_ERR_UNSUPPORTED, "H too large");
    if (d->B * d->T == 0) return SDM_OK;
    const void *ins[6] = {a_raw, b_raw, A, dt_bias, da, db};
    void *outs[5] = {da_raw, db_raw, dA, ddt_bias, workspace};
    for (const void *p : ins)
        if (!p || !aligned(p, 4)) return fail(SDM_ERR_INVALID_ARG, "NULL or misaligned input");
    for (const void *p : outs)
        if (!p || !aligned(p, 4)) return fail(SDM_ERR_INVALID_ARG, "NULL or misaligned output or workspace");
    const size_t need = sdm_gates_backward_workspace_size(d);
    if (workspace_bytes < need)
        return fail(SDM_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    const int64_t n = d->B * d->T * d->H;
    const size_t nb = sizeof(float) * (size_t)n, hb = sizeof(float) * (size_t)d->H;
    const size_t isz[6] = {nb, nb, hb, hb, nb, nb}, osz[5] = {nb, nb, hb, hb, need};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], osz[i], ins[j], isz[j])) return fail(SDM_ERR_INVALID_ARG, "an output overlaps an input");
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], osz[i], outs[j], osz[j]))
                return fail(SDM_ERR_INVALID_ARG, "outputs (or the workspace) overlap");
    }
    sdm::GateBwdArgs G{a_raw, b_raw, A, dt_bias, da, db, da_raw, db_raw, dA, ddt_bias,
                       static_cast<float *>(workspace), n, d->H};
    hipError_t e = sdm::launch_gates_backward(G, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_gates_backward launch");
}

static bool norm_dims_ok(const sdm_dims *d)
{
    return d && d->reserved == 0 && d->B >= 0 && d->T >= 0 && d->H >= 1 && d->d_v >= 1 && d->d_v % 32 == 0 &&
           d->d_v <= kMaxDv && (d->in_dtype == SDM_F32 || d->in_dtype == SDM_BF16);
}

size_t sdm_output_norm_gate_backward_workspace_size(const sdm_dims *d)
{
    if (!norm_dims_ok(d)) return 0;
    const int64_t rows = d->B * d->T * d->H;
    return sizeof(float) * (size_t)sdm::norm_bwd_blocks(rows) * (size_t)d->d_v;
}

sdm_status sdm_output_norm_gate_backward(const float *o, const void *g, const float *gamma, float eps,
                                         const float *dy, const sdm_dims *d, float *dout, float *dg,
                                         float *dgamma, void *workspace, size_t workspace_bytes,
                                         sdm_stream_t stream)
{
    if (!d) return fail(SDM_ERR_INVALID_ARG, "dims is NULL");
    if (d->reserved != 0) return fail(SDM_ERR_INVALID_ARG, "dims.reserved must be 0");
    if (d->B < 0 || d->T < 0 || d->H < 1 || d->d_v < 1)
        return fail(SDM_ERR_INVALID_ARG, "need B >= 0, T >= 0, H >= 1, d_v >= 1");
    if (d->in_dtype != SDM_F32 && d->in_dtype != SDM_BF16)
        return fail(SDM_ERR_INVALID_ARG, "in_dtype must be SDM_F32 or SDM_BF16");
    if (d->d_v % 32 != 0 || d->d_v > kMaxDv)
        return fail(SDM_ERR_UNSUPPORTED, "d_v must be a multiple of 32 and <= %lld", (long long)kMaxDv);
    if (!(eps >= 0.0f) || !(eps <= 3.4e38f)) return fail(SDM_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (d->B * d->T == 0) return SDM_OK;
    if (!o || !g || !gamma || !dy || !dout || !dg || !dgamma || !workspace)
        return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    const size_t gal = d->in_dtype == SDM_BF16 ? 8 : 16;
    if (!aligned(o, 16) || !aligned(gamma, 16) || !aligned(g, gal) || !aligned(dy, 16) || !aligned(dout, 16) ||
        !aligned(dg, 16) || !aligned(dgamma, 4) || !aligned(workspace, 16))
        return fail(SDM_ERR_INVALID_ARG, "o, gamma, dy, dout, dg and the workspace must be 16-byte aligned, g %zu-byte",
                    gal);
    const int64_t rows = d->B * d->T * d->H;
    const size_t need = sdm_output_norm_gate_backward_workspace_size(d);
    if (workspace_bytes < need)
        return fail(SDM_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    const size_t ob = sizeof(float) * (size_t)(rows * d->d_v), gb = in_size(d) * (size_t)(rows * d->d_v);
    const size_t vb = sizeof(float) * (size_t)d->d_v;
    const void *ins[4] = {o, g, gamma, dy};
    const size_t isz[4] = {ob, gb, vb, ob};
    const void *outs[4] = {dout, dg, dgamma, workspace};
    const size_t osz[4] = {ob, ob, vb, need};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j)
            if (overlap(outs[i], osz[i], ins[j], isz[j])) return fail(SDM_ERR_INVALID_ARG, "an output overlaps an input");
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], osz[i], outs[j], osz[j]))
                return fail(SDM_ERR_INVALID_ARG, "outputs (or the workspace) overlap");
    }
    sdm::NormBwdArgs A{o, g, gamma, dy, dout, dg, dgamma, static_cast<float *>(workspace), rows, (int)d->d_v, eps};
    hipError_t e = sdm::launch_out_norm_gate_backward(A, d->in_dtype == SDM_BF16, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_output_norm_gate_backward launch");
}

sdm_status sdm_gdn_dense_forward(float *S, const void *k, const void *q, const void *v, const float *a,
                                 const float *b, float *o, const sdm_dims *d, sdm_stream_t stream)
{
    if (!d) return fail(SDM_ERR_INVALID_ARG, "dims is NULL");
    if (d->reserved != 0) return fail(SDM_ERR_INVALID_ARG, "dims.reserved must be 0");
    if (d->B < 0 || d->T < 0 || d->H < 1 || d->d_k < 1 || d->d_v < 1)
        return fail(SDM_ERR_INVALID_ARG, "need B >= 0, T >= 0, H >= 1, d_k >= 1, d_v >= 1");
    if (d->in_dtype != SDM_F32 && d->in_dtype != SDM_BF16)
        return fail(SDM_ERR_INVALID_ARG, "in_dtype must be SDM_F32 or SDM_BF16");
    if (d->d_k != 16 && d->d_k != 32 && d->d_k != 64 && d->d_k != 128 && d->d_k != 256)
        return fail(SDM_ERR_UNSUPPORTED, "d_k must be 16, 32, 64, 128 or 256 (got %lld)", (long long)d->d_k);
    if (d->d_v > (1 << 20) || d->H > (1 << 20)) return fail(SDM_ERR_UNSUPPORTED, "H and d_v must be <= 2^20");
    if (d->B * d->T == 0) return SDM_OK;
    if (!S || !k || !q || !v || !a || !b || !o) return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(k, 16) || !aligned(q, 16) || !aligned(S, 4) || !aligned(o, 4) || !aligned(a, 4) || !aligned(b, 4) ||
        !aligned(v, in_size(d)))
        return fail(SDM_ERR_INVALID_ARG, "k and q must be 16-byte aligned, the other arrays element-aligned");
    const int64_t rows = d->B * d->T * d->H;
    const size_t sb = sizeof(float) * (size_t)(d->B * d->H * d->d_k * d->d_v);
    const size_t ob = sizeof(float) * (size_t)(rows * d->d_v);
    if (overlap(o, ob, S, sb)) return fail(SDM_ERR_INVALID_ARG, "o overlaps S");
    if (overlap(S, sb, k, in_size(d) * (size_t)(rows * d->d_k)) || overlap(S, sb, q, in_size(d) * (size_t)(rows * d->d_k)) ||
        overlap(S, sb, v, in_size(d) * (size_t)(rows * d->d_v)) || overlap(o, ob, k, in_size(d) * (size_t)(rows * d->d_k)) ||
        overlap(o, ob, q, in_size(d) * (size_t)(rows * d->d_k)) || overlap(o, ob, v, in_size(d) * (size_t)(rows * d->d_v)))
        return fail(SDM_ERR_INVALID_ARG, "S or o overlaps an input");
    if (d->B * d->H * ((d->d_v + 15) / 16) > 0x7fffffff) return fail(SDM_ERR_UNSUPPORTED, "B*H*d_v too large");
    sdm::GdnArgs A{S, k, q, v, a, b, o, d->B, d->T, (int)d->H, (int)d->d_k, (int)d->d_v};
    hipError_t e = sdm::launch_gdn_dense(A, d->in_dtype == SDM_BF16, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_gdn_dense_forward launch");
}

size_t sdm_scan_backward_workspace_size(const sdm_dims *d)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1 || d->W < 1 || d->R < 1 || d->W > kMaxList || d->R > kMaxList ||
        d->d_v < 32 || d->d_v % 32 != 0 || d->d_v > 256 || (d->in_dtype != SDM_F32 && d->in_dtype != SDM_BF16))
        return 0;
    return sdm::scan_bwd_workspace_bytes(d->B, d->T, d->H, (int)d->W, (int)d->R, (int)d->d_v,
                                         d->in_dtype == SDM_BF16);
}

sdm_status sdm_scan_backward(float *dM, const int32_t *widx, const float *wwt, const int32_t *ridx, const float *rwt,
                             const void *v, const float *a, const float *b, const float *dout, const float *xsave,
                             const float *zsave, float *dv, float *da, float *db, float *dw, float *dr,
                             void *workspace, size_t workspace_bytes, const sdm_dims *d, sdm_stream_t stream)
{
    sdm_status st = check_memory_dims(d);
    if (st != SDM_OK) return st;
    if (d->T < 0) return fail(SDM_ERR_INVALID_ARG, "T must be >= 0");
    if (d->in_dtype != SDM_F32 && d->in_dtype != SDM_BF16)
        return fail(SDM_ERR_INVALID_ARG, "in_dtype must be SDM_F32 or SDM_BF16");
    if (d->W < 1 || d->R < 1) return fail(SDM_ERR_INVALID_ARG, "need W, R >= 1");
    if (d->W > kMaxList || d->R > kMaxList)
        return fail(SDM_ERR_UNSUPPORTED, "W and R must be <= %lld", (long long)kMaxList);
    if (d->d_v > 256) return fail(SDM_ERR_UNSUPPORTED, "the backward scan needs d_v <= 256");
    if (d->B * d->T == 0) return SDM_OK;
    if (!dM || !widx || !wwt || !ridx || !rwt || !v || !a || !b || !dout || !xsave || !zsave || !dv || !da || !db ||
        !dw || !dr)
        return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(dM, 16) || !aligned(dout, 16) || !aligned(xsave, 16) || !aligned(zsave, 16) || !aligned(dv, 16) ||
        !aligned(v, d->in_dtype == SDM_BF16 ? 8 : 16))
        return fail(SDM_ERR_INVALID_ARG, "dM, dout, xsave, zsave and dv must be 16-byte aligned, v 8 (bf16) or 16");
    if (!aligned(widx, 4) || !aligned(wwt, 4) || !aligned(ridx, 4) || !aligned(rwt, 4) || !aligned(a, 4) ||
        !aligned(b, 4) || !aligned(da, 4) || !aligned(db, 4) || !aligned(dw, 4) || !aligned(dr, 4))
        return fail(SDM_ERR_INVALID_ARG, "index, weight, gate and gradient arrays must be 4-byte aligned");
    const int64_t N = d->n_sub * d->n_sub, rows = d->B * d->T * d->H;
    const size_t msz = sizeof(float) * (size_t)(d->B * d->H * N * d->d_v);
    const size_t vsz = sizeof(float) * (size_t)(rows * d->d_v);
    const size_t outs[5] = {vsz, sizeof(float) * (size_t)rows, sizeof(float) * (size_t)rows,
                            sizeof(float) * (size_t)(rows * d->W), sizeof(float) * (size_t)(rows * d->R)};
    const void *optr[5] = {dv, da, db, dw, dr};
    for (int i = 0; i < 5; ++i) {
        if (overlap(optr[i], outs[i], dM, msz)) return fail(SDM_ERR_INVALID_ARG, "a gradient output overlaps dM");
        for (int k = 0; k < i; ++k)
            if (overlap(optr[i], outs[i], optr[k], outs[k])) return fail(SDM_ERR_INVALID_ARG, "gradient outputs overlap");
    }
    // dM and the gradient outputs are written while the inputs are read
    const size_t lw = 4 * (size_t)(rows * d->W), lr = 4 * (size_t)(rows * d->R);
    const void *iptr[10] = {widx, wwt, ridx, rwt, v, a, b, dout, xsave, zsave};
    const size_t isz[10] = {lw, lw, lr, lr, in_size(d) * (size_t)(rows * d->d_v), 4 * (size_t)rows,
                            4 * (size_t)rows, vsz, 4 * (size_t)(rows * d->W * d->d_v),
                            4 * (size_t)(rows * d->R * d->d_v)};
    for (int j = 0; j < 10; ++j) {
        if (overlap(dM, msz, iptr[j], isz[j])) return fail(SDM_ERR_INVALID_ARG, "dM overlaps an input");
        for (int i = 0; i < 5; ++i)
            if (overlap(optr[i], outs[i], iptr[j], isz[j]))
                return fail(SDM_ERR_INVALID_ARG, "a gradient output overlaps an input");
    }
    const bool bf16 = d->in_dtype == SDM_BF16;
    // no workspace at all: the token-serial kernels (no workspace needed)
    const size_t need = (!workspace && workspace_bytes == 0)
                            ? 0
                            : sdm::scan_bwd_workspace_bytes(d->B, d->T, d->H, (int)d->W, (int)d->R, (int)d->d_v, bf16);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(SDM_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
        if (!aligned(workspace, 16)) return fail(SDM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
        // the workspace is written while the inputs are read and the outputs written
        if (overlap(workspace, need, dM, msz)) return fail(SDM_ERR_INVALID_ARG, "the workspace overlaps dM");
        for (int i = 0; i < 5; ++i)
            if (overlap(workspace, need, optr[i], outs[i]))
                return fail(SDM_ERR_INVALID_ARG, "the workspace overlaps a gradient output");
        for (int j = 0; j < 10; ++j)
            if (overlap(workspace, need, iptr[j], isz[j]))
                return fail(SDM_ERR_INVALID_ARG, "the workspace overlaps an input");
    }
    sdm::BwdArgs A{dM, widx, ridx, wwt, rwt, v, a, b, dout, xsave, zsave, dv, da, db, dw, dr,
                   d->B, d->T, (int)d->H, (int)N, (int)d->d_v, (int)d->W, (int)d->R};
    hipError_t e = need > 0 ? sdm::launch_scan_backward_lanes(A, bf16, workspace, as_stream(stream))
                            : sdm::launch_scan_backward(A, bf16, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_scan_backward launch");
}

size_t sdm_address_backward_workspace_size(const sdm_dims *d)
{
    if (!d || d->B < 0 || d->T < 0 || d->H < 1 || d->W < 1 || d->R < 1 || d->d_k < 2 || (d->d_k & 1) ||
        d->n_sub < 1 || d->W > kMaxList || d->R > kMaxList || d->d_k > 512)
        return 0;
    return sdm::address_bwd_workspace_bytes(d->B, d->T, d->H, (int)d->W, (int)d->R, (int)d->n_sub, (int)(d->d_k / 2));
}

sdm_status sdm_address_backward(const void *k, const void *q, const void *C_w, const void *C_r,
                                const int32_t *widx, const float *wwt, const int32_t *ridx, const float *rwt,
                                const float *dw, const float *dr, const sdm_dims *d, float *dk, float *dq,
                                float *dC_w, float *dC_r, void *workspace, size_t workspace_bytes,
                                sdm_stream_t stream)
{
    sdm_status st = check_method_dims(d, true);
    if (st != SDM_OK) return st;
    if (d->B * d->T == 0) return SDM_OK;
    if (!k || !q || !C_w || !C_r || !widx || !wwt || !ridx || !rwt || !dw || !dr || !dk || !dq || !dC_w || !dC_r)
        return fail(SDM_ERR_INVALID_ARG, "NULL pointer argument");
    const size_t ial = in_size(d);
    if (!aligned(k, ial) || !aligned(q, ial) || !aligned(C_w, ial) || !aligned(C_r, ial) || !aligned(widx, 4) ||
        !aligned(wwt, 4) || !aligned(ridx, 4) || !aligned(rwt, 4) || !aligned(dw, 4) || !aligned(dr, 4) ||
        !aligned(dk, 4) || !aligned(dq, 4) || !aligned(dC_w, 4) || !aligned(dC_r, 4) || !aligned(workspace, 16))
        return fail(SDM_ERR_INVALID_ARG, "misaligned argument");
    const int64_t rows = d->B * d->T * d->H;
    // token-head rows and the list entries of one (kind, head) are indexed with int32
    if (rows > 0x7fffffff || d->B * d->T * (d->W > d->R ? d->W : d->R) > 0x7fffffff ||
        d->H * d->n_sub * d->d_k > 0x7fffffff)
        return fail(SDM_ERR_UNSUPPORTED, "B*T*H, B*T*max(W, R) and the codebook size must be < 2^31");
    const size_t need = sdm::address_bwd_workspace_bytes(d->B, d->T, d->H, (int)d->W, (int)d->R, (int)d->n_sub,
                                                         (int)(d->d_k / 2));
    if (!workspace || workspace_bytes < need)
        return fail(SDM_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    const size_t xb = sizeof(float) * (size_t)(rows * d->d_k);
    const size_t cb = sizeof(float) * (size_t)(d->H * 2 * d->n_sub * (d->d_k / 2));
    const void *outs[4] = {dk, dq, dC_w, dC_r};
    const size_t osz[4] = {xb, xb, cb, cb};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], osz[i], workspace, need)) return fail(SDM_ERR_INVALID_ARG, "an output overlaps the workspace");
        for (int j = 0; j < i; ++j)
            if (!(i == 3 && j == 2 && dC_w == dC_r) && overlap(outs[i], osz[i], outs[j], osz[j]))
                return fail(SDM_ERR_INVALID_ARG, "outputs overlap (only dC_w and dC_r may be the same buffer)");
    }
    // the outputs and the workspace are written while the inputs are read
    const size_t ib = ial * (size_t)(rows * d->d_k), icb = ial * (size_t)(d->H * 2 * d->n_sub * (d->d_k / 2));
    const size_t lw = 4 * (size_t)(rows * d->W), lr = 4 * (size_t)(rows * d->R);
    const void *ins[10] = {k, q, C_w, C_r, widx, wwt, ridx, rwt, dw, dr};
    const size_t isz[10] = {ib, ib, icb, icb, lw, lw, lr, lr, lw, lr};
    for (int j = 0; j < 10; ++j) {
        if (overlap(workspace, need, ins[j], isz[j])) return fail(SDM_ERR_INVALID_ARG, "the workspace overlaps an input");
        for (int i = 0; i < 4; ++i)
            if (overlap(outs[i], osz[i], ins[j], isz[j])) return fail(SDM_ERR_INVALID_ARG, "an output overlaps an input");
    }
    sdm::AddrBwdArgs A{k, q, C_w, C_r, widx, ridx, wwt, rwt, dw, dr, dk, dq, dC_w, dC_r, rows, (int)d->H,
                       (int)d->d_k, (int)d->n_sub, (int)d->W, (int)d->R};
    hipError_t e = sdm::launch_address_backward(A, d->in_dtype == SDM_BF16, workspace, as_stream(stream));
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_address_backward launch");
}

}  // extern "C"
