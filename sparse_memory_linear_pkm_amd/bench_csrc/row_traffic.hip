// row_traffic.hip -- the memory-access pattern of the prefill scan without
// its arithmetic, for measuring what the MI355X delivers for it.
//
// Built into libsdm_bench.so (measurement only; not part of the SDM library).
// The scan of "Sparse Delta Memory: Scaling the State of Linear RNNs through
// Sparsity" (Sec. 3.1, Eq. 4) gathers, per token, W rows to update and R
// rows to read from an HBM-resident slot table and writes the W rows back;
// the blog summary "Sparse Delta Memory: Scaling Linear RNN States to 1M
// Tokens via Sparsity" (Critical Analysis & Hardware Realities) names these
// gathers and scatters as the hard part.  This kernel issues exactly that
// traffic in the scan's form -- workgroups of G waves own one G*16-byte
// segment of every row of one chain, each wave moves 64/G rows per kind and
// step with one 16-byte LDS-destination buffer load per lane, D steps are in
// flight, and the write rows' segments are stored back from LDS -- with row
// indices drawn by a hash instead of slot lists, and no arithmetic between
// the load and the store.  With P > 1 token groups a workgroup runs P such
// streams of independent rows on the same segment (P times the waves and the
// rows in flight per CU).  Two variants isolate what the rate depends on: the
// gathers alone (every store goes past the buffer range, so it is issued but
// moves nothing), and the gathers with another cache policy (non-temporal, or
// device scope, which bypasses the CU's vector L1).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

[[maybe_unused]] constexpr int kWave = 64;   // (used by the device pass only)
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t mix(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// (group, member) of workgroup `id` for ngroups groups of nmem members, such
// that the members of a group -- the workgroups whose segments share one
// 128-byte line -- run on the same XCD (ids are dealt to the 8 XCDs
// round-robin), so that its L2 fetches each line once: the scan's placement.
__device__ __forceinline__ void xcd_place(uint32_t id, uint32_t ngroups, uint32_t nmem, uint32_t &group,
                                          uint32_t &member)
{
    constexpr uint32_t kX = 8;
    const uint32_t full = ngroups / kX;
    const uint32_t per_xcd = full * nmem;
    const uint32_t k = id / kX;
    if (k < per_xcd) {
        group = (k / nmem) * kX + id % kX;
        member = k % nmem;
    } else {
        const uint32_t rest = id - per_xcd * kX;
        group = full * kX + rest / nmem;
        member = rest % nmem;
    }
}

template <int K>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
}

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// grid: chains * (row_bytes / (16 G)) workgroups of G * P waves (P token
// groups of G waves, each group moving its own rows); rows per chain must be
// a power of two.
// LA: cache-policy bits of the gathers (0, 2 = nt, 17 = sc0 sc1); ST: the
// write rows are stored (else the stores go past the range).
template <int G, int P, int D, int LA, bool ST>
__global__ void __launch_bounds__(64 * G * P) row_traffic_kernel(float *M, uint32_t nrows_log2, uint32_t row_bytes,
                                                                 uint32_t steps, uint32_t seed)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int RPW = kWave / G;
    constexpr int NVM = 3;   // two gathers and one store per step
    __shared__ f32x4 gath_all[P][D][2][kWave][G];
    const uint32_t nline = row_bytes / 128u;   // 128-byte lines per row
    uint32_t grp, part;
    xcd_place(blockIdx.x, (uint32_t)gridDim.x / (8u / G), 8u / G, grp, part);
    const uint32_t chain = grp / nline, seg = (grp % nline) * (8u / G) + part;
    const int wave_all = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int tg = wave_all / G, wave = wave_all % G;   // token group, wave within it
    auto &gath = gath_all[tg];
    const int lane = (int)(threadIdx.x & 63);
    const uint32_t rr = (uint32_t)(wave * RPW + lane / G);   // row of the step this lane moves
    const uint32_t piece = (uint32_t)(lane % G);
    const uint32_t chain_bytes = row_bytes << nrows_log2;   // < 2^31 (checked on the host)
    const __amdgpu_buffer_rsrc_t Mrs = rsrc(reinterpret_cast<unsigned char *>(M) + (size_t)chain * chain_bytes,
                                            chain_bytes);
    const uint32_t rmask = (1u << nrows_log2) - 1u;
    const uint32_t col = seg * 16u * G + piece * 16u;
    auto offset = [&](uint32_t step, uint32_t kind) {
        const uint32_t row = mix(seed ^ mix(chain * 0x9E3779B1u + step * 0x85EBCA6Bu + (rr * 2u + kind + 1024u * (uint32_t)tg) * 0xC2B2AE35u)) &
                             rmask;
        return row * row_bytes + col;
    };
    uint32_t ofw[D];
    auto gathers = [&](int sl, uint32_t step) __attribute__((always_inline)) {
        const uint32_t ow = offset(step, 0u), orr = offset(step, 1u);
        ofw[sl] = step < steps ? ow : 0x80000000u;   // past the range: dropped
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            Mrs, (__attribute__((address_space(3))) void *)&gath[sl][0][wave * RPW][0], 16,
            step < steps ? ow : 0x80000000u, 0, 0, LA);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            Mrs, (__attribute__((address_space(3))) void *)&gath[sl][1][wave * RPW][0], 16,
            step < steps ? orr : 0x80000000u, 0, 0, LA);
    };
    static_for<0, D>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        gathers(s, (uint32_t)s);
        // keep the store count per step fixed: one store past the range
        __builtin_amdgcn_raw_buffer_store_b128((f32x4){0.f, 0.f, 0.f, 0.f}, Mrs, 0x80000000u, 0, 0);
    });
    for (uint32_t s0 = 0; s0 < steps; s0 += D) {
        static_for<0, D>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            const uint32_t step = s0 + s;
            wait_vmcnt<(D - 1) * NVM>();
            f32x4 x;
            asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(x)
                         : "v"((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) f32x4 *)&gath[s][0][rr][piece])
                         : "memory");
            __builtin_amdgcn_raw_buffer_store_b128(x, Mrs, ST ? ofw[s] : 0x80000000u, 0, 0);
            gathers(s, step + D);
        });
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
#endif
}

template <int G, int P, int LA = 0, bool ST = true>
hipError_t launch_g(float *M, int64_t chains, int nrows_log2, int row_bytes, int64_t steps, uint32_t seed,
                    hipStream_t st)
{
    const int64_t wgs = chains * (row_bytes / (16 * G));
    hipLaunchKernelGGL((row_traffic_kernel<G, P, 4, LA, ST>), dim3((unsigned)wgs), dim3(64 * G * P), 0, st, M,
                       (uint32_t)nrows_log2, (uint32_t)row_bytes, (uint32_t)steps, seed);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// Moves `steps` scan steps of traffic over `chains` tables of 2^nrows_log2
// rows of row_bytes bytes at M (device memory, chains * rows * row_bytes
// bytes, contents overwritten with values read from it): per step and
// workgroup, 64 write rows and 64 read rows of one seg_bytes-byte segment
// are gathered and the 64 write-row segments stored back.  seg_bytes = 32,
// 64 or 128 (G = 2, 4 or 8 waves per workgroup); token_groups = P streams of
// independent rows per workgroup (1, or 4 with 32-byte and 2 with 128-byte
// segments); row_bytes a multiple of 128 (whole lines); one chain below
// 2 GiB.  variant: 0 = the scan's form; with one token group and 32- or
// 128-byte segments also 1 = gathers only (the stores go past the range),
// 2 = gathers non-temporal, 3 = gathers at device scope (L1 bypassed).
// Returns 0 or a HIP error code (-1 for invalid arguments).  Bytes moved:
// chains * row_bytes / seg_bytes * P * steps * 64 * (3, or 2 for variant 1)
// * seg_bytes.
int sdm_bench_row_traffic(float *M, int64_t chains, int nrows_log2, int row_bytes, int seg_bytes, int token_groups,
                          int variant, int64_t steps, uint32_t seed, hipStream_t stream)
{
    if (!M || chains < 1 || nrows_log2 < 6 || nrows_log2 > 24 || row_bytes < 128 || row_bytes % 128 ||
        steps < 1 || steps > (1 << 30) || ((uint64_t)row_bytes << nrows_log2) >= (1ull << 31) || variant < 0 ||
        variant > 3 || (variant != 0 && (token_groups != 1 || (seg_bytes != 32 && seg_bytes != 128))))
        return -1;
    if (variant != 0) {
        const bool g2 = seg_bytes == 32;
        switch (variant) {
        case 1: return (int)(g2 ? launch_g<2, 1, 0, false>(M, chains, nrows_log2, row_bytes, steps, seed, stream)
                                : launch_g<8, 1, 0, false>(M, chains, nrows_log2, row_bytes, steps, seed, stream));
        case 2: return (int)(g2 ? launch_g<2, 1, 2>(M, chains, nrows_log2, row_bytes, steps, seed, stream)
                                : launch_g<8, 1, 2>(M, chains, nrows_log2, row_bytes, steps, seed, stream));
        default: return (int)(g2 ? launch_g<2, 1, 17>(M, chains, nrows_log2, row_bytes, steps, seed, stream)
                                 : launch_g<8, 1, 17>(M, chains, nrows_log2, row_bytes, steps, seed, stream));
        }
    }
    switch (seg_bytes * 8 + token_groups) {
    case 32 * 8 + 1: return (int)launch_g<2, 1>(M, chains, nrows_log2, row_bytes, steps, seed, stream);
    case 32 * 8 + 4: return (int)launch_g<2, 4>(M, chains, nrows_log2, row_bytes, steps, seed, stream);
    case 64 * 8 + 1: return (int)launch_g<4, 1>(M, chains, nrows_log2, row_bytes, steps, seed, stream);
    case 128 * 8 + 1: return (int)launch_g<8, 1>(M, chains, nrows_log2, row_bytes, steps, seed, stream);
    case 128 * 8 + 2: return (int)launch_g<8, 2>(M, chains, nrows_log2, row_bytes, steps, seed, stream);
    default: return -1;
    }
}

}  // extern "C"
