// lanes_common.h -- pieces shared by the lane-parallel scans (the forward in
// sdm_scan_lanes.hip, its backward in sdm_scan_bwd_lanes.hip): the buffer
// offset conventions of the preparation streams, exact vmcnt waits, LDS reads
// that wait for themselves, and the XCD-aware workgroup placement.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace sdm {
namespace lanes {

constexpr uint32_t kOOB = 0x80000000u;       // past every buffer range used here (all < 2 GiB)
constexpr uint32_t kRowBias = 0x40000000u;   // row offsets are stored plus this (0: no row)

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int K>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(K >= 0 && K <= 63, "vmcnt out of range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
}

template <class T>
__device__ __forceinline__ uint32_t lds_addr(const T *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T *)p;
}

// LDS reads written as asm blocks that wait for their own results: the
// compiler would otherwise wait for every outstanding LDS-destination load
// before an LDS read it cannot tell apart from their targets.
__device__ __forceinline__ void lds_read2(f32x4 &x, f32x4 &y, uint32_t ax, uint32_t ay)
{
    asm volatile("ds_read_b128 %0, %2\n\t"
                 "ds_read_b128 %1, %3\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(x), "=&v"(y)
                 : "v"(ax), "v"(ay)
                 : "memory");
}

__device__ __forceinline__ f32x4 lds_read16(uint32_t addr)
{
    f32x4 x;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(addr) : "memory");
    return x;
}

// (group, member) of workgroup `id` for ngroups groups of nmem members, such
// that all members of a group run on the same XCD (workgroup ids are dealt to
// the 8 XCDs round-robin).  Groups past the last multiple of 8 take plain order.
__device__ __forceinline__ void xcd_decode(uint32_t id, uint32_t ngroups, uint32_t nmem, uint32_t &group,
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

}  // namespace lanes
}  // namespace sdm
