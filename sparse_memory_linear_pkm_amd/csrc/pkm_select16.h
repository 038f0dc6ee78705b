// pkm_select16.h -- the prefill addressing's selections, four token rows per
// wave, sixteen lanes per row.
//
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 2 (Product-Key Memories: top-k' of each half, then the best slots of
// the k' x k' outer sum) and Sec. 4 (softmax over the selected scores).
//
// Every selection here is exact: the result is the top of the list in the
// total order (score descending, index ascending), the same lists the
// one-row routines of pkm_address.h produce (and the decode step uses), and
// the weights are computed with the same operations in the same order, so
// the prefill and the decode step give bit-identical slots and weights.
//
// Layout: lane l of a wave serves row group g = l / 16 (one token row) as
// lane c = l % 16 of that group.  A list of up to 64 values of a row lives
// in the group's 16 lanes x 4 registers (element i = 4c + r), so the
// compare-exchanges of a sort are register pairs inside a lane or lane pairs
// inside a 16-lane DPP row (quad_perm, row_ror, row_mirror, bank-masked
// row_shl/row_shr); the four rows of a wave never exchange data.
//
// Selection of the n best of a row's candidates (n <= 64):
//   1. group maxima: every lane folds its candidates into 4 running maxima
//      (64 per row); tau = the n-th largest of them, found by sorting the 64,
//      or for n <= 32 (when every maximum is a real candidate) the 32nd
//      largest, found with a shorter network (tau32_top).  At least n
//      candidates reach tau (one per group maximum above it), so the n best
//      all do.  (A later part of a half split in parts instead takes the n-th
//      best score of the earlier parts as tau.)
//   2. the candidates that reach tau (typically 1.1-1.4 x 32) are compacted into
//      a per-row LDS buffer (a per-lane bit mask, a prefix sum of the lanes'
//      counts over the row group's DPP row, then the set bits);
//   3. the survivors are sorted as 32-bit keys: the score bits above tau,
//      shifted right just enough to leave room for the index in the low
//      bits.  Where the shift drops bits, two different scores can share a
//      key prefix; the sorted list is then checked pair by pair against the
//      full (score, index) order.  A row with a misordered pair, or with more
//      than 64 survivors, is redone by the one-row exact routine.
#pragma once

#include "device_common.h"
#include "pkm_address.h"

namespace sdm {

constexpr int kGroupLanes = 16;

// x of lane (c ^ M) of the same 16-lane row, M in {1, 2, 3, 4, 7, 8, 15}.
template <int M>
__device__ __forceinline__ uint32_t row_xor(uint32_t x)
{
    const int xi = (int)x;
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    } else if constexpr (M == 3) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x1B, 0xF, 0xF, false);    // quad_perm [3,2,1,0]
    } else if constexpr (M == 4) {
        // banks 0 and 2 (lanes 0-3, 8-11) read 4 lanes up, banks 1 and 3 read 4 lanes down
        const int up = __builtin_amdgcn_update_dpp(xi, xi, 0x104, 0xF, 0x5, false);    // row_shl:4
        return (uint32_t)__builtin_amdgcn_update_dpp(up, xi, 0x114, 0xF, 0xA, false);  // row_shr:4
    } else if constexpr (M == 7) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x141, 0xF, 0xF, false);   // row_half_mirror
    } else if constexpr (M == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x128, 0xF, 0xF, false);   // row_ror:8
    } else {
        static_assert(M == 15, "lane distance within a row");
        return (uint32_t)__builtin_amdgcn_mov_dpp(xi, 0x140, 0xF, 0xF, false);   // row_mirror
    }
}

// One compare-exchange stage of the list x (element i = 4c + r): i and
// i ^ M are compared and the lower index keeps the larger value.
template <int M>
__device__ __forceinline__ void cmpx_stage(uint32_t (&x)[4])
{
    constexpr int HB = M >= 32 ? 32 : M >= 16 ? 16 : M >= 8 ? 8 : M >= 4 ? 4 : M >= 2 ? 2 : 1;   // highest bit of M
    constexpr int LM = M >> 2, RM = M & 3;
    if constexpr (LM == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if ((r & HB) == 0) {
                const uint32_t a = x[r], b = x[r ^ RM];
                x[r] = a > b ? a : b;
                x[r ^ RM] = a > b ? b : a;
            }
        }
    } else {
        // the lower lane of a pair keeps the larger value: med3(x, y, m) with
        // m = all ones there and 0 in the upper lane (one v_med3_u32 instead
        // of a max, a min and a select)
        const uint32_t m = (lane_id() & (HB >> 2)) == 0 ? 0xFFFFFFFFu : 0u;
        // (the exchanges read the registers in the order the previous stage
        // wrote them, so that a DPP read rarely waits on a fresh VALU write)
        uint32_t y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q ^ RM] = row_xor<LM>(x[q]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t hi = x[r] > y[r] ? x[r] : y[r], lo = x[r] > y[r] ? y[r] : x[r];
            const uint32_t c = hi < m ? hi : m;
            x[r] = c > lo ? c : lo;
        }
    }
}

// Sorts each 16-lane row's 64 values (lanes x 4 registers) descending: a
// bitonic network whose merges start with a flip (i against i ^ (K - 1)),
// so that every comparator points the same way.
__device__ __forceinline__ void sort64_desc(uint32_t (&x)[4])
{
    cmpx_stage<1>(x);
    cmpx_stage<3>(x); cmpx_stage<1>(x);
    cmpx_stage<7>(x); cmpx_stage<2>(x); cmpx_stage<1>(x);
    cmpx_stage<15>(x); cmpx_stage<4>(x); cmpx_stage<2>(x); cmpx_stage<1>(x);
    cmpx_stage<31>(x); cmpx_stage<8>(x); cmpx_stage<4>(x); cmpx_stage<2>(x); cmpx_stage<1>(x);
    cmpx_stage<63>(x); cmpx_stage<16>(x); cmpx_stage<8>(x); cmpx_stage<4>(x); cmpx_stage<2>(x); cmpx_stage<1>(x);
}

// The 32nd largest (tau) and the largest (top) of each 16-lane row's 64
// values, in every lane of the row (x is overwritten).  The two halves of 32
// (lanes 0-7, lanes 8-15) are sorted descending, then element i is compared
// with element 63 - i: the larger of each pair are the 32 largest of the 64
// (a bitonic half-cleaner), and every lane holds such a pair, lanes c and
// 15 - c the same ones.  So the minimum and maximum over each half of the
// row's lanes are the 32nd largest and the largest: the last five stages of
// a full sort and the readout of ranks are not needed.
__device__ __forceinline__ void tau32_top(uint32_t (&x)[4], uint32_t &tau, uint32_t &top)
{
    cmpx_stage<1>(x);
    cmpx_stage<3>(x); cmpx_stage<1>(x);
    cmpx_stage<7>(x); cmpx_stage<2>(x); cmpx_stage<1>(x);
    cmpx_stage<15>(x); cmpx_stage<4>(x); cmpx_stage<2>(x); cmpx_stage<1>(x);
    cmpx_stage<31>(x); cmpx_stage<8>(x); cmpx_stage<4>(x); cmpx_stage<2>(x); cmpx_stage<1>(x);
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t y = row_xor<15>(x[3 - r]);   // element 63 - (4c + r)
        const uint32_t mx = x[r] > y ? x[r] : y;
        lo = mx < lo ? mx : lo;
        hi = mx > hi ? mx : hi;
    }
    uint32_t t;
    t = row_xor<1>(lo); lo = t < lo ? t : lo;
    t = row_xor<1>(hi); hi = t > hi ? t : hi;
    t = row_xor<2>(lo); lo = t < lo ? t : lo;
    t = row_xor<2>(hi); hi = t > hi ? t : hi;
    t = row_xor<4>(lo); lo = t < lo ? t : lo;
    t = row_xor<4>(hi); hi = t > hi ? t : hi;
    tau = lo;
    top = hi;
}

// The value lane 16 g + c0 (c0 uniform) holds, in every lane of row group g
// (four readlanes and a select: no LDS round trip).
__device__ __forceinline__ uint32_t row_lane_value(uint32_t v, int c0)
{
    const uint32_t v0 = (uint32_t)__builtin_amdgcn_readlane((int)v, c0);
    const uint32_t v1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16 + c0);
    const uint32_t v2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32 + c0);
    const uint32_t v3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48 + c0);
    const int g = lane_id() >> 4;
    return g == 0 ? v0 : g == 1 ? v1 : g == 2 ? v2 : v3;
}

// The element of rank j (uniform) of a sorted row list, in every lane of the row.
__device__ __forceinline__ uint32_t rank_value(const uint32_t (&x)[4], int j)
{
    const int r = j & 3;
    const uint32_t v = r == 0 ? x[0] : r == 1 ? x[1] : r == 2 ? x[2] : x[3];
    return row_lane_value(v, j >> 2);
}

// Inclusive prefix sum over the 16 lanes of each row group (DPP row_shr with
// zero fill).
__device__ __forceinline__ uint32_t row_inclusive_sum(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    return x;
}

// The next element of the sorted row list (rank 4c + r + 1); lane 15's last
// register receives 0.
__device__ __forceinline__ void next_in_list(const uint32_t (&x)[4], uint32_t (&nx)[4])
{
    nx[0] = x[1];
    nx[1] = x[2];
    nx[2] = x[3];
    nx[3] = (uint32_t)__builtin_amdgcn_mov_dpp((int)x[0], 0x101, 0xF, 0xF, true);   // row_shl:1, lane 15 gets 0
}

__device__ __forceinline__ uint32_t group_max16(uint32_t x)
{
    uint32_t y;
    y = row_xor<1>(x); x = x > y ? x : y;
    y = row_xor<2>(x); x = x > y ? x : y;
    y = row_xor<4>(x); x = x > y ? x : y;
    y = row_xor<8>(x); x = x > y ? x : y;
    return x;
}

// Raw fp32 bits of order-preserving score bits (inverse of score_bits).
__device__ __forceinline__ uint32_t raw_of_score_bits(uint32_t u)
{
    return (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
}

// Shift that fits (score bits - tau) >> sh, plus one, below 2^(32 - ib).
__device__ __forceinline__ uint32_t key_shift(uint32_t span, int ib)
{
    const int lim = 31 - ib;   // (span >> sh) < 2^lim
    const int bl = span ? 32 - __clz((int)span) : 0;
    return bl > lim ? (uint32_t)(bl - lim) : 0u;
}

// m = (m << 1) | (x >= t) for fp32 x, t (-0 equals +0; no NaNs): one
// compare into VCC and one add with carry.
__device__ __forceinline__ void push_ge_f32(uint32_t &m, float x, float t)
{
    asm volatile("v_cmp_ge_f32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc" : "+v"(m) : "v"(x), "v"(t) : "vcc");
}

// max(a, b, c) of fp32 values that are never NaN, in one instruction
// (fmaxf would also quiet each operand first, an extra instruction per value).
__device__ __forceinline__ float max3_f32(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Per-row survivor buffers of a wave: 4 rows x 64 entries.
struct RowBuf {
    uint32_t *buf;   // [4][64]
};

// Compacts the candidates of this lane whose bit is set in mask[] into the
// row's buffer, lanes in order (a prefix sum of the lanes' counts over the
// row group).  pos_of(q) maps mask bit q to the stored value.  Returns the
// row's survivor count (all lanes of the row); entries past 64 are dropped.
template <int NMW, class PosOf>
__device__ __forceinline__ uint32_t compact_row(const uint32_t (&mask)[NMW], RowBuf rb, PosOf pos_of)
{
    const int g = lane_id() >> 4;
    uint32_t n = 0;
#pragma unroll
    for (int w = 0; w < NMW; ++w) n += __popc(mask[w]);
    const uint32_t incl = row_inclusive_sum(n);
    uint32_t pos = incl - n;
#pragma unroll
    for (int w = 0; w < NMW; ++w) {
        uint32_t m = mask[w];
        while (m) {
            const int b = __ffs((int)m) - 1;
            m &= m - 1u;
            if (pos < 64u) rb.buf[g * 64 + pos] = pos_of(32 * w + b);
            ++pos;
        }
    }
    wave_lds_sync();
    return row_lane_value(incl, 15);
}

// Top-k' of one half for the 4 rows of this wave (row of lane group g =
// row_g): S holds the row's raw fp32 scores at S + row_g * sst, -inf from
// n_sub up to the next multiple of 64.  Lane c of the row's group receives
// entries 4c .. 4c + 3 of the row's list (best first) in ent[] (entries past
// k' are undefined).  Returns true if this lane's row must be redone by the
// exact one-row routine (ent[] is then undefined).
// With use_floor (uniform over the wave), the threshold is floor_bits (the
// row's, as score bits) instead of the k'-th group maximum: only candidates
// at or above it are listed, `count` of them (at most k'; entries past count
// are undefined).  A caller that needs only the candidates above a score
// already known to have k' others at or above it skips the threshold sort.  Scores are compared as floats while
// scanning (the same order as score_bits for finite values) and as
// score_bits in the sorts.
__device__ __forceinline__ bool half_topk16(const uint32_t *S, int sst, int row_g, int n_sub, int kp, RowBuf rb,
                                            HalfEntry (&ent)[4], uint32_t &count, bool use_floor = false,
                                            uint32_t floor_bits = 0u)
{
    const int c = lane_id() & (kGroupLanes - 1);
    const uint32_t *Sr = S + (size_t)row_g * sst;
    const int nch = (n_sub + 63) >> 6;   // 64 candidates of a row per chunk, 4 per lane
    // Maxima over the chunks, kMaxBatch chunks' LDS reads in flight together
    // (chunk positions clamped to the last one: a chunk read twice leaves a
    // maximum unchanged).
    constexpr int kMaxBatch = 4;
    float mf[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    auto fold = [&](const float4 (&v)[kMaxBatch]) {
        mf[0] = max3_f32(mf[0], v[0].x, v[1].x);
        mf[1] = max3_f32(mf[1], v[0].y, v[1].y);
        mf[2] = max3_f32(mf[2], v[0].z, v[1].z);
        mf[3] = max3_f32(mf[3], v[0].w, v[1].w);
        mf[0] = max3_f32(mf[0], v[2].x, v[3].x);
        mf[1] = max3_f32(mf[1], v[2].y, v[3].y);
        mf[2] = max3_f32(mf[2], v[2].z, v[3].z);
        mf[3] = max3_f32(mf[3], v[2].w, v[3].w);
    };
    if (nch % kMaxBatch == 0) {   // uniform: no clamping needed
        for (int i0 = 0; i0 < nch; i0 += kMaxBatch) {
            float4 v[kMaxBatch];
#pragma unroll
            for (int b = 0; b < kMaxBatch; ++b) v[b] = *reinterpret_cast<const float4 *>(Sr + 64 * (i0 + b) + 4 * c);
            fold(v);
        }
    } else {
        for (int i0 = 0; i0 < nch; i0 += kMaxBatch) {
            float4 v[kMaxBatch];
#pragma unroll
            for (int b = 0; b < kMaxBatch; ++b)
                v[b] = *reinterpret_cast<const float4 *>(Sr + 64 * min(i0 + b, nch - 1) + 4 * c);
            fold(v);
        }
    }
    // an all-padding group (-inf) maps below every finite score
    uint32_t m[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = score_bits(mf[r]);
    uint32_t tau, top;
    if (use_floor) {
        uint32_t mx = m[0] > m[1] ? m[0] : m[1];
        mx = mx > m[2] ? mx : m[2];
        mx = mx > m[3] ? mx : m[3];
        top = group_max16(mx);
        tau = floor_bits;
        top = top > tau ? top : tau;   // no candidate reaches tau: none survives
    } else if (kp <= 32 && n_sub >= 64) {
        // every group maximum is a real score: the 32nd largest of them is
        // reached by at least 32 >= k' candidates
        tau32_top(m, tau, top);
    } else {
        sort64_desc(m);
        tau = rank_value(m, kp - 1);
        top = rank_value(m, 0);
    }
    const float tauf = __uint_as_float(raw_of_score_bits(tau));
    // candidates reaching tau: word w holds chunks 8w .. 8w + 7, candidate
    // (chunk i, k) at bit 31 - (4 (i - 8w) + k).  All 8 chunks of a word are
    // read before the first compare (positions past the row clamped to its
    // last chunk and compared with +inf, which no score reaches, so their
    // bits are 0).
    uint32_t mask[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if (8 * w < nch) {   // uniform
            float4 v[8];
            uint32_t mw = 0u;
            if (8 * w + 8 <= nch) {   // uniform: a whole word
#pragma unroll
                for (int k8 = 0; k8 < 8; ++k8)
                    v[k8] = *reinterpret_cast<const float4 *>(Sr + 64 * (8 * w + k8) + 4 * c);
#pragma unroll
                for (int k8 = 0; k8 < 8; ++k8) {
                    push_ge_f32(mw, v[k8].x, tauf);
                    push_ge_f32(mw, v[k8].y, tauf);
                    push_ge_f32(mw, v[k8].z, tauf);
                    push_ge_f32(mw, v[k8].w, tauf);
                }
            } else {
#pragma unroll
                for (int k8 = 0; k8 < 8; ++k8)
                    v[k8] = *reinterpret_cast<const float4 *>(Sr + 64 * min(8 * w + k8, nch - 1) + 4 * c);
#pragma unroll
                for (int k8 = 0; k8 < 8; ++k8) {
                    const float t = 8 * w + k8 < nch ? tauf : INFINITY;   // uniform
                    push_ge_f32(mw, v[k8].x, t);
                    push_ge_f32(mw, v[k8].y, t);
                    push_ge_f32(mw, v[k8].z, t);
                    push_ge_f32(mw, v[k8].w, t);
                }
            }
            mask[w] = mw;
        }
    }
    const uint32_t total = compact_row<4>(mask, rb, [&](int q) {
        const int e = 32 * (q >> 5) + 31 - (q & 31);   // candidate number 4i + k
        return (uint32_t)(64 * (e >> 2) + 4 * c + (e & 3));
    });
    const int g = lane_id() >> 4;
    int ib = 1;   // bits of a sub-key index
    while ((1 << ib) < n_sub) ++ib;
    const uint32_t imask = (1u << ib) - 1u;
    const uint32_t sh = key_shift(top - tau, ib);
    uint32_t key[4];
    const uint4 e = *reinterpret_cast<const uint4 *>(rb.buf + g * 64 + 4 * c);
    const uint32_t sv[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t j = (uint32_t)(4 * c + r);
        const uint32_t p = j < total ? sv[r] : 0u;
        const uint32_t s = score_bits(__uint_as_float(Sr[p]));
        key[r] = j < total ? ((((s - tau) >> sh) + 1u) << ib) | (imask - p) : 0u;
    }
    wave_lds_sync();   // the buffer is free for the next selection
    sort64_desc(key);
    // full scores of the sorted list, and the check of neighbouring pairs
    // whose shifted scores tie
    uint32_t p[4], s[4], nk[4], ns[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        p[r] = imask - (key[r] & imask);
        s[r] = key[r] ? score_bits(__uint_as_float(Sr[p[r]])) : 0u;
    }
    next_in_list(key, nk);
    next_in_list(s, ns);
    // every neighbouring pair of survivors in the full order (a misordered
    // pair anywhere in a run of tied prefixes could reach the top k')
    bool bad = total > 64u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool tie = nk[r] && (key[r] >> ib) == (nk[r] >> ib);
        bad = bad || (tie && s[r] < ns[r]);
    }
    // one lane's verdict for the whole row
    const uint64_t bb = __ballot(bad);
    const bool row_bad = ((bb >> (16 * g)) & 0xFFFFull) != 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        ent[r].score = raw_of_score_bits(s[r]);
        ent[r].index = p[r];
    }
    count = total < (uint32_t)kp ? total : (uint32_t)kp;
    return row_bad;
}

// Compare-exchange stage of 64-bit keys (element i = 4c + r): i and i ^ M
// are compared and the lower index keeps the larger key; M in {1, 2, 4, 8,
// 16, 32}.
template <int M>
__device__ __forceinline__ void cmpx64_stage(uint64_t (&x)[4])
{
    constexpr int LM = M >> 2, RM = M & 3;
    if constexpr (LM == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if ((r & RM) == 0) {
                const uint64_t a = x[r], b = x[r ^ RM];
                x[r] = a > b ? a : b;
                x[r ^ RM] = a > b ? b : a;
            }
        }
    } else {
        const bool lower = (lane_id() & LM) == 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t lo = row_xor<LM>((uint32_t)x[r]), hi = row_xor<LM>((uint32_t)(x[r] >> 32));
            const uint64_t y = ((uint64_t)hi << 32) | lo;
            const bool take = (y > x[r]) == lower;
            x[r] = take ? y : x[r];
        }
    }
}

// The best kp (<= 32) of two sorted lists, the first of kp entries and the
// second of nb <= kp (best first in the total order score descending, index
// ascending), one list per 16-lane group as half_topk16 leaves them (lane c:
// entries 4c .. 4c + 3; nb is the row's, the same in its 16 lanes).  The
// first list followed by the second in reverse is a bitonic sequence of 64
// keys; six half-cleaner stages sort it, and its first kp elements are the
// answer, exact (the keys are the full (score, index) order).  Lane c
// receives entries 4c .. 4c + 3 of the result in out[].
__device__ __forceinline__ void merge_sorted16(const HalfEntry (&a)[4], const HalfEntry (&b)[4], int kp, int nb,
                                               HalfEntry (&out)[4])
{
    const int c = lane_id() & (kGroupLanes - 1);
    uint64_t ka[4], kb[4], x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        ka[r] = 4 * c + r < kp ? score_key(__uint_as_float(a[r].score), a[r].index) : 0ull;
        kb[r] = 4 * c + r < nb ? score_key(__uint_as_float(b[r].score), b[r].index) : 0ull;
    }
    // element 32 + 4k + r (lane 8 + k) = second list's entry 31 - 4k - r,
    // held by lane 7 - k in register 3 - r: a row_mirror of the registers in
    // reverse order
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = row_xor<15>((uint32_t)kb[3 - r]), hi = row_xor<15>((uint32_t)(kb[3 - r] >> 32));
        x[r] = c < 8 ? ka[r] : (((uint64_t)hi << 32) | lo);
    }
    cmpx64_stage<32>(x);
    cmpx64_stage<16>(x);
    cmpx64_stage<8>(x);
    cmpx64_stage<4>(x);
    cmpx64_stage<2>(x);
    cmpx64_stage<1>(x);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        out[r].score = __float_as_uint(key_score(x[r]));
        out[r].index = key_index(x[r]);
    }
}

// Merge of the two half lists of the 4 rows of this wave into the best n
// slots and their softmax weights.  L0, L1: this lane's row's k' entries of
// half 0 and half 1.  On success lane (c, r) holds rank 4c + r: slot[r],
// wt[r] (ranks >= n hold weight 0).  Returns true if this lane's row must
// be redone by the exact one-row routine (merge_softmax<1>).
__device__ __forceinline__ bool merge16(const HalfEntry *L0, const HalfEntry *L1, int kp, int n_sub, int n,
                                        const uint16_t *stair, int nstair, RowBuf rb, int (&slot)[4],
                                        float (&wt)[4])
{
    constexpr int kMaxPer = (kMaxStair + kGroupLanes - 1) / kGroupLanes;   // staircase entries per lane
    const int c = lane_id() & (kGroupLanes - 1);
    const int g = lane_id() >> 4;
    uint32_t sb[kMaxPer];
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    // the staircase's candidate scores, 16 lanes x kMaxPer; the first
    // kFirst per lane (128 entries, the whole staircase for k', n <= 32)
    // without branches, so that all their LDS reads are in flight together
    constexpr int kFirst = 8;
    auto cand = [&](int i) {
        const int sp = c + kGroupLanes * i;
        const uint32_t ab = stair[min(sp, nstair - 1)];
        const float sum = __uint_as_float(L0[ab >> 8].score) + __uint_as_float(L1[ab & 0xff].score);
        return sp < nstair ? score_bits(sum) : 0u;
    };
#pragma unroll
    for (int i = 0; i < kFirst; ++i) sb[i] = cand(i);
#pragma unroll
    for (int i = kFirst; i < kMaxPer; ++i) sb[i] = kGroupLanes * i < nstair ? cand(i) : 0u;   // uniform
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) m[i & 3] = sb[i] > m[i & 3] ? sb[i] : m[i & 3];
    uint32_t tau, top;
    if (n <= 32 && nstair >= 64) {
        // every group maximum is a candidate: the 32nd largest of them is
        // reached by at least 32 >= n candidates
        tau32_top(m, tau, top);
    } else {
        sort64_desc(m);
        tau = rank_value(m, n - 1);
        top = rank_value(m, 0);
    }
    uint32_t mask[1] = {0u};
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) mask[0] |= (sb[i] >= tau && sb[i] != 0u) ? 1u << i : 0u;
    const uint32_t total = compact_row<1>(mask, rb, [&](int q) { return (uint32_t)(c + kGroupLanes * q); });
    constexpr int ib = 9;   // staircase positions < 512
    constexpr uint32_t imask = (1u << ib) - 1u;
    const uint32_t sh = key_shift(top - tau, ib);
    uint32_t key[4];
    const uint4 e = *reinterpret_cast<const uint4 *>(rb.buf + g * 64 + 4 * c);
    const uint32_t ent[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t j = (uint32_t)(4 * c + r);
        const uint32_t sp = j < total ? ent[r] : 0u;
        const uint32_t ab = stair[sp];
        const uint32_t s = score_bits(__uint_as_float(L0[ab >> 8].score) + __uint_as_float(L1[ab & 0xff].score));
        key[r] = j < total ? ((((s - tau) >> sh) + 1u) << ib) | (imask - sp) : 0u;
    }
    wave_lds_sync();
    sort64_desc(key);
    uint32_t s[4], sl[4], nk[4], ns[4], nsl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t sp = imask - (key[r] & imask);
        const uint32_t ab = key[r] ? stair[sp] : 0u;
        const HalfEntry a = L0[ab >> 8], b = L1[ab & 0xff];
        s[r] = key[r] ? score_bits(__uint_as_float(a.score) + __uint_as_float(b.score)) : 0u;
        sl[r] = a.index * (uint32_t)n_sub + b.index;
    }
    next_in_list(key, nk);
    next_in_list(s, ns);
    next_in_list(sl, nsl);
    bool bad = total > 64u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        // every neighbouring pair of survivors in (score desc, slot asc) order
        const bool ordered = s[r] > ns[r] || (s[r] == ns[r] && sl[r] < nsl[r]);
        bad = bad || (nk[r] != 0u && !ordered);
    }
    // the staircase holds the top n unless a pair just outside it reaches
    // the n-th score: (a, n / (a + 1)) bounds every pair outside
    uint32_t fb = 0u;
    for (int a = c; a < kp; a += kGroupLanes) {
        const int b0 = n / (a + 1);
        if (b0 < kp) {
            const uint32_t v = score_bits(__uint_as_float(L0[a].score) + __uint_as_float(L1[b0].score));
            fb = v > fb ? v : fb;
        }
    }
    fb = group_max16(fb);
    const uint32_t nth = rank_value(s, n - 1);
    bad = bad || !(nth > fb);
    const uint64_t bb = __ballot(bad);
    const bool row_bad = ((bb >> (16 * g)) & 0xFFFFull) != 0;
    // softmax over the n best, the sums in the order of wave_sum_f32 over
    // ranks (pairs of neighbouring ranks first), so the weights match the
    // one-row routine's bit for bit
    const float smax = key_score((uint64_t)rank_value(s, 0) << 32);
    float ex[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int j = 4 * c + r;
        ex[r] = j < n ? __expf(key_score((uint64_t)s[r] << 32) - smax) : 0.f;
    }
    float z = (ex[0] + ex[1]) + (ex[2] + ex[3]);
    z += __uint_as_float(row_xor<1>(__float_as_uint(z)));
    z += __uint_as_float(row_xor<2>(__float_as_uint(z)));
    z += __uint_as_float(row_xor<4>(__float_as_uint(z)));
    z += __uint_as_float(row_xor<8>(__float_as_uint(z)));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        wt[r] = __fdividef(ex[r], z);
        slot[r] = (int)sl[r];
    }
    return row_bad;
}

}  // namespace sdm
