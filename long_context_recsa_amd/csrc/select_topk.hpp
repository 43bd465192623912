// Wave-level selection of the m largest of n fp32 logits for gfx950.
//
// RecSA, abstract: each level above the tokens keeps at most k candidates.
// Equal logits go to the lower candidate index.
//
// On CDNA a wave-wide reduction followed by a read of its result (or an LDS
// round trip) costs on the order of a hundred cycles, so this selection uses
// a constant number of them instead of one per kept candidate:
//   1. every lane maps its logits (candidates lane, lane+64, ...) to ordered
//      32-bit keys and takes their max;
//   2. DPP reduces the lane maxima to the max of each group of G lanes
//      (G = 16, 8, 4 or 2, so that there are at least m groups); tau, the
//      smallest group max, is a lower bound of the m-th largest key: each
//      group holds a key >= tau;
//   3. the candidates with key >= tau (a few dozen) are compacted into LDS
//      with a DPP prefix sum;
//   4. each survivor is ranked exactly against the others (larger key
//      first, then lower index), reading them back 8 at a time by LDS
//      broadcast; rank < m keeps it, and the kept ones are ordered by index.
// Levels of at most 5 * 64 candidates instead find the threshold by bisection
// with ballots over register-resident keys, which is faster there (it stops as
// soon as exactly m keys lie above it); levels too wide for registers and the
// rare filter that lets more than 128 candidates through (many equal logits)
// use a 32-step bisection over the keys in LDS.
#pragma once

#include <math.h>

#include "recsa_internal.hpp"

namespace recsa {
namespace sel {

__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                     // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Max / min over the 64 lanes, uniform result.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    v = max(v, dpp<0x111, 0xf>(0u, v));
    v = max(v, dpp<0x112, 0xf>(0u, v));
    v = max(v, dpp<0x114, 0xf>(0u, v));
    v = max(v, dpp<0x118, 0xf>(0u, v));
    v = max(v, dpp<0x142, 0xa>(0u, v));   // row_bcast:15
    v = max(v, dpp<0x143, 0xc>(0u, v));   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
    v = min(v, dpp<0x111, 0xf>(~0u, v));
    v = min(v, dpp<0x112, 0xf>(~0u, v));
    v = min(v, dpp<0x114, 0xf>(~0u, v));
    v = min(v, dpp<0x118, 0xf>(~0u, v));
    v = min(v, dpp<0x142, 0xa>(~0u, v));
    v = min(v, dpp<0x143, 0xc>(~0u, v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_scan_add(uint32_t v) {
    v += dpp<0x111, 0xf>(0u, v);
    v += dpp<0x112, 0xf>(0u, v);
    v += dpp<0x114, 0xf>(0u, v);
    v += dpp<0x118, 0xf>(0u, v);
    v += dpp<0x142, 0xa>(0u, v);
    v += dpp<0x143, 0xc>(0u, v);
    return v;
}

// Max over aligned groups of G lanes, in every lane of the group.
template <int G>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
    v = max(v, dpp<0xB1, 0xf>(0u, v));                          // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v = max(v, dpp<0x4E, 0xf>(0u, v));    // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v = max(v, dpp<0x141, 0xf>(0u, v));   // row_half_mirror
    if constexpr (G >= 16) v = max(v, dpp<0x140, 0xf>(0u, v));  // row_mirror
    return v;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Candidates of one level: i < nchild is child (i mod b) of kept parent
// parents[i / b]; the rest are orphans from node orphan0 on; at the top
// level (top != 0) candidate i is node i.
struct Cands {
    int32_t n, nchild, b, top;
    int32_t orphan0;
};

__device__ __forceinline__ int32_t node_id(int32_t i, const Cands &c, const int32_t *parents) {
    if (c.top) return i;
    if (i < c.nchild) {
        const int32_t q = i / c.b;
        return parents[q] * c.b + (i - q * c.b);
    }
    return c.orphan0 + (i - c.nchild);
}

// LDS scratch the selection needs.
constexpr int kScratchBytes = 128 * 8 + 128 * 4 + 16;

// out[0] = level max, out[1] = m-th largest, out[2] = (m+1)-th largest logit.
__device__ __noinline__ void select_bisect(const float *z, uint8_t *flag, int32_t *kept, int32_t m,
                                           Cands cd, const int32_t *parents, int lane,
                                           float *out) {
    const int32_t n = cd.n;
    const int nT = (n + 63) >> 6;
    auto key = [&](int t) -> uint32_t {
        const int32_t i = lane + 64 * t;
        return i < n ? ordered_bits(z[i]) : 0u;
    };
    uint32_t lmax = 0;
    for (int t = 0; t < nT; ++t) lmax = max(lmax, key(t));
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t trial = T | (1u << bit);
        int c = 0;
        for (int t = 0; t < nT; ++t) c += __popcll(__ballot(key(t) >= trial));
        if (c >= m) T = trial;
    }
    int gt = 0, eq = 0;
    for (int t = 0; t < nT; ++t) {
        gt += __popcll(__ballot(key(t) > T));
        eq += __popcll(__ballot(key(t) == T));
    }
    int need = m - gt;
    int32_t pos = 0;
    uint32_t below = 0;
    for (int t = 0; t < nT; ++t) {
        const int32_t i = lane + 64 * t;
        const uint32_t kv = key(t);
        if (i < n && kv < T) below = max(below, kv);
        const uint64_t e = __ballot(kv == T);
        const bool f = (i < n) && ((kv > T) || (kv == T && __popcll(e & lanes_below(lane)) < need));
        const int ce = __popcll(e);
        need -= ce < need ? ce : need;
        const uint64_t mask = __ballot(f);
        if (f) {
            kept[pos + __popcll(mask & lanes_below(lane))] = node_id(i, cd, parents);
            flag[i] = 1;
        }
        pos += __popcll(mask);
    }
    const uint32_t kmax = wave_umax(lmax);
    const uint32_t kn = (gt + eq > m) ? T : wave_umax(below);
    if (lane == 0) {
        out[0] = from_ordered(kmax);
        out[1] = from_ordered(T);
        out[2] = (n > m) ? from_ordered(kn) : NAN;
    }
}

// Keep the m largest of z[0..cd.n) (1 <= m <= n): kept[0..m) gets their node ids in
// ascending candidate order and flag[i] = 1 marks them.  KT >= ceil(n / 64) logits
// per lane live in registers (KT == 0: bisection over LDS).  Results in out[0..3):
// level max, m-th and (m+1)-th largest logit (NaN when n == m); visible to the
// calling wave on return.
// Bisection for the m-th largest key with the keys in registers (narrow levels:
// ballot rounds over KT registers beat the filter's LDS round trips there).
// The largest threshold T with at least m of the keys (NT registers per lane;
// unused slots 0) >= T, bit by bit from bit `top` down, starting from T (a value
// with at least m keys >= it, zero below bit `top`).  Once exactly m keys are >=
// the trial threshold, every threshold in that gap keeps the same m keys: stop there.
template <int NT>
__device__ __forceinline__ uint32_t bisect_threshold(const uint32_t *kk, int m, uint32_t T, int top) {
    for (int bit = top; bit >= 0; --bit) {
        const uint32_t trial = T | (1u << bit);
        int c = 0;
        #pragma unroll
        for (int t = 0; t < NT; ++t) c += __popcll(__ballot(kk[t] >= trial));
        if (c >= m) {
            T = trial;
            if (c == m) break;
        }
    }
    return T;
}

// The ordered keys of candidates lane, lane + 64, ... of z[0..n) (0 past n: valid
// keys are > 0).
template <int KT>
__device__ __forceinline__ void load_keys(const float *z, int32_t n, int lane, uint32_t (&kk)[KT]) {
    #pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int32_t i = lane + 64 * t;
        kk[t] = (i < n) ? ordered_bits(z[i]) : 0u;
    }
}

template <int KT>
__device__ __forceinline__ void select_bisect_regs(const uint32_t (&kk)[KT], uint8_t *flag, int32_t *kept,
                                                   int32_t m, Cands cd, const int32_t *parents,
                                                   int lane, float *out) {
    // wave-uniform counts in scalar registers (they may come from a vector load)
    const int32_t n = __builtin_amdgcn_readfirstlane(cd.n);
    m = __builtin_amdgcn_readfirstlane(m);
    const int nT = (n + 63) >> 6;                       // registers that hold keys
    uint32_t lmax = 0;
    #pragma unroll
    for (int t = 0; t < KT; ++t) lmax = max(lmax, kk[t]);
    const uint32_t kmax = wave_umax(lmax);
    // The m-th largest key K lies in [tau, kmax], with tau the smallest of the maxima
    // of 64/G >= m lane groups (each group holds a key >= tau; a group without valid
    // keys has maximum 0, and then tau = 0).  Every value in that range shares the
    // bits above the highest bit where tau and kmax differ, so the bisection starts
    // there: the threshold with those bits and zeros below has >= m keys above it.
    uint32_t T = 0;
    int top = 31;
    if (m <= 32) {
        uint32_t gmax;
        if (m <= 4) gmax = group_umax<16>(lmax);
        else if (m <= 8) gmax = group_umax<8>(lmax);
        else if (m <= 16) gmax = group_umax<4>(lmax);
        else gmax = group_umax<2>(lmax);
        const uint32_t tau = wave_umin(gmax);
        const uint32_t d = tau ^ kmax;
        top = d == 0u ? -1 : 31 - (int)__builtin_clz(d);
        T = top < 0 ? kmax : (top == 31 ? 0u : kmax & ~((2u << top) - 1u));
    }
    if (nT <= 1)
        T = bisect_threshold<1>(kk, m, T, top);
    else if (nT <= 2 || KT <= 2)
        T = bisect_threshold<(KT < 2 ? KT : 2)>(kk, m, T, top);
    else if (nT <= 3 || KT <= 3)
        T = bisect_threshold<(KT < 3 ? KT : 3)>(kk, m, T, top);
    else if (nT <= 4 || KT <= 4)
        T = bisect_threshold<(KT < 4 ? KT : 4)>(kk, m, T, top);
    else
        T = bisect_threshold<KT>(kk, m, T, top);
    // kept: every key > T, then keys == T in ascending index until m are kept
    int gt = 0;
    #pragma unroll
    for (int t = 0; t < KT; ++t)
        if (t < nT) gt += __popcll(__ballot(kk[t] > T));
    int need = m - gt;
    int32_t pos = 0;
    uint32_t kmin = 0xFFFFFFFFu, below = 0;
    #pragma unroll
    for (int t = 0; t < KT; ++t) {
        if (t >= nT) break;
        const int32_t i = lane + 64 * t;
        const uint64_t e = __ballot(i < n && kk[t] == T);
        const bool f = (i < n) && ((kk[t] > T) || (kk[t] == T && __popcll(e & lanes_below(lane)) < need));
        const int ce = __popcll(e);
        need -= ce < need ? ce : need;
        const uint64_t mask = __ballot(f);
        if (f) {
            kept[pos + __popcll(mask & lanes_below(lane))] = node_id(i, cd, parents);
            flag[i] = 1;
            kmin = min(kmin, kk[t]);
        } else if (i < n) {
            below = max(below, kk[t]);
        }
        pos += __popcll(mask);
    }
    kmin = wave_umin(kmin);
    below = wave_umax(below);
    if (lane == 0) {
        out[0] = from_ordered(kmax);
        out[1] = from_ordered(kmin);
        out[2] = (n > m) ? from_ordered(below) : NAN;
    }
}

// The selection with the keys already in registers (KT > 0, from load_keys); z is
// read again only by the rare fallback of the wide filter.
template <int KT>
__device__ __forceinline__ void select_from_keys(const uint32_t (&kk)[KT], const float *z, uint8_t *flag,
                                                 int32_t *kept, int32_t m, Cands cd,
                                                 const int32_t *parents, int lane,
                                                 unsigned char *scratch, float *out) {
    static_assert(KT > 0, "register keys");
    if constexpr (KT <= 5) {
        select_bisect_regs<KT>(kk, flag, kept, m, cd, parents, lane, out);
        __threadfence_block();
        return;
    } else {
        const int32_t n = cd.n;
        uint2 *list = reinterpret_cast<uint2 *>(scratch);                 // [128] (key, index)
        uint32_t *keep = reinterpret_cast<uint32_t *>(scratch + 128 * 8);  // [128]
        uint32_t lmax = 0;
        #pragma unroll
        for (int t = 0; t < KT; ++t) lmax = max(lmax, kk[t]);
        uint32_t gmax;
        if (m <= 4) gmax = group_umax<16>(lmax);
        else if (m <= 8) gmax = group_umax<8>(lmax);
        else if (m <= 16) gmax = group_umax<4>(lmax);
        else gmax = group_umax<2>(lmax);
        // at least m groups each hold a key >= tau (or a group holds no valid key,
        // n < 64, and tau = 0 lets every valid candidate through)
        const uint32_t tau = (m <= 32) ? wave_umin(gmax) : 0u;
        uint32_t cnt = 0;
        #pragma unroll
        for (int t = 0; t < KT; ++t) cnt += (lane + 64 * t < n && kk[t] >= tau) ? 1u : 0u;
        const uint32_t incl = wave_scan_add(cnt);
        const uint32_t C = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        if (C > 128) {
            select_bisect(z, flag, kept, m, cd, parents, lane, out);
            __threadfence_block();
            return;
        }
        uint32_t at = incl - cnt;
        #pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int32_t i = lane + 64 * t;
            if (i < n && kk[t] >= tau) list[at++] = make_uint2(kk[t], (uint32_t)i);
        }
        __threadfence_block();
        // exact rank of each survivor: larger key first, then lower index
        const bool h0 = (uint32_t)lane < C, h1 = (uint32_t)lane + 64 < C;
        const uint2 e0 = h0 ? list[lane] : make_uint2(0u, 0u);
        const uint2 e1 = h1 ? list[lane + 64] : make_uint2(0u, 0u);
        uint32_t r0 = 0, r1 = 0;
        const uint4 *list4 = reinterpret_cast<const uint4 *>(list);
        for (uint32_t j0 = 0; j0 < C; j0 += 8) {
            uint4 q[4];
            #pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = list4[j0 / 2 + u];
            #pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t ox = (u & 1) ? q[u >> 1].z : q[u >> 1].x;
                const uint32_t oy = (u & 1) ? q[u >> 1].w : q[u >> 1].y;
                const bool valid = j0 + u < C;
                r0 += (valid && (ox > e0.x || (ox == e0.x && oy < e0.y))) ? 1u : 0u;
                r1 += (valid && (ox > e1.x || (ox == e1.x && oy < e1.y))) ? 1u : 0u;
            }
        }
        const bool k0 = h0 && r0 < (uint32_t)m;
        const bool k1 = h1 && r1 < (uint32_t)m;
        if (h0) keep[lane] = k0 ? e0.y : 0xFFFFFFFFu;
        if (h1) keep[lane + 64] = k1 ? e1.y : 0xFFFFFFFFu;
        if (h0) {
            if (r0 == 0) out[0] = from_ordered(e0.x);
            if (r0 == (uint32_t)m - 1) out[1] = from_ordered(e0.x);
            if (r0 == (uint32_t)m) out[2] = from_ordered(e0.x);
        }
        if (h1) {
            if (r1 == 0) out[0] = from_ordered(e1.x);
            if (r1 == (uint32_t)m - 1) out[1] = from_ordered(e1.x);
            if (r1 == (uint32_t)m) out[2] = from_ordered(e1.x);
        }
        if (C == (uint32_t)m) {          // the (m+1)-th largest is below tau
            uint32_t below = 0;
            #pragma unroll
            for (int t = 0; t < KT; ++t)
                below = max(below, (lane + 64 * t < n && kk[t] < tau) ? kk[t] : 0u);
            below = wave_umax(below);
            if (lane == 0) out[2] = (n > m) ? from_ordered(below) : NAN;
        }
        __threadfence_block();
        // ascending position among the kept
        uint32_t p0 = 0, p1 = 0;
        const uint4 *keep4 = reinterpret_cast<const uint4 *>(keep);
        for (uint32_t j0 = 0; j0 < C; j0 += 16) {
            uint4 q[4];
            #pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = keep4[j0 / 4 + u];
            #pragma unroll
            for (int u = 0; u < 16; ++u) {
                const uint4 v = q[u >> 2];
                const uint32_t o = (u & 3) == 0 ? v.x : (u & 3) == 1 ? v.y : (u & 3) == 2 ? v.z : v.w;
                const bool valid = j0 + u < C;
                p0 += (valid && o < e0.y) ? 1u : 0u;
                p1 += (valid && o < e1.y) ? 1u : 0u;
            }
        }
        if (k0) {
            kept[p0] = node_id((int32_t)e0.y, cd, parents);
            flag[e0.y] = 1;
        }
        if (k1) {
            kept[p1] = node_id((int32_t)e1.y, cd, parents);
            flag[e1.y] = 1;
        }
        __threadfence_block();
    }
}

template <int KT>
__device__ __forceinline__ void select(const float *z, uint8_t *flag, int32_t *kept, int32_t m,
                                       Cands cd, const int32_t *parents, int lane,
                                       unsigned char *scratch, float *out) {
    if constexpr (KT == 0) {
        select_bisect(z, flag, kept, m, cd, parents, lane, out);
        __threadfence_block();
    } else {
        uint32_t kk[KT];
        load_keys<KT>(z, cd.n, lane, kk);
        select_from_keys<KT>(kk, z, flag, kept, m, cd, parents, lane, scratch, out);
    }
}

}  // namespace sel
}  // namespace recsa
