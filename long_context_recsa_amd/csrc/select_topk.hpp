// Wave-level selection of the m largest of n fp32 logits for gfx950.
//
// RecSA, abstract (sentence on selection): no more than k candidates survive a level.
// Equal logits go to the lower candidate index.
//
// On CDNA a wave-wide reduction followed by a read of its result (or an LDS
// round trip) costs on the order of a hundred cycles, so the selection takes a
// short, fixed sequence of wave-wide steps rather than one per kept candidate:
//   - levels of at most 64 candidates (every top level) rank each candidate
//     exactly by counting the candidates ahead of it (select_small);
//   - wider levels whose logits fit in registers (up to 17 per lane) find the
//     m-th largest key by bisection with ballots: the search starts at the
//     highest bit where the level's largest key and tau differ (tau, the
//     smallest of >= m lane-group maxima, bounds the m-th largest from below)
//     and stops as soon as exactly m keys lie above the threshold;
//   - levels too wide for registers run a 32-step bisection over the keys in
//     LDS.
// The kept candidates are then flagged and listed in ascending index order.
// (A filter that ranks the keys >= tau against each other was measured slower
// than the register bisection at 512 to 1087 candidates: 3.5 / 4.6 / 7.6 us
// against 1.6 / 2.7 / 3.7 us per level at the 1M-token, fanout-64 workload.)
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

// Orders LDS writes of some lanes of a wave before later reads by other lanes of the
// same wave.  (Readers in other waves need a workgroup barrier as well.)  A
// workgroup-scope fence would also wait for every global load the wave has in
// flight, such as the next row's prefetched logits.
__device__ __forceinline__ void wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Candidates of one level: i < nchild is child (i mod b) of kept parent
// parents[i / b]; the rest are orphans from node orphan0 on; at the top
// level (top != 0) candidate i is node i.
struct Cands {
    int32_t n, nchild, b, top;
    int32_t orphan0;
    uint32_t bmul;      // fanout_magic(b): i / b == umulhi(i, bmul) for candidate indexes
};

// The multiplier m = floor((2^32 - 1) / b) + 1 (b >= 2).  With m b = 2^32 + e, 0 <= e < b,
// i m / 2^32 = i / b + i e / (b 2^32), whose floor is floor(i / b) whenever i b < 2^32:
// far above any level's candidate count times its fanout.
__host__ __device__ __forceinline__ uint32_t fanout_magic(uint32_t b) { return 0xFFFFFFFFu / b + 1u; }

__device__ __forceinline__ int32_t node_id(int32_t i, const Cands &c, const int32_t *parents) {
    if (c.top) return i;
    if (i < c.nchild) {
        const int32_t q = (int32_t)__umulhi((uint32_t)i, c.bmul);
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
// ascending candidate order and flag[i] = 1 marks them (ordered for the calling wave
// on return; other waves read them after a barrier).  KT >= ceil(n / 64) logits
// per lane live in registers (KT == 0: bisection over LDS).  Results in out[0..3):
// level max, m-th and (m+1)-th largest logit (NaN when n == m); visible to the
// calling wave on return.
// Bisection with the keys in registers: a threshold T with at least m of the keys
// (NT registers per lane; unused slots 0) >= T, raised bit by bit from bit `top`
// down, starting from T (a value with at least m keys >= it, zero below bit `top`).
// It stops as soon as at most `cap` keys are >= the threshold (they include the m
// largest, which the caller then ranks), else at the m-th largest key itself.
template <int NT>
__device__ __forceinline__ uint32_t bisect_threshold(const uint32_t *kk, int m, uint32_t T, int top, int cap) {
    for (int bit = top; bit >= 0; --bit) {
        const uint32_t trial = T | (1u << bit);
        int c = 0;
        #pragma unroll
        for (int t = 0; t < NT; ++t) c += __popcll(__ballot(kk[t] >= trial));
        if (c >= m) {
            T = trial;
            if (c <= cap) break;
        }
    }
    return T;
}

// Number of keys >= x over the first nT registers (x >= 1: unused slots hold 0).
template <int KT>
__device__ __forceinline__ int count_ge(const uint32_t (&kk)[KT], int nT, uint32_t x) {
    int c = 0;
    #pragma unroll
    for (int t = 0; t < KT; ++t)
        if (t < nT) c += __popcll(__ballot(kk[t] >= x));
    return c;
}

// The ordered keys of candidates lane, lane + 64, ... of z[0..n) (0 past n: valid
// keys are > 0).  Every lane reads inside z[0..n) (past n it reads z[n - 1] and drops
// it), so the KT loads go out together instead of one guarded load at a time.
template <int KT>
__device__ __forceinline__ void load_keys(const float *z, int32_t n, int lane, uint32_t (&kk)[KT]) {
    float v[KT];
    #pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int32_t i = lane + 64 * t;
        v[t] = z[i < n ? i : n - 1];
    }
    #pragma unroll
    for (int t = 0; t < KT; ++t) kk[t] = (lane + 64 * t < n) ? ordered_bits(v[t]) : 0u;
}

// Rank of this lane's key among the keys of lanes [0, c) (c <= 64): the number of them
// ahead of it, a larger key or an equal key in a lower lane.  Lanes from c on must
// hold key 0 (below every valid key), so reading up to seven past c changes nothing.
// Key and lane go into one 64-bit value, key:(63 - lane), so "ahead" is a single
// unsigned comparison and each lane costs a read, a compare and an add on the vector
// unit (separate key and index comparisons had chained vector and scalar instructions
// through the condition masks, about 115 cycles a lane); eight lanes per step keep
// eight reads in flight.
__device__ __forceinline__ int rank_among(uint32_t key, int32_t c, int lane) {
    const uint64_t mine = ((uint64_t)key << 32) | (uint32_t)(63 - lane);
    int rank = 0;
    const int32_t c8 = (c + 7) & ~7;
    for (int32_t j = 0; j < c8; j += 8) {
        #pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, j + u);
            const uint64_t other = ((uint64_t)kj << 32) | (uint32_t)(63 - (j + u));
            rank += other > mine ? 1 : 0;
        }
    }
    return rank;
}

// The m largest of c <= 64 survivor keys (every key >= T, the rest are < T), listed
// in ascending candidate order in cs[0..c) (keys) and cs[64..64+c) (candidate
// indexes): each survivor's rank is counted exactly, as in select_small.  `below` is
// this lane's largest key under T (the (m+1)-th largest when exactly m survive).
__device__ __forceinline__ void rank_survivors(const uint32_t *cs, int32_t c, uint32_t kmax, uint32_t below,
                                               uint8_t *flag, int32_t *kept, int32_t m, Cands cd,
                                               const int32_t *parents, int lane, float *out) {
    const bool valid = lane < c;
    const uint32_t key = valid ? cs[lane] : 0u;
    const int32_t idx = valid ? (int32_t)cs[64 + lane] : 0;
    // the node id's parent read goes out before the ranking, which hides it
    const int32_t nid = node_id(idx, cd, parents);
    const int rank = rank_among(key, c, lane);
    const bool keep = valid && rank < m;
    const uint64_t km = __ballot(keep);
    if (keep) {
        kept[__popcll(km & lanes_below(lane))] = nid;
        flag[idx] = 1;
    }
    const uint64_t rm1 = __ballot(valid && rank == m - 1);
    const uint64_t rm = __ballot(valid && rank == m);
    const uint32_t kb = wave_umax(below);
    if (lane == 0) {
        out[0] = from_ordered(kmax);
        out[1] = from_ordered((uint32_t)__builtin_amdgcn_readlane((int)key, (int)__builtin_ctzll(rm1)));
        out[2] = c > m ? from_ordered((uint32_t)__builtin_amdgcn_readlane((int)key, (int)__builtin_ctzll(rm)))
                       : (cd.n > m ? from_ordered(kb) : NAN);
    }
}

template <int KT>
__device__ __forceinline__ void select_bisect_regs(const uint32_t (&kk)[KT], uint8_t *flag, int32_t *kept,
                                                   int32_t m, Cands cd, const int32_t *parents,
                                                   int lane, uint32_t *cs, float *out) {
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
    // survivors: keys >= a threshold that at least m and at most 64 keys reach; they
    // are then ranked exactly.  The lower bound tau often leaves few enough already.
    uint32_t Ts = 0;
    int cT = 0;
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
        Ts = tau > 1u ? tau : 1u;
        cT = count_ge<KT>(kk, nT, Ts);
    }
    if (cT == 0 || cT > 64) {
        if (nT <= 1)
            T = bisect_threshold<1>(kk, m, T, top, 64);
        else if (nT <= 2 || KT <= 2)
            T = bisect_threshold<(KT < 2 ? KT : 2)>(kk, m, T, top, 64);
        else if (nT <= 3 || KT <= 3)
            T = bisect_threshold<(KT < 3 ? KT : 3)>(kk, m, T, top, 64);
        else if (nT <= 4 || KT <= 4)
            T = bisect_threshold<(KT < 4 ? KT : 4)>(kk, m, T, top, 64);
        else
            T = bisect_threshold<KT>(kk, m, T, top, 64);
        Ts = T > 1u ? T : 1u;
        cT = count_ge<KT>(kk, nT, Ts);
    }
    if (cT <= 64) {
        // compact the survivors, in ascending candidate order, into cs.  Every register
        // is visited (those past nT hold 0, below Ts >= 1, and index no candidate), so
        // the loop is straight-line code: all the ballots first, then the stores.
        uint64_t mask[KT];
        #pragma unroll
        for (int t = 0; t < KT; ++t) mask[t] = __ballot(kk[t] >= Ts);
        int32_t base = 0;
        uint32_t below = 0;
        #pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int32_t i = lane + 64 * t;
            const bool sv = kk[t] >= Ts;
            if (sv) {
                const int32_t p = base + __popcll(mask[t] & lanes_below(lane));
                cs[p] = kk[t];
                cs[64 + p] = (uint32_t)i;
            } else if (i < n) {
                below = max(below, kk[t]);
            }
            base += __popcll(mask[t]);
        }
        wave_fence();
        rank_survivors(cs, cT, kmax, below, flag, kept, m, cd, parents, lane, out);
        return;
    }
    // more than 64 keys tie at the m-th largest: T is that key
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

// Levels of at most 64 candidates (every top level: fewer than b nodes), one key per
// lane: each candidate's rank is counted exactly, the number of candidates ahead of it
// (a larger key, or an equal key at a lower index), and ranks below m are kept.  A
// constant number of steps per candidate, where the bisection's rounds run from the
// highest bit when the level has fewer than m lane groups holding keys.
__device__ __forceinline__ void select_small(uint32_t key, uint8_t *flag, int32_t *kept, int32_t m,
                                             Cands cd, const int32_t *parents, int lane, float *out) {
    const int32_t n = __builtin_amdgcn_readfirstlane(cd.n);
    m = __builtin_amdgcn_readfirstlane(m);
    const bool valid = lane < n;
    const int rank = rank_among(key, n, lane);
    const bool keep = valid && rank < m;
    const uint64_t km = __ballot(keep);
    if (keep) {
        kept[__popcll(km & lanes_below(lane))] = node_id(lane, cd, parents);
        flag[lane] = 1;
    }
    // level max, m-th and (m+1)-th largest: the keys of ranks 0, m - 1 and m
    const uint64_t r0 = __ballot(valid && rank == 0);
    const uint64_t rm1 = __ballot(valid && rank == m - 1);
    const uint64_t rm = __ballot(valid && rank == m);
    if (lane == 0) {
        out[0] = from_ordered((uint32_t)__builtin_amdgcn_readlane((int)key, (int)__builtin_ctzll(r0)));
        out[1] = from_ordered((uint32_t)__builtin_amdgcn_readlane((int)key, (int)__builtin_ctzll(rm1)));
        out[2] = n > m ? from_ordered((uint32_t)__builtin_amdgcn_readlane((int)key, (int)__builtin_ctzll(rm)))
                       : NAN;
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
    if (cd.n <= 64) {
        select_small(kk[0], flag, kept, m, cd, parents, lane, out);
        wave_fence();
        return;
    }
    select_bisect_regs<KT>(kk, flag, kept, m, cd, parents, lane, reinterpret_cast<uint32_t *>(scratch), out);
    wave_fence();
}

template <int KT>
__device__ __forceinline__ void select(const float *z, uint8_t *flag, int32_t *kept, int32_t m,
                                       Cands cd, const int32_t *parents, int lane,
                                       unsigned char *scratch, float *out) {
    if constexpr (KT == 0) {
        select_bisect(z, flag, kept, m, cd, parents, lane, out);
        wave_fence();
    } else {
        uint32_t kk[KT];
        load_keys<KT>(z, cd.n, lane, kk);
        select_from_keys<KT>(kk, z, flag, kept, m, cd, parents, lane, scratch, out);
    }
}

}  // namespace sel
}  // namespace recsa
