// Level-wise descent with candidate-index RoPE and the mixed softmax, for
// decode and (row by row) for causal prefill, on gfx950.
//
// RecSA, abstract: each level above the tokens keeps at most k candidates;
// the summaries of the candidates not kept share one softmax with the exact
// tokens; each entry's RoPE position is its index among its level's
// candidates.  The query's position at a level is that level's candidate
// count n.
//
// Position split.  Below the top, candidate i of a level is child c of the
// r-th kept parent (i = r*b + c), or orphan c after the m kept parents'
// children (i = m*b + c); either way c = node mod b.  With rotate-half RoPE
//     <rope(q, n), rope(key, i)> = <R((n - r*b) theta) q, R(c theta) key>,
// so a row needs one rotated query per rank r (at most k + 1 per level,
// built once per level into LDS) and each key is rotated only by its child
// offset c.  A slot (16-lane group) takes every NSLOT-th candidate; when b
// divides NSLOT its child offset never changes, and when b = 2 * NSLOT it
// alternates between two, so the key rotation comes from registers.  Other
// fanouts read the rotation of c from the table per candidate.
//
// One workgroup owns one row (a query and a query head).  A lane holds D/32
// RoPE pairs (i, i + D/2), so rotations stay inside a lane; a row is two
// contiguous half-row loads per lane group.  Once level l's kept set is
// known, one pass issues the value loads of level l's entries and the key
// loads of level l-1's candidates together (CB candidates per slot, loads
// branch-free), folds the values into the running softmax and scores the
// keys: a row pays one dependent round trip per level.
//
// Selection (wave 0): logits map to ordered 32-bit integers kept in
// registers; a 32-step bisection with ballots finds the m-th largest, ties
// at it go to the lowest candidate indices, and the kept nodes are written
// in ascending order.  The running max is shared by all slots, so their
// partial softmax states add up at the end without rescaling.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "recsa_internal.hpp"
#include "select_topk.hpp"

namespace recsa {
namespace {

constexpr int kMaxCandidates = 4096;   // selection keeps at most 64 logits per lane
constexpr int kRegKeys = 17;           // registers hold up to 17 * 64 = 1088 logits

__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                     // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Max over the 64 lanes (DPP row shifts, then row broadcasts), uniform result.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    v = max(v, dpp_u32<0x111, 0xf>(0u, v));
    v = max(v, dpp_u32<0x112, 0xf>(0u, v));
    v = max(v, dpp_u32<0x114, 0xf>(0u, v));
    v = max(v, dpp_u32<0x118, 0xf>(0u, v));
    v = max(v, dpp_u32<0x142, 0xa>(0u, v));   // row_bcast:15
    v = max(v, dpp_u32<0x143, 0xc>(0u, v));   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over each 16-lane DPP row; the total lands in the row's lane 15.
__device__ __forceinline__ float row_sum16(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false));
    return v;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// PP elements of T as loaded (bf16 stays packed two per register until use).
template <typename T, int PP> struct Raw;
template <int PP> struct Raw<bf16_t, PP> {
    uint32_t w[PP / 2];
    __device__ __forceinline__ void load(const bf16_t *p) {
        if constexpr (PP == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(p);
        } else {
            #pragma unroll
            for (int i = 0; i < PP / 2; i += 2) {
                const uint2 v = *reinterpret_cast<const uint2 *>(p + 2 * i);
                w[i] = v.x; w[i + 1] = v.y;
            }
        }
    }
    __device__ __forceinline__ void get(float *out) const {
        #pragma unroll
        for (int i = 0; i < PP / 2; ++i) {
            out[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
            out[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    }
};
template <int PP> struct Raw<float, PP> {
    float w[PP];
    __device__ __forceinline__ void load(const float *p) { Vec<float, PP>::load(p, w); }
    __device__ __forceinline__ void get(float *out) const {
        #pragma unroll
        for (int i = 0; i < PP; ++i) out[i] = w[i];
    }
};

// PP consecutive (cos, sin) pairs of one table row (PP * 8 bytes, 16-byte aligned).
template <int PP>
__device__ __forceinline__ void load_cs(const float2 *p, float *c, float *s) {
    #pragma unroll
    for (int q = 0; q < PP; q += 2) {
        const float4 v = *reinterpret_cast<const float4 *>(p + q);
        c[q] = v.x; s[q] = v.y; c[q + 1] = v.z; s[q + 1] = v.w;
    }
}

struct LevelGeom {
    int32_t n;          // candidates at this level
    int32_t nchild;     // candidates that are children of kept parents (b * kept)
    int64_t orphan0;    // node id of the first orphan
    int32_t top;        // 1 at the top level (candidate i is node i)
};

// Level l of a row over n_ctx tokens (pw = b^l), below a level that kept `kept_above`.
__device__ __forceinline__ LevelGeom level_geom(int64_t n_ctx, int64_t pw, int32_t b, bool top,
                                                int32_t kept_above) {
    LevelGeom lg;
    const int64_t Nl = n_ctx / pw;
    lg.top = top;
    if (top) {
        lg.n = (int32_t)Nl;
        lg.nchild = 0;
        lg.orphan0 = 0;
    } else {
        const int64_t Nup = n_ctx / (pw * b);
        lg.nchild = b * kept_above;
        lg.orphan0 = Nup * b;
        lg.n = lg.nchild + (int32_t)(Nl - Nup * b);
    }
    return lg;
}

__device__ __forceinline__ int32_t div_b(int32_t i, int32_t b, int32_t b_shift) {
    return b_shift >= 0 ? (i >> b_shift) : i / b;
}

// Node id of candidate i (any i >= 0; meaningful for i < lg.n).
__device__ __forceinline__ int64_t cand_node(int32_t i, const LevelGeom &lg, const int32_t *parents,
                                             int32_t b, int32_t b_shift) {
    if (lg.top) return i;
    if (i < lg.nchild) {
        const int32_t q = div_b(i, b, b_shift);
        return (int64_t)parents[q] * b + (i - q * b);
    }
    return lg.orphan0 + (i - lg.nchild);
}

// Same selection for levels too wide for registers (logits re-read from LDS).
__device__ void select_topk_lds(const float *z, uint8_t *flag, int32_t *kept_now, int32_t n,
                                int32_t m, const LevelGeom &lg, const int32_t *parents, int32_t b,
                                int32_t b_shift, int lane, float *zmax_out, float *gap_out,
                                int32_t *dbg_sel, int32_t k) {
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
        int cnt = 0;
        for (int t = 0; t < nT; ++t) cnt += __popcll(__ballot(key(t) >= trial));
        if (cnt >= m) T = trial;
    }
    int gt = 0, eq = 0;
    for (int t = 0; t < nT; ++t) {
        gt += __popcll(__ballot(key(t) > T));
        eq += __popcll(__ballot(key(t) == T));
    }
    const uint32_t kmax = wave_umax(lmax);
    uint32_t kn = T;
    if (n > m && gt + eq <= m) {
        uint32_t below = 0;
        for (int t = 0; t < nT; ++t) below = max(below, key(t) < T ? key(t) : 0u);
        kn = wave_umax(below);
    }
    int need = m - gt;
    int32_t cnt = 0;
    for (int t = 0; t < nT; ++t) {
        const int32_t i = lane + 64 * t;
        const uint32_t kv = key(t);
        const uint64_t e = __ballot(kv == T);
        const bool f = (kv > T) || (kv == T && __popcll(e & lanes_below(lane)) < need);
        const int ce = __popcll(e);
        need -= ce < need ? ce : need;
        const uint64_t mask = __ballot(f);
        if (f) {
            const int32_t pos = cnt + __popcll(mask & lanes_below(lane));
            const int64_t node = cand_node(i, lg, parents, b, b_shift);
            kept_now[pos] = (int32_t)node;
            flag[i] = 1;
            if (dbg_sel != nullptr) dbg_sel[pos] = (int32_t)node;
        }
        cnt += __popcll(mask);
    }
    if (lane == 0) {
        *zmax_out = from_ordered(kmax);
        *gap_out = (n > m) ? from_ordered(T) - from_ordered(kn) : NAN;
        if (dbg_sel != nullptr)
            for (int q = m; q < k; ++q) dbg_sel[q] = -1;
    }
}

// CSETS: child-offset rotations a slot keeps in registers (1: b divides NSLOT,
// 2: b == 2 * NSLOT); 0: read the rotation of (i mod b) from the table per candidate.
template <typename T, int D, int NW, int CB, int CSETS, bool POW2>
__global__ __launch_bounds__(NW * 64) void descend_kernel(TreeView tv, DescendArgs a,
                                                          DebugView dbg, int32_t b_shift) {
    constexpr int H2 = D / 2;
    constexpr int PP = D / 32;                 // RoPE pairs per lane
    constexpr int NSLOT = NW * 4;
    static_assert(CSETS != 2 || CB % 2 == 0, "two child offsets alternate between candidates");
    extern __shared__ __align__(16) unsigned char smem[];
    const int32_t maxc = a.max_cand;
    const int32_t b = a.b;
    const int32_t nrank = (maxc + b - 1) / b;
    float *zbuf = reinterpret_cast<float *>(smem);                        // [2][maxc]
    float *U = zbuf + 2 * maxc;                                           // [nrank][D]
    float *red = U + (size_t)nrank * D;                                   // [NW][D]
    float *red_l = red + NW * D;                                          // [NW]
    float *misc = red_l + NW;                                             // [4]: level max by parity
    unsigned char *scratch = reinterpret_cast<unsigned char *>(misc + 4); // selection scratch
    int32_t *kept = reinterpret_cast<int32_t *>(scratch + sel::kScratchBytes);  // [2][k]
    uint8_t *flagbuf = reinterpret_cast<uint8_t *>(kept + 2 * a.k);       // [2][maxc]

    const int64_t row = blockIdx.x;
    const int64_t qi = row / a.Hq;
    const int h = (int)(row - qi * a.Hq);
    const int g = h / a.G;
    const int64_t n_ctx = a.ctx_base + qi * a.ctx_step;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 4, sub = lane & 15;
    const int slot = wave * 4 + grp;
    const int j0 = sub * PP;
    const int nlev = tv.n_levels;
    const float2 *rope = tv.rope;

    // levels above the tokens for this row: H = max{l : n_ctx / b^l >= 1}
    int H = 0;
    int64_t pwH = 1;
    while (n_ctx / (pwH * b) >= 1) { pwH *= b; ++H; }

    float qa[PP], qb[PP];
    {
        const T *qp = static_cast<const T *>(a.q) + row * D;
        Vec<T, PP>::load(qp + j0, qa);
        Vec<T, PP>::load(qp + H2 + j0, qb);
    }
    // rotations of this slot's child offsets
    float cc[CSETS > 0 ? CSETS : 1][PP], cs[CSETS > 0 ? CSETS : 1][PP];
    if constexpr (CSETS > 0) {
        #pragma unroll
        for (int q = 0; q < CSETS; ++q) {
            const int32_t c = (slot + NSLOT * q) % b;
            load_cs<PP>(rope + (int64_t)c * H2 + j0, cc[q], cs[q]);
        }
    }

    if (threadIdx.x == 0) {
        for (int l = H + 1; l <= nlev; ++l) {
            if (dbg.selected != nullptr)
                for (int t = 0; t < a.k; ++t) dbg.selected[(row * nlev + l - 1) * a.k + t] = -1;
            if (dbg.kth_gap != nullptr) dbg.kth_gap[row * nlev + l - 1] = NAN;
        }
    }

    const T *kcache = static_cast<const T *>(tv.k_cache) + (int64_t)g * tv.cap * D;
    const T *vcache = static_cast<const T *>(tv.v_cache) + (int64_t)g * tv.cap * D;
    auto key_base = [&](int l) -> const T * {
        return l == 0 ? kcache : static_cast<const T *>(tv.key[l]) + (int64_t)g * tv.node_cap[l] * D;
    };
    auto val_base = [&](int l) -> const T * {
        return l == 0 ? vcache : static_cast<const T *>(tv.val[l]) + (int64_t)g * tv.node_cap[l] * D;
    };
    // candidate i of a level -> node id, with selects only (i >= lg.n gives a junk id)
    auto node_of = [&](int32_t i, const LevelGeom &lg, const int32_t *parents) -> uint32_t {
        int32_t q, r;
        if constexpr (POW2) {
            q = i >> b_shift;
            r = i & (b - 1);
        } else {
            q = i / b;
            r = i - q * b;
        }
        const int32_t qc = q < a.k ? q : a.k - 1;
        const uint32_t child = (uint32_t)parents[qc] * (uint32_t)b + (uint32_t)r;
        const uint32_t orphan = (uint32_t)lg.orphan0 + (uint32_t)(i - lg.nchild);
        return lg.top ? (uint32_t)i : (i < lg.nchild ? child : orphan);
    };
    constexpr uint32_t ROWB = D * sizeof(T);       // bytes of one key/value row
    const float kLog2e = 1.4426950408889634f;
    // U[r] = R((n - r*b) theta) q for the ranks r < ceil(n / b) of a level with n candidates;
    // slots first_slot, first_slot + stride, ... share the ranks.
    auto build_ranks = [&](int32_t n, int first_slot, int stride) {
        const int32_t R = (n + b - 1) / b;
        for (int32_t r = slot - first_slot; r < R; r += stride) {
            float c[PP], s[PP];
            load_cs<PP>(rope + (int64_t)(n - r * b) * H2 + j0, c, s);
            float ua[PP], ub[PP];
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                ua[p] = qa[p] * c[p] - qb[p] * s[p];
                ub[p] = qb[p] * c[p] + qa[p] * s[p];
            }
            Vec<float, PP>::store(U + (size_t)r * D + j0, ua);
            Vec<float, PP>::store(U + (size_t)r * D + H2 + j0, ub);
        }
    };

    float M = -INFINITY, lsum = 0.f, acc_a[PP], acc_b[PP];
    #pragma unroll
    for (int p = 0; p < PP; ++p) { acc_a[p] = 0.f; acc_b[p] = 0.f; }
    int64_t keys_scored = 0;

    // One pass over candidate indices [0, max(nA, nS)): entries of level A (values, weights
    // zA) and candidates of level S (keys scored into zS).  nA or nS may be 0.
    auto fused_pass = [&](const LevelGeom &lgA, const int32_t *parentsA, const float *zA,
                          const uint8_t *flagA, bool maskA, const T *vA, const LevelGeom &lgS,
                          const int32_t *parentsS, const T *kS, float *zS, uint8_t *flagS) {
        const int32_t nA = lgA.n, nS = lgS.n;
        const int32_t nmax = nA > nS ? nA : nS;
        const char *vAb = reinterpret_cast<const char *>(vA) + j0 * sizeof(T);
        const char *kSb = reinterpret_cast<const char *>(kS) + j0 * sizeof(T);
        const float Ml2 = M * kLog2e;
        for (int32_t base = 0; base < nmax; base += NSLOT * CB) {
            uint32_t offA[CB], offS[CB];
            float ea[CB];                              // log2 of the softmax weight, -inf if none
            #pragma unroll
            for (int t = 0; t < CB; ++t) {
                const int32_t i = base + t * NSLOT + slot;
                const int32_t ic = i < maxc ? i : maxc - 1;
                const bool okA = (i < nA) && !(maskA && flagA[ic]);
                ea[t] = okA ? zA[ic] * kLog2e - Ml2 : -INFINITY;
                offA[t] = okA ? node_of(i, lgA, parentsA) * ROWB : 0u;
                offS[t] = (i < nS) ? node_of(i, lgS, parentsS) * ROWB : 0u;
            }
            Raw<T, PP> va[CB], vb[CB], ka[CB], kb[CB];
            if (nA > 0) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    va[t].load(reinterpret_cast<const T *>(vAb + offA[t]));
                    vb[t].load(reinterpret_cast<const T *>(vAb + offA[t] + H2 * sizeof(T)));
                }
            }
            if (base < nS) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    ka[t].load(reinterpret_cast<const T *>(kSb + offS[t]));
                    kb[t].load(reinterpret_cast<const T *>(kSb + offS[t] + H2 * sizeof(T)));
                }
            }
            if (nA > 0) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    const float pz = __builtin_amdgcn_exp2f(ea[t]);    // 0 for -inf
                    float fa[PP], fb[PP];
                    va[t].get(fa);
                    vb[t].get(fb);
                    lsum += pz;
                    #pragma unroll
                    for (int p = 0; p < PP; ++p) {
                        acc_a[p] += pz * fa[p];
                        acc_b[p] += pz * fb[p];
                    }
                }
            }
            if (base < nS) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    const int32_t i = base + t * NSLOT + slot;
                    const int32_t ic = i < nS ? i : nS - 1;
                    int32_t r;
                    if constexpr (POW2) r = ic >> b_shift; else r = ic / b;
                    float c[PP], s[PP];
                    if constexpr (CSETS == 1) {
                        #pragma unroll
                        for (int p = 0; p < PP; ++p) { c[p] = cc[0][p]; s[p] = cs[0][p]; }
                    } else if constexpr (CSETS == 2) {
                        #pragma unroll
                        for (int p = 0; p < PP; ++p) { c[p] = cc[t & 1][p]; s[p] = cs[t & 1][p]; }
                    } else {
                        load_cs<PP>(rope + (int64_t)(ic - r * b) * H2 + j0, c, s);
                    }
                    float ua[PP], ub[PP], fa[PP], fb[PP];
                    Vec<float, PP>::load(U + (size_t)r * D + j0, ua);
                    Vec<float, PP>::load(U + (size_t)r * D + H2 + j0, ub);
                    ka[t].get(fa);
                    kb[t].get(fb);
                    float dot = 0.f;
                    #pragma unroll
                    for (int p = 0; p < PP; ++p) {
                        const float ra = fa[p] * c[p] - fb[p] * s[p];
                        const float rb = fb[p] * c[p] + fa[p] * s[p];
                        dot += ua[p] * ra + ub[p] * rb;
                    }
                    dot = row_sum16(dot);
                    if (sub == 15 && i < nS) {
                        zS[i] = a.scale * dot;
                        flagS[i] = 0;
                    }
                }
            }
        }
    };

    // ---- top level: score all N_H nodes ----------------------------------------------
    LevelGeom lgA = level_geom(n_ctx, pwH, b, true, 0);
    {
        LevelGeom none{};
        build_ranks(lgA.n, 0, NSLOT);
        __syncthreads();
        fused_pass(none, kept, zbuf, flagbuf, false, nullptr, lgA, kept, key_base(H),
                   zbuf + (H & 1) * maxc, flagbuf + (H & 1) * maxc);
        keys_scored += lgA.n;
    }

    int64_t pw = pwH;
    for (int l = H; l >= 0; --l, pw /= b) {
        __syncthreads();
        float *zA = zbuf + (l & 1) * maxc;
        uint8_t *flagA = flagbuf + (l & 1) * maxc;
        const int32_t nA = lgA.n;
        const int32_t mA = (l > 0) ? (a.k < nA ? a.k : nA) : 0;
        const int32_t *parentsA = kept + ((l + 1) & 1) * a.k;
        int32_t *keptA = kept + (l & 1) * a.k;
        LevelGeom lgS{};
        if (l > 0) lgS = level_geom(n_ctx, pw / b, b, false, mA);
        // ---- selection at level l (wave 0); the other waves build level l-1's ranks ---
        if (wave == 0) {
            if (l > 0) {
                int32_t *ds = dbg.selected ? dbg.selected + (row * nlev + l - 1) * a.k : nullptr;
                float gap;
                auto nodeA = [&](int32_t i) { return cand_node(i, lgA, parentsA, b, b_shift); };
                sel::Result res{};
#define RECSA_SELECT(KT_) \
    res = sel::select<KT_>(zA, flagA, keptA, nA, mA, lane, scratch, nodeA)
                if (nA <= 64) RECSA_SELECT(1);
                else if (nA <= 64 * 2) RECSA_SELECT(2);
                else if (nA <= 64 * 4) RECSA_SELECT(4);
                else if (nA <= 64 * 8) RECSA_SELECT(8);
                else if (nA <= 64 * kRegKeys) RECSA_SELECT(kRegKeys);
                else select_topk_lds(zA, flagA, keptA, nA, mA, lgA, parentsA, b, b_shift, lane,
                                     &res.zmax, &res.gap, nullptr, a.k);
#undef RECSA_SELECT
                if (lane == 0) misc[l & 1] = res.zmax;
                if (lane == 0 && dbg.kth_gap != nullptr) dbg.kth_gap[row * nlev + l - 1] = res.gap;
                if (ds != nullptr) {
                    __threadfence_block();
                    for (int q = lane; q < a.k; q += 64) ds[q] = q < mA ? keptA[q] : -1;
                }
            } else {
                float mx = -INFINITY;
                for (int32_t i = lane; i < nA; i += 64) mx = fmaxf(mx, zA[i]);
                #pragma unroll
                for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
                if (lane == 0) misc[l & 1] = mx;
            }
        } else if (l > 0) {
            build_ranks(lgS.n, 4, NSLOT - 4);
        }
        __syncthreads();

        // ---- fused pass: entries of level l, candidates of level l-1 ---------------------
        const float Mn = fmaxf(M, misc[l & 1]);
        const float corr = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
        lsum *= corr;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { acc_a[p] *= corr; acc_b[p] *= corr; }
        M = Mn;
        fused_pass(lgA, parentsA, zA, flagA, l > 0, val_base(l), lgS, keptA,
                   l > 0 ? key_base(l - 1) : nullptr, zbuf + ((l + 1) & 1) * maxc,
                   flagbuf + ((l + 1) & 1) * maxc);
        keys_scored += lgS.n;
        lgA = lgS;
    }

    // combine the slots: four lane groups by shuffles, the waves through LDS
    #pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        lsum += __shfl_xor(lsum, off);
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            acc_a[p] += __shfl_xor(acc_a[p], off);
            acc_b[p] += __shfl_xor(acc_b[p], off);
        }
    }
    if (grp == 0) {
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            red[wave * D + j0 + p] = acc_a[p];
            red[wave * D + H2 + j0 + p] = acc_b[p];
        }
        if (sub == 0) red_l[wave] = lsum;
    }
    __syncthreads();
    if (wave == 0 && grp == 0) {
        float oa[PP], ob[PP], L = 0.f;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { oa[p] = 0.f; ob[p] = 0.f; }
        for (int w = 0; w < NW; ++w) {
            L += red_l[w];
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                oa[p] += red[w * D + j0 + p];
                ob[p] += red[w * D + H2 + j0 + p];
            }
        }
        #pragma unroll
        for (int p = 0; p < PP; ++p) { oa[p] /= L; ob[p] /= L; }
        if (a.out_bf16) {
            bf16_t *o = static_cast<bf16_t *>(a.out) + row * D;
            Vec<bf16_t, PP>::store(o + j0, oa);
            Vec<bf16_t, PP>::store(o + H2 + j0, ob);
        } else {
            float *o = static_cast<float *>(a.out) + row * D;
            Vec<float, PP>::store(o + j0, oa);
            Vec<float, PP>::store(o + H2 + j0, ob);
        }
        if (sub == 0 && dbg.n_keys != nullptr) dbg.n_keys[row] = (int32_t)keys_scored;
    }
}

template <int NW>
size_t descend_smem(int32_t maxc, int32_t k, int32_t b, int D) {
    const size_t nrank = ((size_t)maxc + b - 1) / b;
    return sizeof(float) * (2 * (size_t)maxc + nrank * D + (size_t)NW * D + NW + 4) +
           sel::kScratchBytes + sizeof(int32_t) * 2 * (size_t)k + 2 * (size_t)maxc;
}

template <typename T, int D, int NW, int CB, int CSETS, bool POW2>
hipError_t launch_descend_t(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                            int32_t b_shift, hipStream_t s) {
    const size_t smem = descend_smem<NW>(a.max_cand, a.k, a.b, D);
    if (smem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)descend_kernel<T, D, NW, CB, CSETS, POW2>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((descend_kernel<T, D, NW, CB, CSETS, POW2>), dim3((unsigned)a.rows),
                       dim3(NW * 64), smem, s, tv, a, dbg, b_shift);
    return hipGetLastError();
}

template <typename T, int D, int NW, int CB>
hipError_t launch_csets(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                        hipStream_t s) {
    constexpr int NSLOT = NW * 4;
    int32_t b_shift = -1;
    if ((a.b & (a.b - 1)) == 0) {
        b_shift = 0;
        while ((1 << b_shift) < a.b) ++b_shift;
    }
    if (b_shift >= 0) {
        if (NSLOT % a.b == 0) return launch_descend_t<T, D, NW, CB, 1, true>(tv, a, dbg, b_shift, s);
        if constexpr (CB % 2 == 0) {
            if (a.b == 2 * NSLOT)
                return launch_descend_t<T, D, NW, CB, 2, true>(tv, a, dbg, b_shift, s);
        }
        return launch_descend_t<T, D, NW, CB, 0, true>(tv, a, dbg, b_shift, s);
    }
    return launch_descend_t<T, D, NW, CB, 0, false>(tv, a, dbg, b_shift, s);
}

// Launch shape: (waves per row, candidates per slot per pass).
// RECSA_DESCEND_SHAPE="NW,CB" overrides the choice (for tuning sweeps).
template <typename T, int D>
hipError_t dispatch(const TreeView &tv, const DescendArgs &a, const DebugView &dbg, hipStream_t s) {
    int nw = 4, cb = 4;
    if (const char *e = getenv("RECSA_DESCEND_SHAPE")) {
        int x = 0, y = 0;
        if (sscanf(e, "%d,%d", &x, &y) == 2) { nw = x; cb = y; }
    }
    if (nw == 4 && cb == 4) return launch_csets<T, D, 4, 4>(tv, a, dbg, s);
    if (nw == 4 && cb == 8) return launch_csets<T, D, 4, 8>(tv, a, dbg, s);
    if (nw == 8 && cb == 2) return launch_csets<T, D, 8, 2>(tv, a, dbg, s);
    if (nw == 8 && cb == 8) return launch_csets<T, D, 8, 8>(tv, a, dbg, s);
    return launch_csets<T, D, 8, 4>(tv, a, dbg, s);
}

}  // namespace

size_t descend_lds_bytes(int32_t maxc, int32_t k, int32_t b, int32_t D) {
    return descend_smem<8>(maxc, k, b, D);
}
int32_t descend_max_candidates() { return kMaxCandidates; }

hipError_t launch_descend(const TreeView &tv, recsa_dtype st, int32_t D, const DescendArgs &a,
                          const DebugView &dbg, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (st == RECSA_BF16) {
        if (D == 128) return dispatch<bf16_t, 128>(tv, a, dbg, s);
        return dispatch<bf16_t, 64>(tv, a, dbg, s);
    }
    if (D == 128) return dispatch<float, 128>(tv, a, dbg, s);
    return dispatch<float, 64>(tv, a, dbg, s);
}

}  // namespace recsa
