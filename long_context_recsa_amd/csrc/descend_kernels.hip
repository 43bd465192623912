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
// so a row needs one rotated query per rank r (at most k + 1 per level, built
// once per level into LDS) and each key is rotated only by its child offset c.
// The top level has fewer than b candidates, so r = 0 and c = i there.
//
// Work split.  One workgroup owns one row (a query and a query head).  A
// 16-lane group (a "slot", one DPP row) handles one candidate at a time; a
// lane holds D/32 RoPE pairs (i, i + D/2), so rotations stay inside a lane and
// a key row is two contiguous half-row loads per slot.  Slot s owns the child
// offsets c = s, s + NSLOT, ... and, for each, the ranks r = 0, 1, ...: only
// one child-offset rotation is live at a time and no candidate index needs a
// division.  Once level l's kept set is known, one pass issues the value loads
// of level l's entries and the key loads of level l-1's candidates together
// (CB ranks per slot, branch-free, 32-bit offsets from uniform bases), folds
// the values into the running softmax and scores the keys: a row pays one
// dependent round trip per level.  The running max is shared by all slots,
// so their partial softmax states add up at the end without rescaling.
//
// Selection runs on wave 0 (see select_topk.hpp) while the other waves build
// the next level's rotated queries.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "recsa_internal.hpp"
#include "select_topk.hpp"

namespace recsa {
namespace {

constexpr int kMaxCandidates = 4096;   // the LDS selection handles up to 64 logits per lane

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

__device__ __forceinline__ float row_sum16(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false));
    return v;   // the 16-lane row sum, in the row's lane 15
}

// Candidates of level l of a row over n_ctx tokens (pw = b^l), below a level that
// kept `kept_above` nodes.
__device__ __forceinline__ sel::Cands level_cands(int64_t n_ctx, int64_t pw, int32_t b, bool top,
                                                  int32_t kept_above) {
    sel::Cands c;
    const int64_t Nl = n_ctx / pw;
    c.b = b;
    c.top = top;
    if (top) {
        c.n = (int32_t)Nl;
        c.nchild = 0;
        c.orphan0 = 0;
    } else {
        const int64_t Nup = n_ctx / (pw * b);
        c.nchild = b * kept_above;
        c.orphan0 = (int32_t)(Nup * b);
        c.n = c.nchild + (int32_t)(Nl - Nup * b);
    }
    return c;
}

// Node id of candidate i = r*b + c (c < b).
__device__ __forceinline__ uint32_t node_rc(int32_t i, int32_t r, int32_t c, const sel::Cands &cd,
                                            const int32_t *parents) {
    if (cd.top) return (uint32_t)i;
    return i < cd.nchild ? (uint32_t)(parents[r] * cd.b + c) : (uint32_t)(cd.orphan0 + (i - cd.nchild));
}

// One pass over this slot's candidates of two levels: entries of level A (values,
// logits zA, kept ones flagged when maskA) fold into the running softmax, and the
// candidates of level S are scored into zS.  Either level may be empty.
template <typename T, int D, int NW, int CB>
__device__ __forceinline__ void fused_pass(
    sel::Cands A, const int32_t *parA, const float *zA, const uint8_t *flagA, bool maskA,
    const T *vA, sel::Cands S, const int32_t *parS, const T *kS, float *zS, uint8_t *flagS,
    const T *vS, const float *U, const float2 *rope, int32_t maxc, int32_t kmax, int slot, int sub,
    float scale, float &M, float &lsum, float *acc_a, float *acc_b) {
    constexpr int H2 = D / 2, PP = D / 32, NSLOT = NW * 4;
    constexpr uint32_t ROWB = D * sizeof(T);
    constexpr float kLog2e = 1.4426950408889634f;
    const int32_t b = A.n > 0 ? A.b : S.b;
    const int32_t nmax = A.n > S.n ? A.n : S.n;
    const int32_t R = (nmax + b - 1) / b;
    const int j0 = sub * PP;
    const char *vAb = reinterpret_cast<const char *>(vA) + j0 * sizeof(T);
    const char *kSb = reinterpret_cast<const char *>(kS) + j0 * sizeof(T);
    // vS: the S candidates are tokens, entries as soon as they are scored; their values
    // come in with their keys and join this slot's softmax online (M is then per slot)
    const bool online = vS != nullptr;
    const char *vSb = reinterpret_cast<const char *>(online ? vS : kS) + j0 * sizeof(T);
    for (int32_t c = slot; c < b; c += NSLOT) {
        float cr[PP], sr[PP];
        if (S.n > 0) load_cs<PP>(rope + (int64_t)c * H2 + j0, cr, sr);
        for (int32_t r0 = 0; r0 < R; r0 += CB) {
            uint32_t offA[CB], offS[CB];
            float ea[CB];
            #pragma unroll
            for (int t = 0; t < CB; ++t) {
                const int32_t r = r0 + t;
                const int32_t i = r * b + c;
                const int32_t ic = i < maxc ? i : maxc - 1;
                const int32_t rc = r < kmax ? r : kmax - 1;
                const bool okA = (i < A.n) && !(maskA && flagA[ic]);
                ea[t] = okA ? zA[ic] * kLog2e : -INFINITY;
                offA[t] = okA ? node_rc(i, rc, c, A, parA) * ROWB : 0u;
                offS[t] = (i < S.n) ? node_rc(i, rc, c, S, parS) * ROWB : 0u;
            }
            Raw<T, PP> va[CB], vb[CB], ka[CB], kb[CB], sa[CB], sb[CB];
            if (online) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    sa[t].load(reinterpret_cast<const T *>(vSb + offS[t]));
                    sb[t].load(reinterpret_cast<const T *>(vSb + offS[t] + H2 * sizeof(T)));
                }
            }
            if (A.n > 0) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    va[t].load(reinterpret_cast<const T *>(vAb + offA[t]));
                    vb[t].load(reinterpret_cast<const T *>(vAb + offA[t] + H2 * sizeof(T)));
                }
            }
            if (S.n > 0) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    ka[t].load(reinterpret_cast<const T *>(kSb + offS[t]));
                    kb[t].load(reinterpret_cast<const T *>(kSb + offS[t] + H2 * sizeof(T)));
                }
            }
            if (A.n > 0) {
                const float Ml2 = M * kLog2e;
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    const float pz = __builtin_amdgcn_exp2f(ea[t] - Ml2);    // 0 for -inf
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
            if (S.n > 0) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    const int32_t r = r0 + t;
                    const int32_t i = r * b + c;
                    const int32_t ru = (i < S.n) ? r : 0;
                    float ua[PP], ub[PP], fa[PP], fb[PP];
                    Vec<float, PP>::load(U + (size_t)ru * D + j0, ua);
                    Vec<float, PP>::load(U + (size_t)ru * D + H2 + j0, ub);
                    ka[t].get(fa);
                    kb[t].get(fb);
                    float dot = 0.f;
                    #pragma unroll
                    for (int p = 0; p < PP; ++p) {
                        const float ra = fa[p] * cr[p] - fb[p] * sr[p];
                        const float rb = fb[p] * cr[p] + fa[p] * sr[p];
                        dot += ua[p] * ra + ub[p] * rb;
                    }
                    dot = row_sum16(dot);
                    if (online) {
                        // the logit to all 16 lanes of the slot, then an online softmax step
                        const float z = scale * __shfl(dot, (threadIdx.x & 63) | 15);
                        if (i < S.n) {
                            const float Mn = fmaxf(M, z);
                            const float sc = __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
                            const float pz = __builtin_amdgcn_exp2f((z - Mn) * kLog2e);
                            float fa2[PP], fb2[PP];
                            sa[t].get(fa2);
                            sb[t].get(fb2);
                            lsum = lsum * sc + pz;
                            #pragma unroll
                            for (int p = 0; p < PP; ++p) {
                                acc_a[p] = acc_a[p] * sc + pz * fa2[p];
                                acc_b[p] = acc_b[p] * sc + pz * fb2[p];
                            }
                            M = Mn;
                        }
                    } else if (sub == 15 && i < S.n) {
                        zS[i] = scale * dot;
                        flagS[i] = 0;
                    }
                }
            }
        }
    }
}

template <typename T, int D, int NW, int CB, int KT>
__global__ __launch_bounds__(NW * 64) void descend_kernel(TreeView tv, DescendArgs a,
                                                          DebugView dbg) {
    constexpr int H2 = D / 2;
    constexpr int PP = D / 32;
    constexpr int NSLOT = NW * 4;
    constexpr float kLog2e = 1.4426950408889634f;
    extern __shared__ __align__(16) unsigned char smem[];
    const int32_t maxc = a.max_cand;
    const int32_t b = a.b;
    const int32_t nrank = (maxc + b - 1) / b;
    float *zbuf = reinterpret_cast<float *>(smem);                        // [2][maxc]
    float *U = zbuf + 2 * maxc;                                           // [nrank][D]
    float *red = U + (size_t)nrank * D;                                   // [NW][D]
    float *red_l = red + NW * D;                                          // [NW]
    float *red_m = red_l + NW;                                            // [NW]
    float *misc = red_m + NW;                                             // [4]
    unsigned char *scratch = reinterpret_cast<unsigned char *>(misc + 4); // selection scratch
    int32_t *kept = reinterpret_cast<int32_t *>(scratch + sel::kScratchBytes);  // [2][k]
    uint8_t *flagbuf = reinterpret_cast<uint8_t *>(kept + 2 * a.k);       // [2][maxc]

    const int64_t row = blockIdx.x;
    const int64_t qi = row / a.Hq;
    const int h = (int)(row - qi * a.Hq);
    const int g = h / a.G;
    int64_t n_ctx = a.ctx_base + qi * a.ctx_step;
    // multi-sequence decode: this query's sequence, as byte offsets from sequence 0's buffers
    int64_t dk = 0, dv = 0, dt = 0;
    if (a.seqs != nullptr || a.n_inline > 0) {
        const SeqEntry e = a.n_inline > 0 ? a.seq_inline[qi] : a.seqs[qi];
        const SeqEntry e0 = a.n_inline > 0 ? a.seq_inline[0] : a.seqs[0];
        n_ctx = e.length;
        dk = static_cast<const char *>(e.k_cache) - static_cast<const char *>(e0.k_cache);
        dv = static_cast<const char *>(e.v_cache) - static_cast<const char *>(e0.v_cache);
        dt = static_cast<const char *>(e.tree) - static_cast<const char *>(e0.tree);
    }
    // level l's keys / values of KV head g (l >= 1), in this query's tree
    auto lkey = [&](int l) {
        return reinterpret_cast<const T *>(static_cast<const char *>(tv.key[l]) + dt) +
               (int64_t)g * tv.node_cap[l] * D;
    };
    auto lval = [&](int l) {
        return reinterpret_cast<const T *>(static_cast<const char *>(tv.val[l]) + dt) +
               (int64_t)g * tv.node_cap[l] * D;
    };
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

    // The top level (H >= 1) has fewer than b nodes, all of them candidates at rank 0:
    // with at most 64 of them, their keys and child-offset rotations are loaded now,
    // alongside the query, instead of after the query's rotation is built.
    constexpr int CT = NSLOT >= 64 ? 1 : 64 / NSLOT;
    sel::Cands cA = level_cands(n_ctx, pwH, b, true, 0);
    const bool top_early = H >= 1 && cA.n <= CT * NSLOT;
    Raw<T, PP> tka[CT], tkb[CT];
    float tc[CT][PP], ts[CT][PP];
    if (top_early) {
        const T *kH = lkey(H);
        #pragma unroll
        for (int t = 0; t < CT; ++t) {
            const int32_t c = slot + t * NSLOT;
            const int32_t cc = c < cA.n ? c : 0;
            tka[t].load(kH + (int64_t)cc * D + j0);
            tkb[t].load(kH + (int64_t)cc * D + H2 + j0);
            load_cs<PP>(rope + (int64_t)cc * H2 + j0, tc[t], ts[t]);
        }
    }
    float qa[PP], qb[PP];
    {
        const T *qp = static_cast<const T *>(a.q) + row * D;
        Vec<T, PP>::load(qp + j0, qa);
        Vec<T, PP>::load(qp + H2 + j0, qb);
    }
    if (threadIdx.x == 0) {
        for (int l = H + 1; l <= nlev; ++l) {
            if (dbg.selected != nullptr)
                for (int t = 0; t < a.k; ++t) dbg.selected[(row * nlev + l - 1) * a.k + t] = -1;
            if (dbg.kth_gap != nullptr) dbg.kth_gap[row * nlev + l - 1] = NAN;
        }
    }

    const T *kcache = reinterpret_cast<const T *>(static_cast<const char *>(tv.k_cache) + dk) +
                      (int64_t)g * tv.cap * D;
    const T *vcache = reinterpret_cast<const T *>(static_cast<const char *>(tv.v_cache) + dv) +
                      (int64_t)g * tv.cap * D;

    // U[r] = R((n - r*b) theta) q for the ranks r < ceil(n / b) of a level with n
    // candidates; slots from first_slot on share the ranks.
    auto build_ranks = [&](int32_t n, int first_slot) {
        const int32_t R = (n + b - 1) / b;
        for (int32_t r = slot - first_slot; r < R; r += NSLOT - first_slot) {
            float c[PP], s[PP], ua[PP], ub[PP];
            load_cs<PP>(rope + (int64_t)(n - r * b) * H2 + j0, c, s);
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

    // ---- top level: score all of its candidates -------------------------------------
    {
        build_ranks(cA.n, 0);
        __syncthreads();
        if (top_early) {
            float ua[PP], ub[PP];
            Vec<float, PP>::load(U + j0, ua);
            Vec<float, PP>::load(U + H2 + j0, ub);
            float *zH = zbuf + (H & 1) * maxc;
            uint8_t *fH = flagbuf + (H & 1) * maxc;
            #pragma unroll
            for (int t = 0; t < CT; ++t) {
                const int32_t c = slot + t * NSLOT;
                float fa[PP], fb[PP];
                tka[t].get(fa);
                tkb[t].get(fb);
                float dot = 0.f;
                #pragma unroll
                for (int p = 0; p < PP; ++p) {
                    const float ra = fa[p] * tc[t][p] - fb[p] * ts[t][p];
                    const float rb = fb[p] * tc[t][p] + fa[p] * ts[t][p];
                    dot += ua[p] * ra + ub[p] * rb;
                }
                dot = row_sum16(dot);
                if (sub == 15 && c < cA.n) {
                    zH[c] = a.scale * dot;
                    fH[c] = 0;
                }
            }
        } else {
            sel::Cands none = cA;
            none.n = 0;
            const T *kH = H == 0 ? kcache : lkey(H);
            // with no level above the tokens, the top candidates are tokens: entries at once
            fused_pass<T, D, NW, CB>(none, kept, zbuf, flagbuf, false, kH, cA, kept, kH,
                                     zbuf + (H & 1) * maxc, flagbuf + (H & 1) * maxc,
                                     H == 0 ? vcache : nullptr, U, rope, maxc, a.k, slot, sub, a.scale,
                                     M, lsum, acc_a, acc_b);
        }
        keys_scored += cA.n;
    }

    // Levels H..1: select level l, then one pass over level l's entries and level l-1's
    // candidates.  At l = 1 those are tokens, which join the softmax as they are scored,
    // so the tokens' keys and values come in one round trip.
    int64_t pw = pwH;
    for (int l = H; l >= 1; --l, pw /= b) {
        __syncthreads();
        float *zA = zbuf + (l & 1) * maxc;
        uint8_t *flagA = flagbuf + (l & 1) * maxc;
        const int32_t mA = (l > 0) ? (a.k < cA.n ? a.k : cA.n) : 0;
        const int32_t *parentsA = kept + ((l + 1) & 1) * a.k;
        int32_t *keptA = kept + (l & 1) * a.k;
        sel::Cands cS = cA;
        cS.n = 0;
        if (l > 0) cS = level_cands(n_ctx, pw / b, b, false, mA);
        // ---- selection at level l (wave 0); the other waves build level l-1's ranks -----
        if (wave == 0) {
            if (l > 0) {
                if constexpr (KT > 0) {
                    if (cA.n <= 64 * KT)
                        sel::select<KT>(zA, flagA, keptA, mA, cA, parentsA, lane, scratch, misc);
                    else
                        sel::select<0>(zA, flagA, keptA, mA, cA, parentsA, lane, scratch, misc);
                } else {
                    sel::select<0>(zA, flagA, keptA, mA, cA, parentsA, lane, scratch, misc);
                }
                if (lane == 0 && dbg.kth_gap != nullptr)
                    dbg.kth_gap[row * nlev + l - 1] = misc[1] - misc[2];
                if (dbg.selected != nullptr) {
                    int32_t *ds = dbg.selected + (row * nlev + l - 1) * a.k;
                    for (int q = lane; q < a.k; q += 64) ds[q] = q < mA ? keptA[q] : -1;
                }
            } else {
                float mx = -INFINITY;
                for (int32_t i = lane; i < cA.n; i += 64) mx = fmaxf(mx, zA[i]);
                #pragma unroll
                for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
                if (lane == 0) misc[0] = mx;
            }
        } else if (l > 0) {
            build_ranks(cS.n, 4);
        }
        __syncthreads();

        // ---- fused pass: entries of level l, candidates of level l-1 ---------------------
        const float Mn = fmaxf(M, misc[0]);
        const float corr = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
        lsum *= corr;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { acc_a[p] *= corr; acc_b[p] *= corr; }
        M = Mn;
        const T *vA = l == 0 ? vcache : lval(l);
        const T *kS = l == 1 ? kcache : l > 1 ? lkey(l - 1) : vA;
        fused_pass<T, D, NW, CB>(cA, parentsA, zA, flagA, l > 0, vA, cS, keptA, kS,
                                 zbuf + ((l + 1) & 1) * maxc, flagbuf + ((l + 1) & 1) * maxc,
                                 l == 1 ? vcache : nullptr, U, rope, maxc, a.k, slot, sub, a.scale, M,
                                 lsum, acc_a, acc_b);
        keys_scored += cS.n;
        cA = cS;
    }

    // combine the slots: each has its own running max after the tokens; rescale to the
    // largest, then add the four lane groups by shuffles and the waves through LDS
    {
        float mw = fmaxf(M, __shfl_xor(M, 16));
        mw = fmaxf(mw, __shfl_xor(mw, 32));
        if (lane == 0) red_m[wave] = mw;
        __syncthreads();
        float mf = red_m[0];
        for (int w = 1; w < NW; ++w) mf = fmaxf(mf, red_m[w]);
        const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M - mf) * kLog2e);
        lsum *= sc;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { acc_a[p] *= sc; acc_b[p] *= sc; }
    }
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
    return sizeof(float) * (2 * (size_t)maxc + nrank * D + (size_t)NW * D + 2 * NW + 4) +
           sel::kScratchBytes + sizeof(int32_t) * 2 * (size_t)k + 2 * (size_t)maxc;
}

template <typename T, int D, int NW, int CB, int KT>
hipError_t launch_descend_t(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                            hipStream_t s) {
    const size_t smem = descend_smem<NW>(a.max_cand, a.k, a.b, D);
    if (smem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)descend_kernel<T, D, NW, CB, KT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((descend_kernel<T, D, NW, CB, KT>), dim3((unsigned)a.rows), dim3(NW * 64),
                       smem, s, tv, a, dbg);
    return hipGetLastError();
}

// Logits per lane the selection keeps in registers, from the widest level.
template <typename T, int D, int NW, int CB>
hipError_t launch_kt(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                     hipStream_t s) {
    const int32_t n = a.max_cand;
    if (n <= 64 * 2) return launch_descend_t<T, D, NW, CB, 2>(tv, a, dbg, s);
    if (n <= 64 * 5) return launch_descend_t<T, D, NW, CB, 5>(tv, a, dbg, s);
    if (n <= 64 * 9) return launch_descend_t<T, D, NW, CB, 9>(tv, a, dbg, s);
    if (n <= 64 * 17) return launch_descend_t<T, D, NW, CB, 17>(tv, a, dbg, s);
    return launch_descend_t<T, D, NW, CB, 0>(tv, a, dbg, s);
}

// Launch shape: (waves per row, ranks per slot per pass).
// RECSA_DESCEND_SHAPE="NW,CB" overrides the choice (for tuning sweeps).
template <typename T, int D>
hipError_t dispatch(const TreeView &tv, const DescendArgs &a, const DebugView &dbg, hipStream_t s) {
    // decode (one context length for all rows): more candidates per slot in flight;
    // prefill (many rows): fewer registers, more rows resident per CU
    int nw = 4, cb = a.ctx_step == 0 ? 4 : 2;
    if (const char *e = getenv("RECSA_DESCEND_SHAPE")) {
        int x = 0, y = 0;
        if (sscanf(e, "%d,%d", &x, &y) == 2) { nw = x; cb = y; }
    }
    if (nw == 8 && cb == 4) return launch_kt<T, D, 8, 4>(tv, a, dbg, s);
    if (nw == 4 && cb == 2) return launch_kt<T, D, 4, 2>(tv, a, dbg, s);
    return launch_kt<T, D, 4, 4>(tv, a, dbg, s);
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
