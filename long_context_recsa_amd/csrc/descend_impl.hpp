// Level-wise descent with candidate-index RoPE and the mixed softmax, for
// decode and (row by row) for causal prefill, on gfx950: the kernel templates,
// instantiated by descend_kernels.hip (one head per row) and descend_grouped_*.hip
// (a KV group's heads per row, sharing one selection).
//
// RecSA, abstract (sentences on selection and on RoPE): a level above the tokens
// keeps no more than k of its candidates; every candidate it drops contributes its
// summary to the same softmax that the exact tokens reached at the bottom join;
// the rotary position of an entry is its rank in the candidate list of its level.
// The query's position at a level is that level's candidate count n.
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
#pragma once
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "recsa_internal.hpp"
#include "select_topk.hpp"

namespace recsa {
namespace descend {


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

// Lane 15 of each 16-lane DPP row, to every lane of that row (row_newbcast:15).
__device__ __forceinline__ float row_bcast15(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x15F, 0xf, 0xf, false));
}

// A wave-uniform 64-bit value held in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Candidates of level l of a row, from its node counts Nl = N_l and Nup = N_{l+1}
// (N_l = floor(n_ctx / b^l)), below a level that kept `kept_above` nodes.
__device__ __forceinline__ sel::Cands level_cands(int32_t Nl, int32_t Nup, int32_t b, bool top,
                                                  int32_t kept_above) {
    sel::Cands c;
    c.b = b;
    c.bmul = sel::fanout_magic((uint32_t)b);
    c.top = top;
    if (top) {
        c.n = Nl;
        c.nchild = 0;
        c.orphan0 = 0;
    } else {
        c.nchild = b * kept_above;
        c.orphan0 = Nup * b;
        c.n = c.nchild + (Nl - Nup * b);
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
// logits zA, kept ones flagged) fold into the running softmax, and the candidates of
// level S are scored into zS.  HAS_A: level A has entries (not so above the top);
// ONLINE: the S candidates are tokens, entries as soon as they are scored, whose
// values (vS) come in with their keys and join this slot's softmax online (M is
// then per slot).  Level S is never empty.
//
// GS query heads share the pass (GS > 1: one selection per KV group).  Head j's logits
// are row j of zA / zS (rows zstride apart) and its rotated queries start at U + j * ustride;
// each value or key row is loaded once for all GS heads.  With GS > 1 the group score
// (the sum of the heads' logits) goes to gS for the selection, and lane 15 of each slot
// keeps, in smax, the largest logit per head that it scored.
//
// The slot's batches (child offset c, CB ranks) run two at a time (one for a group of
// eight heads): both batches' loads are issued before the first is folded in, so a
// pass waits on memory about half as often as batches it has.  Which loads a batch issues is fixed at compile time (no
// branch around a load), which lets the compiler wait for the first batch's loads
// alone; an odd last batch is paired with a dead one whose loads read row 0.
template <typename T, int D, int NW, int CB, int GS, bool HAS_A, bool ONLINE>
__device__ __forceinline__ void fused_pass(
    sel::Cands A, const int32_t *parA, const float *zA, const uint8_t *flagA,
    const T *vA, sel::Cands S, const int32_t *parS, const T *kS, float *zS, float *gS,
    uint8_t *flagS, const T *vS, const float *U, int32_t ustride, const float2 *rope,
    int32_t maxc, int32_t zstride, int32_t kmax, int slot, int sub, float scale, float (&M)[GS],
    float (&lsum)[GS], float (&acc_a)[GS][D / 32], float (&acc_b)[GS][D / 32],
    float (&smax)[GS]) {
    constexpr int H2 = D / 2, PP = D / 32, NSLOT = NW * 4;
    constexpr uint32_t ROWB = D * sizeof(T);
    constexpr float kLog2e = 1.4426950408889634f;
    const int32_t b = S.b;
    const int32_t nmax = A.n > S.n ? A.n : S.n;
    const int32_t R = (nmax + b - 1) / b;
    const int j0 = sub * PP;
    // uniform bases with the lane's slice in the 32-bit offsets: the loads can take a
    // scalar base and one offset register each
    const uint32_t j0b = (uint32_t)(j0 * sizeof(T));
    const char *vAb = reinterpret_cast<const char *>(vA);
    const char *kSb = reinterpret_cast<const char *>(kS);
    const char *vSb = reinterpret_cast<const char *>(vS);
    // The slot's batches: child offsets c = slot, slot + NSLOT, ... and for each the ranks
    // in groups of CB, in that order, as one flat sequence.
    struct Batch {
        int32_t c, r0;
        bool live;
        float ea[CB][GS];
        float cr[PP], sr[PP];
        Raw<T, PP> va[CB], vb[CB], ka[CB], kb[CB], sa[CB], sb[CB];
    };
    // 12 waves (48 slots, not a multiple of the fanout): the (child offset, rank
    // group) pairs form one flat sequence f = c + b * g, and slot s takes f = s,
    // s + NSLOT, ... (ci counts the slot's batches; nrb is 1)
    constexpr bool kFlat = NW == 12;
    const int32_t ngroups = (R + CB - 1) / CB;
    const int32_t nflat = b * ngroups;
    const int32_t nc = kFlat ? (slot < nflat ? (nflat - slot + NSLOT - 1) / NSLOT : 0)
                             : (slot < b ? (b - slot + NSLOT - 1) / NSLOT : 0);
    const int32_t nrb = kFlat ? 1 : ngroups;
    const int32_t NB = nc * nrb;
    auto issue = [&](Batch &B, int32_t ci, int32_t ri, bool live) __attribute__((always_inline)) {
        B.live = live;
        if constexpr (kFlat) {
            const uint32_t f = (uint32_t)(slot + ci * NSLOT);
            const int32_t g = (int32_t)__umulhi(f, S.bmul);
            B.c = live ? (int32_t)f - g * b : 0;
            B.r0 = live ? g * CB : 0;
        } else {
            B.c = live ? slot + ci * NSLOT : 0;
            B.r0 = live ? ri * CB : 0;
        }
        const int32_t c = B.c;
        load_cs<PP>(rope + (int64_t)c * H2 + j0, B.cr, B.sr);
        uint32_t offA[CB], offS[CB];
        #pragma unroll
        for (int t = 0; t < CB; ++t) {
            const int32_t r = B.r0 + t;
            const int32_t i = r * b + c;
            const int32_t ic = i < maxc ? i : maxc - 1;
            const int32_t rc = r < kmax ? r : kmax - 1;
            if constexpr (HAS_A) {
                const bool okA = live && (i < A.n) && !flagA[ic];
                #pragma unroll
                for (int j = 0; j < GS; ++j) B.ea[t][j] = okA ? zA[j * zstride + ic] * kLog2e : -INFINITY;
                offA[t] = (okA ? node_rc(i, rc, c, A, parA) * ROWB : 0u) + j0b;
            }
            offS[t] = ((live && i < S.n) ? node_rc(i, rc, c, S, parS) * ROWB : 0u) + j0b;
        }
        if constexpr (ONLINE) {
            #pragma unroll
            for (int t = 0; t < CB; ++t) {
                B.sa[t].load(reinterpret_cast<const T *>(vSb + offS[t]));
                B.sb[t].load(reinterpret_cast<const T *>(vSb + offS[t] + H2 * sizeof(T)));
            }
        }
        if constexpr (HAS_A) {
            #pragma unroll
            for (int t = 0; t < CB; ++t) {
                B.va[t].load(reinterpret_cast<const T *>(vAb + offA[t]));
                B.vb[t].load(reinterpret_cast<const T *>(vAb + offA[t] + H2 * sizeof(T)));
            }
        }
        #pragma unroll
        for (int t = 0; t < CB; ++t) {
            B.ka[t].load(reinterpret_cast<const T *>(kSb + offS[t]));
            B.kb[t].load(reinterpret_cast<const T *>(kSb + offS[t] + H2 * sizeof(T)));
        }
    };
    auto consume = [&](const Batch &B) __attribute__((always_inline)) {
        const int32_t c = B.c;
        if constexpr (HAS_A) {
            #pragma unroll
            for (int t = 0; t < CB; ++t) {
                float fa[PP], fb[PP];
                B.va[t].get(fa);
                B.vb[t].get(fb);
                #pragma unroll
                for (int j = 0; j < GS; ++j) {
                    const float pz = __builtin_amdgcn_exp2f(B.ea[t][j] - M[j] * kLog2e);  // 0 for -inf
                    lsum[j] += pz;
                    #pragma unroll
                    for (int p = 0; p < PP; ++p) {
                        acc_a[j][p] += pz * fa[p];
                        acc_b[j][p] += pz * fb[p];
                    }
                }
            }
        }
        // non-ONLINE: each rank's logits stay in lane 15 of the slot until the batch's
        // ranks are all scored, then go to LDS under one branch (ranks past the level's
        // candidates write the pad slot at index maxc, which nothing reads)
        float zk[ONLINE ? 1 : CB][GS], gk[ONLINE ? 1 : CB];
        #pragma unroll
        for (int t = 0; t < CB; ++t) {
            const int32_t r = B.r0 + t;
            const int32_t i = r * b + c;
            const int32_t ru = (i < S.n) ? r : 0;
            float fa[PP], fb[PP], ra[PP], rb[PP];
            B.ka[t].get(fa);
            B.kb[t].get(fb);
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                ra[p] = fa[p] * B.cr[p] - fb[p] * B.sr[p];
                rb[p] = fb[p] * B.cr[p] + fa[p] * B.sr[p];
            }
            float fa2[PP], fb2[PP];
            if constexpr (ONLINE) {
                B.sa[t].get(fa2);
                B.sb[t].get(fb2);
            }
            float gsum = 0.f;
            #pragma unroll
            for (int j = 0; j < GS; ++j) {
                float ua[PP], ub[PP];
                const float *Uj = U + (size_t)j * ustride + (size_t)ru * D;
                Vec<float, PP>::load(Uj + j0, ua);
                Vec<float, PP>::load(Uj + H2 + j0, ub);
                float dot = 0.f;
                #pragma unroll
                for (int p = 0; p < PP; ++p) dot += ua[p] * ra[p] + ub[p] * rb[p];
                dot = row_sum16(dot);
                if constexpr (ONLINE) {
                    // the logit to all 16 lanes of the slot, then an online softmax step;
                    // a rank past the level's candidates leaves the state as it is (scale
                    // 1, weight 0: its value row is row 0, finite)
                    const float z = scale * row_bcast15(dot);
                    const bool ok = i < S.n;
                    const float Mn = ok ? fmaxf(M[j], z) : M[j];
                    const float sc = ok ? __builtin_amdgcn_exp2f((M[j] - Mn) * kLog2e) : 1.f;
                    const float pz = ok ? __builtin_amdgcn_exp2f((z - Mn) * kLog2e) : 0.f;
                    lsum[j] = lsum[j] * sc + pz;
                    #pragma unroll
                    for (int p = 0; p < PP; ++p) {
                        acc_a[j][p] = acc_a[j][p] * sc + pz * fa2[p];
                        acc_b[j][p] = acc_b[j][p] * sc + pz * fb2[p];
                    }
                    M[j] = Mn;
                } else {
                    const float z = scale * dot;
                    zk[t][j] = z;
                    if constexpr (GS > 1) {
                        gsum += z;
                        smax[j] = fmaxf(smax[j], i < S.n ? z : -INFINITY);
                    }
                }
            }
            if constexpr (!ONLINE) gk[t] = gsum;
        }
        if constexpr (!ONLINE) {
            if (sub == 15) {
                #pragma unroll
                for (int t = 0; t < CB; ++t) {
                    const int32_t i = (B.r0 + t) * b + c;
                    const int32_t is = i < S.n ? i : maxc;
                    #pragma unroll
                    for (int j = 0; j < GS; ++j) zS[j * zstride + is] = zk[t][j];
                    if constexpr (GS > 1) gS[is] = gk[t];
                    flagS[is] = 0;
                }
            }
        }
    };
    // A group of eight heads keeps 64 accumulators per lane: one batch in flight.
    constexpr bool kPair = GS < 8;
    Batch B0, B1;
    int32_t ci = 0, ri = 0;
    for (int32_t k = 0; k < NB; k += kPair ? 2 : 1) {
        issue(B0, ci, ri, true);
        if (++ri == nrb) { ri = 0; ++ci; }
        if constexpr (kPair) {
            const bool two = k + 1 < NB;
            issue(B1, ci, ri, two);
            if (two && ++ri == nrb) { ri = 0; ++ci; }
            consume(B0);
            if (two) consume(B1);
        } else {
            consume(B0);
        }
    }
}

// The row's node counts N_0..N_H (N_l = floor(n_ctx / b^l)) in LDS: 32-bit entries,
// room for every level the capacity allows, padded to keep 16-byte alignment.
constexpr int kNodeTab = (kMaxLevels + 4) & ~3;

template <int NW, int GS>
struct Smem {
    // logit rows per buffer: one per head, then (GS > 1) the group score
    static constexpr int NZ = GS == 1 ? 1 : GS + 1;
    // logit rows are padded to a multiple of 4 floats, so every array after them is 16-byte aligned
    // with room for a pad slot at index maxc
    __host__ __device__ static int32_t zstride(int32_t maxc) { return (maxc + 4) & ~3; }
    __host__ __device__ static int32_t fstride(int32_t maxc) { return maxc + 4; }
    static size_t bytes(int32_t maxc, int32_t k, int32_t b, int D) {
        const size_t nrank = ((size_t)maxc + b - 1) / b;
        const size_t floats = 2 * NZ * (size_t)zstride(maxc) + GS * nrank * D + (size_t)NW * GS * D +
                              2 * (size_t)NW * GS + (GS > 1 ? 2 * (size_t)NW * GS + (size_t)GS * D : 0) + 4 +
                              kNodeTab;
        return sizeof(float) * floats + sel::kScratchBytes + sizeof(int32_t) * 2 * (size_t)k +
               2 * (size_t)fstride(maxc);
    }
};

// One row is one query and GS query heads of one KV head: GS = 1 (every head selects
// for itself) or GS = G (the group's heads share one selection per level).
// MINW: waves per SIMD the kernel must leave room for (4 lets two 8-wave rows share a
// compute unit; the compiler then keeps to 128 registers).
template <typename T, int D, int NW, int CB, int KT, int GS, int MINW = 1>
__global__ __launch_bounds__(NW * 64, MINW) void descend_kernel(TreeView tv, DescendArgs a,
                                                          DebugView dbg) {
    constexpr int H2 = D / 2;
    constexpr int PP = D / 32;
    constexpr int NSLOT = NW * 4;
    constexpr int NZ = Smem<NW, GS>::NZ;
    constexpr float kLog2e = 1.4426950408889634f;
    extern __shared__ __align__(16) unsigned char smem[];
    const int32_t maxc = a.max_cand;
    const int32_t b = a.b;
    const int32_t nrank = (maxc + b - 1) / b;
    const int32_t mz = Smem<NW, GS>::zstride(maxc);
    const int32_t fs = Smem<NW, GS>::fstride(maxc);
    float *zbuf = reinterpret_cast<float *>(smem);                        // [2][NZ][mz]
    float *U = zbuf + 2 * NZ * mz;                                        // [GS][nrank][D]
    float *red = U + (size_t)GS * nrank * D;                              // [NW][GS][D]
    float *red_l = red + NW * GS * D;                                     // [NW][GS]
    float *red_m = red_l + NW * GS;                                       // [NW][GS]
    float *lmax = red_m + NW * GS;                    // GS > 1: [2][NW][GS] level maxima
    float *qs = lmax + (GS > 1 ? 2 * NW * GS : 0);    // GS > 1: [GS][D] the queries
    float *misc = qs + (GS > 1 ? GS * D : 0);                             // [4]
    int32_t *ntab = reinterpret_cast<int32_t *>(misc + 4);                // [kNodeTab] N_l
    unsigned char *scratch = reinterpret_cast<unsigned char *>(ntab + kNodeTab); // selection scratch
    int32_t *kept = reinterpret_cast<int32_t *>(scratch + sel::kScratchBytes);  // [2][k]
    uint8_t *flagbuf = reinterpret_cast<uint8_t *>(kept + 2 * a.k);       // [2][fs]
    // head j's logits and the selection score of buffer `buf`
    auto zrow = [&](int buf, int j) { return zbuf + (size_t)(buf * NZ + j) * mz; };
    auto zsel = [&](int buf) { return zbuf + (size_t)(buf * NZ + (GS == 1 ? 0 : GS)) * mz; };

    // Workgroups go to the 8 XCDs round robin (block index mod 8) and every XCD has its
    // own L2.  One head per row: block x is the row of rank (x mod 8) * R/8 + x / 8 in
    // KV-head-major order (KV head, query, head within the group), so each XCD takes a
    // contiguous run of rows that read the same KV head's tree (at 8 KV heads, one head
    // per XCD).  A group row (GS = G) already has its KV head at x mod 8.
    // (rows < 2^31, checked on the host: 32-bit index arithmetic)
    uint32_t row = blockIdx.x;
    if constexpr (GS == 1) {
        constexpr uint32_t kXcds = 8;
        const uint32_t R = gridDim.x;
        if (R % kXcds == 0) {
            const uint32_t rp = (blockIdx.x % kXcds) * (R / kXcds) + blockIdx.x / kXcds;
            const uint32_t per_g = (R / (uint32_t)a.Hq) * (uint32_t)a.G;   // rows of one KV head
            const uint32_t gg = rp / per_g, rem = rp - gg * per_g;
            const uint32_t qq = rem / (uint32_t)a.G;
            row = qq * (uint32_t)a.Hq + gg * (uint32_t)a.G + (rem - qq * (uint32_t)a.G);
        }
    }
    const uint32_t rows_per_q = (uint32_t)(a.Hq / GS);
    const uint32_t qi = row / rows_per_q;
    const int h0 = (int)(row - qi * rows_per_q) * GS;     // first query head of the row
    const int g = h0 / a.G;
    int64_t n_ctx = a.ctx_base + (int64_t)qi * a.ctx_step;
    // multi-sequence decode: this query's sequence, as byte offsets from sequence 0's buffers
    int64_t dk = 0, dv = 0, dt = 0;
    if (a.seqs != nullptr || a.n_inline > 0) {
        const SeqEntry e = a.n_inline > 0 ? a.seq_inline[qi] : a.seqs[qi];
        const SeqEntry e0 = a.n_inline > 0 ? a.seq_inline[0] : a.seqs[0];
        n_ctx = e.length;
        dk = static_cast<const char *>(e.k_cache) - static_cast<const char *>(e0.k_cache);
        dv = static_cast<const char *>(e.v_cache) - static_cast<const char *>(e0.v_cache);
        dt = static_cast<const char *>(e.tree) - static_cast<const char *>(e0.tree);
        // the same for every lane: keep them (and the bases built from them) scalar
        dk = uniform64(dk);
        dv = uniform64(dv);
        dt = uniform64(dt);
        n_ctx = uniform64(n_ctx);
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
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int grp = lane >> 4, sub = lane & 15;
    const int slot = wave * 4 + grp;
    const int j0 = sub * PP;
    const int nlev = tv.n_levels;
    const float2 *rope = tv.rope;

    // levels above the tokens for this row, H = max{l : n_ctx / b^l >= 1}, and the node
    // counts N_l by repeated 32-bit division (n_ctx < 2^31; floor(N_l / b) = N_{l+1})
    int H = 0;
    int32_t NH = (int32_t)n_ctx;
    if (threadIdx.x == 0) ntab[0] = NH;
    while (NH >= b) {
        NH /= b;
        ++H;
        if (threadIdx.x == 0) ntab[H] = NH;
    }

    // The top level (H >= 1) has fewer than b nodes, all of them candidates at rank 0:
    // with at most 64 of them, their keys and child-offset rotations are loaded now,
    // alongside the query, instead of after the query's rotation is built.
    constexpr int CT = NSLOT >= 64 ? 1 : 64 / NSLOT;
    sel::Cands cA = level_cands(NH, 0, b, true, 0);
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
    // The top level has one rank (r = 0) and the query sits at its candidate count: the
    // rotation R(n theta) of its rotated queries comes in with the query.
    float topc[PP], tops[PP];
    load_cs<PP>(rope + (int64_t)cA.n * H2 + j0, topc, tops);
    // the row's queries: in registers for one head, in LDS for a group
    float qa[PP], qb[PP];
    const T *qrow = static_cast<const T *>(a.q) + (int64_t)(qi * a.Hq + h0) * D;
    if constexpr (GS == 1) {
        Vec<T, PP>::load(qrow + j0, qa);
        Vec<T, PP>::load(qrow + H2 + j0, qb);
    } else {
        for (int e = threadIdx.x * 2; e < GS * D; e += NW * 64 * 2) {
            float v[2];
            Vec<T, 2>::load(qrow + e, v);
            qs[e] = v[0];
            qs[e + 1] = v[1];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        for (int l = H + 1; l <= nlev; ++l) {
            if (dbg.selected != nullptr)
                for (int t = 0; t < a.k; ++t) dbg.selected[((int64_t)row * nlev + l - 1) * a.k + t] = -1;
            if (dbg.kth_gap != nullptr) dbg.kth_gap[(int64_t)row * nlev + l - 1] = NAN;
        }
    }

    const T *kcache = reinterpret_cast<const T *>(static_cast<const char *>(tv.k_cache) + dk) +
                      (int64_t)g * tv.cap * D;
    const T *vcache = reinterpret_cast<const T *>(static_cast<const char *>(tv.v_cache) + dv) +
                      (int64_t)g * tv.cap * D;

    // U[j][r] = R((n - r*b) theta) q_j for the ranks r < ceil(n / b) of a level with n
    // candidates; slots from first_slot on share the (head, rank) pairs.
    const int32_t ustride = nrank * D;
    auto build_ranks = [&](int32_t n, int first_slot, bool top) {
        const int32_t R = (n + b - 1) / b;
        for (int32_t x = slot - first_slot; x < GS * R; x += NSLOT - first_slot) {
            const int j = GS == 1 ? 0 : x / R;
            const int32_t r = x - j * R;
            float c[PP], s[PP], ua[PP], ub[PP], xa[PP], xb[PP];
            if constexpr (GS == 1) {
                #pragma unroll
                for (int p = 0; p < PP; ++p) { xa[p] = qa[p]; xb[p] = qb[p]; }
            } else {
                Vec<float, PP>::load(qs + j * D + j0, xa);
                Vec<float, PP>::load(qs + j * D + H2 + j0, xb);
            }
            if (top) {
                #pragma unroll
                for (int p = 0; p < PP; ++p) { c[p] = topc[p]; s[p] = tops[p]; }
            } else {
                load_cs<PP>(rope + (int64_t)(n - r * b) * H2 + j0, c, s);
            }
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                ua[p] = xa[p] * c[p] - xb[p] * s[p];
                ub[p] = xb[p] * c[p] + xa[p] * s[p];
            }
            Vec<float, PP>::store(U + (size_t)j * ustride + (size_t)r * D + j0, ua);
            Vec<float, PP>::store(U + (size_t)j * ustride + (size_t)r * D + H2 + j0, ub);
        }
    };
    // GS > 1: the per-head maxima a pass found (lane 15 of each slot) go to lmax[buf]
    auto publish_max = [&](float (&smax)[GS], int buf) {
        if constexpr (GS > 1) {
            #pragma unroll
            for (int j = 0; j < GS; ++j) {
                float v = fmaxf(smax[j], __shfl_xor(smax[j], 16));
                v = fmaxf(v, __shfl_xor(v, 32));
                if (lane == 15) lmax[(buf * NW + wave) * GS + j] = v;
                smax[j] = -INFINITY;
            }
        }
    };

    float M[GS], lsum[GS], acc_a[GS][PP], acc_b[GS][PP], smax[GS];
    #pragma unroll
    for (int j = 0; j < GS; ++j) {
        M[j] = -INFINITY;
        lsum[j] = 0.f;
        smax[j] = -INFINITY;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { acc_a[j][p] = 0.f; acc_b[j][p] = 0.f; }
    }
    int64_t keys_scored = 0;

    // ---- top level: score all of its candidates -------------------------------------
    {
        build_ranks(cA.n, 0, true);
        __syncthreads();
        if (top_early) {
            const int buf = H & 1;
            uint8_t *fH = flagbuf + buf * fs;
            #pragma unroll
            for (int t = 0; t < CT; ++t) {
                const int32_t c = slot + t * NSLOT;
                float fa[PP], fb[PP], ra[PP], rb[PP];
                tka[t].get(fa);
                tkb[t].get(fb);
                #pragma unroll
                for (int p = 0; p < PP; ++p) {
                    ra[p] = fa[p] * tc[t][p] - fb[p] * ts[t][p];
                    rb[p] = fb[p] * tc[t][p] + fa[p] * ts[t][p];
                }
                float gsum = 0.f;
                #pragma unroll
                for (int j = 0; j < GS; ++j) {
                    float ua[PP], ub[PP];
                    Vec<float, PP>::load(U + (size_t)j * ustride + j0, ua);
                    Vec<float, PP>::load(U + (size_t)j * ustride + H2 + j0, ub);
                    float dot = 0.f;
                    #pragma unroll
                    for (int p = 0; p < PP; ++p) dot += ua[p] * ra[p] + ub[p] * rb[p];
                    dot = row_sum16(dot);
                    if (sub == 15 && c < cA.n) {
                        const float z = a.scale * dot;
                        zrow(buf, j)[c] = z;
                        gsum += z;
                        smax[j] = fmaxf(smax[j], z);
                    }
                }
                if (sub == 15 && c < cA.n) {
                    if constexpr (GS > 1) zsel(buf)[c] = gsum;
                    fH[c] = 0;
                }
            }
            publish_max(smax, buf);
        } else {
            sel::Cands none = cA;
            none.n = 0;
            const T *kH = H == 0 ? kcache : lkey(H);
            const int buf = H & 1;
            // with no level above the tokens, the top candidates are tokens: entries at once
            if (H == 0)
                fused_pass<T, D, NW, CB, GS, false, true>(none, kept, zbuf, flagbuf, kH, cA, kept, kH,
                                                          zrow(buf, 0), zsel(buf), flagbuf + buf * fs,
                                                          vcache, U, ustride, rope, maxc, mz, a.k, slot,
                                                          sub, a.scale, M, lsum, acc_a, acc_b, smax);
            else
                fused_pass<T, D, NW, CB, GS, false, false>(none, kept, zbuf, flagbuf, kH, cA, kept, kH,
                                                           zrow(buf, 0), zsel(buf), flagbuf + buf * fs,
                                                           nullptr, U, ustride, rope, maxc, mz, a.k, slot,
                                                           sub, a.scale, M, lsum, acc_a, acc_b, smax);
            if (H > 0) publish_max(smax, buf);
        }
        keys_scored += cA.n;
    }

    // Levels H..1: select level l, then one pass over level l's entries and level l-1's
    // candidates.  At l = 1 those are tokens, which join the softmax as they are scored,
    // so the tokens' keys and values come in one round trip.
    for (int l = H; l >= 1; --l) {
        __syncthreads();
        const int bufA = l & 1, bufS = (l + 1) & 1;
        uint8_t *flagA = flagbuf + bufA * fs;
        const int32_t mA = a.k < cA.n ? a.k : cA.n;
        const int32_t *parentsA = kept + bufS * a.k;
        int32_t *keptA = kept + bufA * a.k;
        const sel::Cands cS = level_cands(ntab[l - 1], ntab[l], b, false, mA);
        // ---- selection at level l (wave 0); the other waves build level l-1's ranks -----
        if (wave == 0) {
            const float *zA = zsel(bufA);
            if constexpr (KT > 0) {
                if (cA.n <= 64 * KT)
                    sel::select<KT>(zA, flagA, keptA, mA, cA, parentsA, lane, scratch, misc);
                else
                    sel::select<0>(zA, flagA, keptA, mA, cA, parentsA, lane, scratch, misc);
            } else {
                sel::select<0>(zA, flagA, keptA, mA, cA, parentsA, lane, scratch, misc);
            }
            if (lane == 0 && dbg.kth_gap != nullptr)
                dbg.kth_gap[(int64_t)row * nlev + l - 1] = misc[1] - misc[2];
            if (dbg.selected != nullptr) {
                int32_t *ds = dbg.selected + ((int64_t)row * nlev + l - 1) * a.k;
                for (int q = lane; q < a.k; q += 64) ds[q] = q < mA ? keptA[q] : -1;
            }
        } else {
            build_ranks(cS.n, 4, false);
        }
        __syncthreads();

        // ---- fused pass: entries of level l, candidates of level l-1 ---------------------
        // the running max moves to the largest logit of level l (per head)
        #pragma unroll
        for (int j = 0; j < GS; ++j) {
            float lm;
            if constexpr (GS == 1) {
                lm = misc[0];
            } else {
                lm = lmax[(bufA * NW) * GS + j];
                for (int w = 1; w < NW; ++w) lm = fmaxf(lm, lmax[(bufA * NW + w) * GS + j]);
            }
            const float Mn = fmaxf(M[j], lm);
            const float corr = (M[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M[j] - Mn) * kLog2e);
            lsum[j] *= corr;
            #pragma unroll
            for (int p = 0; p < PP; ++p) { acc_a[j][p] *= corr; acc_b[j][p] *= corr; }
            M[j] = Mn;
        }
        const T *vA = lval(l);
        const T *kS = l == 1 ? kcache : lkey(l - 1);
        if (l == 1)
            fused_pass<T, D, NW, CB, GS, true, true>(cA, parentsA, zrow(bufA, 0), flagA, vA, cS, keptA, kS,
                                                     zrow(bufS, 0), zsel(bufS), flagbuf + bufS * fs,
                                                     vcache, U, ustride, rope, maxc, mz, a.k, slot, sub,
                                                     a.scale, M, lsum, acc_a, acc_b, smax);
        else
            fused_pass<T, D, NW, CB, GS, true, false>(cA, parentsA, zrow(bufA, 0), flagA, vA, cS, keptA, kS,
                                                      zrow(bufS, 0), zsel(bufS), flagbuf + bufS * fs,
                                                      nullptr, U, ustride, rope, maxc, mz, a.k, slot, sub,
                                                      a.scale, M, lsum, acc_a, acc_b, smax);
        if (l > 1) publish_max(smax, bufS);
        keys_scored += cS.n;
        cA = cS;
    }

    // combine the slots, per head: each slot has its own running max after the tokens;
    // rescale to the largest, then add the four lane groups by shuffles and the waves
    // through LDS
    #pragma unroll
    for (int j = 0; j < GS; ++j) {
        float mw = fmaxf(M[j], __shfl_xor(M[j], 16));
        mw = fmaxf(mw, __shfl_xor(mw, 32));
        if (lane == 0) red_m[wave * GS + j] = mw;
    }
    __syncthreads();
    #pragma unroll
    for (int j = 0; j < GS; ++j) {
        float mf = red_m[j];
        for (int w = 1; w < NW; ++w) mf = fmaxf(mf, red_m[w * GS + j]);
        const float sc = (M[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M[j] - mf) * kLog2e);
        lsum[j] *= sc;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { acc_a[j][p] *= sc; acc_b[j][p] *= sc; }
        #pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            lsum[j] += __shfl_xor(lsum[j], off);
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                acc_a[j][p] += __shfl_xor(acc_a[j][p], off);
                acc_b[j][p] += __shfl_xor(acc_b[j][p], off);
            }
        }
        if (grp == 0) {
            float *rw = red + (size_t)(wave * GS + j) * D;
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                rw[j0 + p] = acc_a[j][p];
                rw[H2 + j0 + p] = acc_b[j][p];
            }
            if (sub == 0) red_l[wave * GS + j] = lsum[j];
        }
    }
    __syncthreads();
    // head j's output: slot j (and j + NSLOT, ...) adds the waves' partial sums
    for (int j = slot; j < GS; j += NSLOT) {
        float oa[PP], ob[PP], L = 0.f;
        #pragma unroll
        for (int p = 0; p < PP; ++p) { oa[p] = 0.f; ob[p] = 0.f; }
        for (int w = 0; w < NW; ++w) {
            const float *rw = red + (size_t)(w * GS + j) * D;
            L += red_l[w * GS + j];
            #pragma unroll
            for (int p = 0; p < PP; ++p) {
                oa[p] += rw[j0 + p];
                ob[p] += rw[H2 + j0 + p];
            }
        }
        #pragma unroll
        for (int p = 0; p < PP; ++p) { oa[p] /= L; ob[p] /= L; }
        const int64_t orow = (int64_t)qi * a.Hq + h0 + j;
        if (a.out_bf16) {
            bf16_t *o = static_cast<bf16_t *>(a.out) + orow * D;
            Vec<bf16_t, PP>::store(o + j0, oa);
            Vec<bf16_t, PP>::store(o + H2 + j0, ob);
        } else {
            float *o = static_cast<float *>(a.out) + orow * D;
            Vec<float, PP>::store(o + j0, oa);
            Vec<float, PP>::store(o + H2 + j0, ob);
        }
    }
    if (threadIdx.x == 0 && dbg.n_keys != nullptr) dbg.n_keys[row] = (int32_t)keys_scored;
}

template <typename T, int D, int NW, int CB, int KT, int GS, int MINW = 1>
hipError_t launch_descend_t(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                            hipStream_t s) {
    const size_t smem = Smem<NW, GS>::bytes(a.max_cand, a.k, a.b, D);
    if (smem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)descend_kernel<T, D, NW, CB, KT, GS, MINW>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((descend_kernel<T, D, NW, CB, KT, GS, MINW>), dim3((unsigned)(a.rows / GS)),
                       dim3(NW * 64), smem, s, tv, a, dbg);
    return hipGetLastError();
}

// Logits per lane the selection keeps in registers, from the widest level.
template <typename T, int D, int NW, int CB, int GS, int MINW = 1>
hipError_t launch_kt(const TreeView &tv, const DescendArgs &a, const DebugView &dbg,
                     hipStream_t s) {
    const int32_t n = a.max_cand;
    if (n <= 64 * 2) return launch_descend_t<T, D, NW, CB, 2, GS, MINW>(tv, a, dbg, s);
    if (n <= 64 * 5) return launch_descend_t<T, D, NW, CB, 5, GS, MINW>(tv, a, dbg, s);
    if (n <= 64 * 9) return launch_descend_t<T, D, NW, CB, 9, GS, MINW>(tv, a, dbg, s);
    if (n <= 64 * 17) return launch_descend_t<T, D, NW, CB, 17, GS, MINW>(tv, a, dbg, s);
    return launch_descend_t<T, D, NW, CB, 0, GS, MINW>(tv, a, dbg, s);
}

}  // namespace descend
}  // namespace recsa
