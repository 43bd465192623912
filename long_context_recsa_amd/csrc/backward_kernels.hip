// Backward of the mixed softmax with the selection held fixed, for gfx950.
//
// RecSA, abstract: the method is trained end to end from a Qwen3-4B
// initialisation, so the attention output's gradient must reach the query, the
// token keys and values and the pooler.  The softmax entries are the
// unselected candidates of every level (summary key and value) and the level-0
// tokens; selection itself is piecewise constant and carries no gradient.
//
// With z = s <rope(q, n), rope(key, i)> = s q . R_(i-n) key, p = softmax(z),
// out = sum p v, and dO the output's gradient:
//   dp_e = <dO, v_e>,  D = <dO, out> = sum_e p_e dp_e,  dz_e = p_e (dp_e - D),
//   dq = s sum_e dz_e R_(i-n) key_e,  dkey_e = s dz_e R_(n-i) q,  dv_e = p_e dO.
//
// bwd_rows: one workgroup per row (query, query head).  It runs the descent
// again (scores, the same selection rule as the forward, and an online
// softmax that also carries sum e^(z-M) dp, so D needs no output vector),
// then walks the entries a second time and adds dkey and dv to the token
// gradients (dk, dv) or to the per-level summary gradients in the workspace,
// with fp32 atomics: rows share entries.  Run in two phases (summaries and dq,
// then the token entries alone) it lets the tree pass below write the token
// gradients first, so they are never read back.
//
// bwd_tree: per level from the top down, one wave per node.  A node's value
// is the mean of its b children's, so each child gets dv / b; its key is the
// pooler over its b stored children's keys,
//   a_c = s_p w . x_c,  alpha = softmax(a),  key = sum alpha_c x_c,
// so with g = dkey: dx_c = alpha_c g + s_p da_c w and dw += s_p sum da_c x_c,
// da_c = alpha_c (<g, x_c> - sum alpha <g, x>).  Children belong to one node,
// so their gradients are read, added to and written without atomics; dw is
// added with atomics.  With write_children the children's gradients are
// written instead, and the rows' own entries of the child level are added
// afterwards: at level 1 that halves the traffic of the one pass that touches
// every token (the tokens' dk, dv are never read back); above it the
// parent-major path does the same with the summaries' gradients.  Storage
// rounding of summaries passes gradients through.
#include <math.h>

#include "recsa_internal.hpp"
#include "select_topk.hpp"

namespace recsa {
namespace {

constexpr int kNW = 4;                  // waves per row workgroup
constexpr int kNSlot = kNW * 4;         // 16-lane slots per row workgroup

__device__ __forceinline__ float row_sum16(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false));
    return v;   // the 16-lane row sum, in the row's lane 15
}

// the row sum of v, in all 16 lanes of the row
__device__ __forceinline__ float slot_sum(float v) {
    return __shfl(row_sum16(v), (int)(threadIdx.x & 63) | 15);
}

// PP consecutive (cos, sin) pairs of one RoPE table row
template <int PP>
__device__ __forceinline__ void load_cs(const float2 *p, float *c, float *s) {
    #pragma unroll
    for (int q = 0; q < PP; ++q) {
        const float2 v = p[q];
        c[q] = v.x;
        s[q] = v.y;
    }
}

// Candidates of a level over n_ctx tokens (pw = b^l), below a level that kept
// `kept_above` nodes (ignored at the top).
__device__ __forceinline__ sel::Cands level_cands(int64_t n_ctx, int64_t pw, int32_t b, bool top,
                                                  int32_t kept_above) {
    sel::Cands c;
    const int64_t Nl = n_ctx / pw;
    c.b = b;
    c.bmul = sel::fanout_magic((uint32_t)b);
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

template <int NW>
size_t rows_smem(int32_t maxc, int32_t k, int32_t nlev, int D) {
    const size_t mz = ((size_t)maxc + 3) & ~(size_t)3;
    return sizeof(float) * (mz + (size_t)NW * D + 4 * kNSlot + 4) + sel::kScratchBytes +
           sizeof(int32_t) * (size_t)(nlev + 2) * k + (size_t)(nlev + 1) * maxc;
}

template <typename T, int D>
__global__ __launch_bounds__(kNW * 64) void bwd_rows(TreeView tv, BwdArgs a, DebugView dbg) {
    constexpr int H2 = D / 2, PP = D / 32;
    extern __shared__ __align__(16) unsigned char smem[];
    const int32_t maxc = a.max_cand, b = a.b, K = a.k;
    const int nlev = tv.n_levels;
    const int32_t mz = (maxc + 3) & ~3;
    float *z = reinterpret_cast<float *>(smem);                          // [mz] logits of a level
    float *red = z + mz;                                                 // [NW][D] dq partials
    float *stat = red + kNW * D;                                         // [NSLOT][4] (M, L, S)
    float *misc = stat + 4 * kNSlot;                                     // [4]
    unsigned char *scratch = reinterpret_cast<unsigned char *>(misc + 4);
    int32_t *kept = reinterpret_cast<int32_t *>(scratch + sel::kScratchBytes);  // [nlev+2][K] by level
    uint8_t *flags = reinterpret_cast<uint8_t *>(kept + (nlev + 2) * K);         // [nlev+1][maxc]

    const int64_t row = blockIdx.x;
    const int64_t qi = row / a.Hq;
    const int h = (int)(row - qi * a.Hq);
    const int g = h / a.G;
    const int64_t n_ctx = a.ctx_base + qi * a.ctx_step;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int grp = lane >> 4, sub = lane & 15;
    const int slot = wave * 4 + grp;
    const int j0 = sub * PP;
    const float2 *rope = tv.rope;

    float qa[PP], qb[PP], da[PP], db[PP];
    {
        const T *qp = static_cast<const T *>(a.q) + row * D;
        Vec<T, PP>::load(qp + j0, qa);
        Vec<T, PP>::load(qp + H2 + j0, qb);
        const float *dp = a.dout + row * D;
        Vec<float, PP>::load(dp + j0, da);
        Vec<float, PP>::load(dp + H2 + j0, db);
    }
    // level l's key / value rows of KV head g (level 0: the caches) and their gradients
    auto key_row = [&](int l, int64_t node) -> const T * {
        if (l == 0) return static_cast<const T *>(tv.k_cache) + ((int64_t)g * tv.cap + node) * D;
        return static_cast<const T *>(tv.key[l]) + ((int64_t)g * tv.node_cap[l] + node) * D;
    };
    auto val_row = [&](int l, int64_t node) -> const T * {
        if (l == 0) return static_cast<const T *>(tv.v_cache) + ((int64_t)g * tv.cap + node) * D;
        return static_cast<const T *>(tv.val[l]) + ((int64_t)g * tv.node_cap[l] + node) * D;
    };
    auto gk_row = [&](int l, int64_t node) -> float * {
        if (l == 0) return a.dk + ((int64_t)g * tv.cap + node) * D;
        return a.gk[l] + ((int64_t)g * tv.node_cap[l] + node) * D;
    };
    auto gv_row = [&](int l, int64_t node) -> float * {
        if (l == 0) return a.dv + ((int64_t)g * tv.cap + node) * D;
        return a.gv[l] + ((int64_t)g * tv.node_cap[l] + node) * D;
    };
    // <R(n theta) q, R(i theta) key> over the slot (all 16 lanes get it)
    auto score = [&](const float *qna, const float *qnb, const T *kp, int32_t i) {
        float ka[PP], kb[PP], c[PP], s[PP];
        Vec<T, PP>::load(kp + j0, ka);
        Vec<T, PP>::load(kp + H2 + j0, kb);
        load_cs<PP>(rope + (int64_t)i * H2 + j0, c, s);
        float dot = 0.f;
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            const float ra = ka[p] * c[p] - kb[p] * s[p];
            const float rb = kb[p] * c[p] + ka[p] * s[p];
            dot += qna[p] * ra + qnb[p] * rb;
        }
        return a.scale * slot_sum(dot);
    };
    auto rotate_q = [&](int32_t n, float *qna, float *qnb) {
        float c[PP], s[PP];
        load_cs<PP>(rope + (int64_t)n * H2 + j0, c, s);
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            qna[p] = qa[p] * c[p] - qb[p] * s[p];
            qnb[p] = qb[p] * c[p] + qa[p] * s[p];
        }
    };

    int H = 0;
    int64_t pwH = 1;
    while (n_ctx / (pwH * b) >= 1) { pwH *= b; ++H; }
    if (threadIdx.x == 0) {
        for (int l = H + 1; l <= nlev; ++l) {
            if (dbg.selected != nullptr)
                for (int t = 0; t < K; ++t) dbg.selected[(row * nlev + l - 1) * K + t] = -1;
            if (dbg.kth_gap != nullptr) dbg.kth_gap[row * nlev + l - 1] = NAN;
        }
    }

    // ---- pass 1: the descent, with an online softmax carrying M, L = sum e^(z-M) and
    // S = sum e^(z-M) <dO, v> per slot -------------------------------------------------
    constexpr float kLog2e = 1.4426950408889634f;
    float M = -INFINITY, Ls = 0.f, Ss = 0.f;
    {
        int32_t m_above = 0;
        int64_t pw = pwH;
        for (int l = H; l >= 0; --l, pw /= b) {
            const sel::Cands cd = level_cands(n_ctx, pw, b, l == H, m_above);
            const int32_t *parents = kept + (l + 1) * K;
            uint8_t *fl = flags + (size_t)l * maxc;
            float qna[PP], qnb[PP];
            rotate_q(cd.n, qna, qnb);
            for (int32_t i = slot; i < cd.n; i += kNSlot) {
                const float zi = score(qna, qnb, key_row(l, sel::node_id(i, cd, parents)), i);
                if (sub == 15) {
                    z[i] = zi;
                    fl[i] = 0;
                }
            }
            __syncthreads();
            int32_t m = 0;
            if (l >= 1) {
                m = K < cd.n ? K : cd.n;
                if (wave == 0) {
                    sel::select<0>(z, fl, kept + l * K, m, cd, parents, lane, scratch, misc);
                    if (lane == 0 && dbg.kth_gap != nullptr) dbg.kth_gap[row * nlev + l - 1] = misc[1] - misc[2];
                    if (dbg.selected != nullptr) {
                        int32_t *ds = dbg.selected + (row * nlev + l - 1) * K;
                        for (int q = lane; q < K; q += 64) ds[q] = q < m ? kept[l * K + q] : -1;
                    }
                }
                __syncthreads();
            }
            for (int32_t i = slot; i < cd.n; i += kNSlot) {
                if (l >= 1 && fl[i]) continue;
                const T *vp = val_row(l, sel::node_id(i, cd, parents));
                float va[PP], vb[PP];
                Vec<T, PP>::load(vp + j0, va);
                Vec<T, PP>::load(vp + H2 + j0, vb);
                float t = 0.f;
                #pragma unroll
                for (int p = 0; p < PP; ++p) t += da[p] * va[p] + db[p] * vb[p];
                const float dp = slot_sum(t);
                const float zi = z[i];
                const float Mn = fmaxf(M, zi);
                const float sc = __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
                const float e = __builtin_amdgcn_exp2f((zi - Mn) * kLog2e);
                Ls = Ls * sc + e;
                Ss = Ss * sc + e * dp;
                M = Mn;
            }
            m_above = m;
            __syncthreads();        // z is rewritten by the next level
        }
    }
    if (sub == 0) {
        stat[4 * slot] = M;
        stat[4 * slot + 1] = Ls;
        stat[4 * slot + 2] = Ss;
    }
    __syncthreads();
    float Mg = -INFINITY;
    for (int s = 0; s < kNSlot; ++s) Mg = fmaxf(Mg, stat[4 * s]);
    float Lg = 0.f, Sg = 0.f;
    for (int s = 0; s < kNSlot; ++s) {
        const float sc = stat[4 * s] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((stat[4 * s] - Mg) * kLog2e);
        Lg += stat[4 * s + 1] * sc;
        Sg += stat[4 * s + 2] * sc;
    }
    const float Dv = Sg / Lg;
    const float invL = 1.f / Lg;

    // ---- pass 2: every entry again; dq in registers, dkey and dv to memory ------------
    // (phase 1 leaves out the token entries' dkey and dv, phase 2 does only those)
    float dqa[PP], dqb[PP];
    #pragma unroll
    for (int p = 0; p < PP; ++p) { dqa[p] = 0.f; dqb[p] = 0.f; }
    {
        int32_t m_above = 0;
        int64_t pw = pwH;
        for (int l = H; l >= 0; --l, pw /= b) {
            const sel::Cands cd = level_cands(n_ctx, pw, b, l == H, m_above);
            const int32_t *parents = kept + (l + 1) * K;
            const uint8_t *fl = flags + (size_t)l * maxc;
            if (a.phase == 2 && l >= 1) {
                m_above = K < cd.n ? K : cd.n;
                continue;
            }
            const bool grads = l >= 1 ? true : a.dk != nullptr && a.phase != 1;   // token gradients may be skipped
            float qna[PP], qnb[PP];
            rotate_q(cd.n, qna, qnb);
            for (int32_t i = slot; i < cd.n; i += kNSlot) {
                if (l >= 1 && fl[i]) continue;
                const int32_t node = sel::node_id(i, cd, parents);
                const T *kp = key_row(l, node);
                const T *vp = val_row(l, node);
                const float zi = score(qna, qnb, kp, i);
                float ka[PP], kb[PP], va[PP], vb[PP], c[PP], s[PP];
                Vec<T, PP>::load(kp + j0, ka);
                Vec<T, PP>::load(kp + H2 + j0, kb);
                Vec<T, PP>::load(vp + j0, va);
                Vec<T, PP>::load(vp + H2 + j0, vb);
                load_cs<PP>(rope + (int64_t)(cd.n - i) * H2 + j0, c, s);   // R((n - i) theta)
                float t = 0.f;
                #pragma unroll
                for (int p = 0; p < PP; ++p) t += da[p] * va[p] + db[p] * vb[p];
                const float dp = slot_sum(t);
                const float pe = __builtin_amdgcn_exp2f((zi - Mg) * kLog2e) * invL;
                const float dz = pe * (dp - Dv) * a.scale;
                #pragma unroll
                for (int p = 0; p < PP; ++p) {
                    // dq += s dz R_(i-n) key
                    dqa[p] += dz * (ka[p] * c[p] + kb[p] * s[p]);
                    dqb[p] += dz * (kb[p] * c[p] - ka[p] * s[p]);
                }
                if (grads) {
                    float *gk = gk_row(l, node);
                    float *gv = gv_row(l, node);
                    #pragma unroll
                    for (int p = 0; p < PP; ++p) {
                        // dkey = s dz R_(n-i) q;  dv = p dO
                        atomicAdd(gk + j0 + p, dz * (qa[p] * c[p] - qb[p] * s[p]));
                        atomicAdd(gk + H2 + j0 + p, dz * (qb[p] * c[p] + qa[p] * s[p]));
                        atomicAdd(gv + j0 + p, pe * da[p]);
                        atomicAdd(gv + H2 + j0 + p, pe * db[p]);
                    }
                }
            }
            m_above = l >= 1 ? (K < cd.n ? K : cd.n) : 0;
        }
    }
    if (a.phase == 2) return;           // dq was written by phase 1
    // dq: add the four slots of each wave, then the waves
    #pragma unroll
    for (int off = 16; off <= 32; off <<= 1)
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            dqa[p] += __shfl_xor(dqa[p], off);
            dqb[p] += __shfl_xor(dqb[p], off);
        }
    if (grp == 0) {
        #pragma unroll
        for (int p = 0; p < PP; ++p) {
            red[wave * D + j0 + p] = dqa[p];
            red[wave * D + H2 + j0 + p] = dqb[p];
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < D; e += kNW * 64) {
        float v = 0.f;
        for (int w = 0; w < kNW; ++w) v += red[w * D + e];
        a.dq[row * D + e] = v;
    }
}

// LDS of the per-wave pooler statistics (4 waves x [2][b] floats), 16-byte aligned.
__host__ __device__ constexpr size_t tree_stats_bytes(int32_t b) {
    return ((size_t)4 * 2 * b * sizeof(float) + 15) / 16 * 16;
}

// Per node of level l, one wave: the node's key and value gradients to its b
// children (level l - 1, or the tokens) and to dw.  A 16-lane group takes
// children grp, grp + 4, ...; each lane holds D/16 contiguous elements of a row.
// Children go four per group at a time, their loads issued together.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_tree(TreeView tv, BwdTreeArgs t) {
    constexpr int NE = D / 16;              // contiguous elements per lane
    constexpr int CB = 4;                   // children per group in flight
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int grp = lane >> 4, sub = lane & 15;
    const int e0 = sub * NE;
    const int32_t b = t.b;
    float *sa = reinterpret_cast<float *>(smem) + (size_t)wave * 2 * b;    // [b] pooler logits, then alpha
    float *sd = sa + b;                                                   // [b] <g, x_c>, then da_c
    // cache_keys: the children's key rows ([b][D] per wave), stored by the first pass
    // and read by the second instead of a second read from memory
    T *kc = reinterpret_cast<T *>(smem + tree_stats_bytes(b)) + (size_t)wave * b * D;
    const bool cache = t.cache_keys != 0;
    const int l = t.level;
    // write_children: the children's gradients are written (this is the first contribution)
    const bool wr = t.write_children != 0 && (l >= 2 || t.dk != nullptr);
    // persistent waves: the S waves of head g take its nodes s, s + S, s + 2S, ..., so the
    // nodes read at one time lie close together (a window of S nodes per head), and dw
    // stays in registers for the head (one set of atomics per head and wave, not per
    // node, which would serialize on dw's few addresses)
    // (node counts and wave counts stay below 2^31)
    const int32_t nwaves = (int32_t)gridDim.x * 4;
    const int32_t wid = (int32_t)blockIdx.x * 4 + wave;
    const int32_t hstep = nwaves < t.Hkv ? nwaves : t.Hkv;          // heads g0, g0 + hstep, ...
    const int32_t S = nwaves < t.Hkv ? 1 : nwaves / t.Hkv;           // waves per head
    if (wid >= S * hstep) return;
    const int g0 = wid % hstep;
    const int32_t s0 = wid / hstep;
    const int32_t nodes = (int32_t)t.nodes;
    float dw[NE];
    #pragma unroll
    for (int e = 0; e < NE; ++e) dw[e] = 0.f;
    auto flush = [&](int gg) {
        float v[NE];
        #pragma unroll
        for (int e = 0; e < NE; ++e) {
            v[e] = dw[e];
            v[e] += __shfl_xor(v[e], 16);
            v[e] += __shfl_xor(v[e], 32);
            dw[e] = 0.f;
        }
        bool nz = false;
        #pragma unroll
        for (int e = 0; e < NE; ++e) nz = nz || v[e] != 0.f;
        if (grp == 0 && nz) {
            #pragma unroll
            for (int e = 0; e < NE; ++e) atomicAdd(t.dw + (int64_t)gg * D + e0 + e, v[e]);
        }
    };
    for (int g = g0; g < t.Hkv; g += hstep) {
    for (int32_t j = s0; j < nodes; j += S) {
    const float *gkp = t.gk + ((int64_t)g * tv.node_cap[l] + j) * D + e0;
    const float *gvp = t.gv + ((int64_t)g * tv.node_cap[l] + j) * D + e0;
    float gk[NE], gv[NE], w[NE];
    Vec<float, NE>::load(gkp, gk);
    Vec<float, NE>::load(gvp, gv);
    Vec<float, NE>::load(t.pool_w + (int64_t)g * D + e0, w);
    bool any = false;
    #pragma unroll
    for (int u = 0; u < NE; ++u) any = any || gk[u] != 0.f || gv[u] != 0.f;
    const int64_t c0 = j * b;
    // the children: stored keys of level l - 1 (tokens at l = 1) and their gradients
    float *ck = l == 1 ? t.dk + ((int64_t)g * tv.cap + c0) * D
                       : t.gk_child + ((int64_t)g * tv.node_cap[l - 1] + c0) * D;
    float *cv = l == 1 ? t.dv + ((int64_t)g * tv.cap + c0) * D
                       : t.gv_child + ((int64_t)g * tv.node_cap[l - 1] + c0) * D;
    if (__ballot(any) == 0) {               // no row read this node
        if (wr) {                           // its children's gradients are still written: zero
            float z[NE];
            #pragma unroll
            for (int e = 0; e < NE; ++e) z[e] = 0.f;
            for (int32_t c = grp; c < b; c += 4) {
                Vec<float, NE>::store(ck + (int64_t)c * D + e0, z);
                Vec<float, NE>::store(cv + (int64_t)c * D + e0, z);
            }
        }
        continue;
    }
    const T *xk = l == 1 ? static_cast<const T *>(tv.k_cache) + ((int64_t)g * tv.cap + c0) * D
                         : static_cast<const T *>(tv.key[l - 1]) + ((int64_t)g * tv.node_cap[l - 1] + c0) * D;
    // child of this group's batch slot u (clamped to the last child; the result is then unused)
    auto child = [&](int32_t cb, int u) {
        const int32_t c = cb + grp + 4 * u;
        return c < b ? c : b - 1;
    };
    for (int32_t cb = 0; cb < b; cb += 4 * CB) {
        float x[CB][NE];
        #pragma unroll
        for (int u = 0; u < CB; ++u) Vec<T, NE>::load(xk + (int64_t)child(cb, u) * D + e0, x[u]);
        if (cache) {
            #pragma unroll
            for (int u = 0; u < CB; ++u) Vec<T, NE>::store(kc + (int64_t)child(cb, u) * D + e0, x[u]);
        }
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            float pa = 0.f, pd = 0.f;
            #pragma unroll
            for (int e = 0; e < NE; ++e) {
                pa += w[e] * x[u][e];
                pd += gk[e] * x[u][e];
            }
            pa = row_sum16(pa);
            pd = row_sum16(pd);
            const int32_t c = cb + grp + 4 * u;
            if (sub == 15 && c < b) {
                sa[c] = t.pool_scale * pa;
                sd[c] = pd;
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float mx = -INFINITY;
    for (int32_t c = lane; c < b; c += 64) mx = fmaxf(mx, sa[c]);
    #pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float se = 0.f, sad = 0.f;
    for (int32_t c = lane; c < b; c += 64) {
        const float e = __expf(sa[c] - mx);
        se += e;
        sad += e * sd[c];
    }
    #pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        se += __shfl_xor(se, off);
        sad += __shfl_xor(sad, off);
    }
    const float avg = sad / se;             // sum_c alpha_c <g, x_c>
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int32_t c = lane; c < b; c += 64) {
        const float al = __expf(sa[c] - mx) / se;
        sd[c] = al * (sd[c] - avg);         // da_c
        sa[c] = al;                         // alpha_c
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float invb = 1.f / (float)b;
    const bool child_grads = l >= 2 || t.dk != nullptr;     // token gradients may be skipped
    for (int32_t cb = 0; cb < b; cb += 4 * CB) {
        float x[CB][NE], ok[CB][NE], ov[CB][NE];
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int64_t c = child(cb, u);
            if (cache) Vec<T, NE>::load(kc + c * D + e0, x[u]);
            else Vec<T, NE>::load(xk + c * D + e0, x[u]);
            if (child_grads && !wr) {
                Vec<float, NE>::load(ck + c * D + e0, ok[u]);
                Vec<float, NE>::load(cv + c * D + e0, ov[u]);
            } else {
                #pragma unroll
                for (int e = 0; e < NE; ++e) { ok[u][e] = 0.f; ov[u][e] = 0.f; }
            }
        }
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int32_t c = cb + grp + 4 * u;
            if (c >= b) continue;
            const float al = sa[c], dac = t.pool_scale * sd[c];
            #pragma unroll
            for (int e = 0; e < NE; ++e) dw[e] += dac * x[u][e];
            if (child_grads) {
                #pragma unroll
                for (int e = 0; e < NE; ++e) {
                    ok[u][e] += al * gk[e] + dac * w[e];
                    ov[u][e] += gv[e] * invb;
                }
                Vec<float, NE>::store(ck + (int64_t)c * D + e0, ok[u]);
                Vec<float, NE>::store(cv + (int64_t)c * D + e0, ov[u]);
            }
        }
    }
    // the next node reuses sa / sd
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    flush(g);
    }
}

// Level 1 in one pass over a node's children with an online softmax: dw only (the
// distillation step), or dw and the tokens' dk, dv written (WR; fanout <= 32).  With
// e_c = exp(a_c - m), q_c = <g, x_c> and r a reference (child 0's q),
//   l = sum e_c,  A = sum e_c x_c,  S = sum e_c (q_c - r),  B = sum e_c (q_c - r) x_c,
// the node adds s_p (B / l - (S / l)(A / l)) = s_p sum_c da_c x_c to dw (the shift by r
// cancels; it keeps the subtraction well conditioned when the q_c share a large part).
// A child's gradients need only its a_c and q_c: alpha_c = e_c / l,
// da_c = alpha_c (q_c - r - S / l), dk_c = alpha_c g + s_p da_c w, dv_c = g_v / b, so
// WR keeps them in registers and writes each token row once, reading no key twice.
// Each lane group takes children grp, grp + 4, ..., all of its (up to 8) rows in
// flight at once, so a node waits on memory once.  Persistent waves keep dw per head:
// the S waves of head g take its nodes s, s + S, s + 2S, ..., so the nodes read at one
// time lie close together (a window of S nodes per head) and each wave adds to dw once.
// BF (with WR): the token rows are bf16; each adds the staged sums of the rows' own
// entries (the node's level-0 items) to its tree part before the one rounding.
template <typename T, int D, bool WR, bool BF>
__global__ __launch_bounds__(256) void bwd_tree_one(TreeView tv, BwdTreeArgs t) {
    constexpr int NE = D / 16;              // contiguous elements per lane
    constexpr int RIF = 8;                  // rows of a lane group in flight
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int grp = lane >> 4, sub = lane & 15;
    const int e0 = sub * NE;
    const int32_t b = t.b;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int64_t wid = (int64_t)blockIdx.x * 4 + wave;
    const int64_t hstep = nwaves < t.Hkv ? nwaves : t.Hkv;          // heads g0, g0 + hstep, ...
    const int64_t S = nwaves < t.Hkv ? 1 : nwaves / t.Hkv;           // waves per head
    if (wid >= S * hstep) return;
    const int g0 = (int)(wid % hstep);
    const int64_t s0 = wid / hstep;
    float dw[NE], w[NE];
    #pragma unroll
    for (int e = 0; e < NE; ++e) dw[e] = 0.f;
    auto flush = [&](int gg) {
        float v[NE];
        #pragma unroll
        for (int e = 0; e < NE; ++e) {
            v[e] = dw[e];
            v[e] += __shfl_xor(v[e], 16);
            v[e] += __shfl_xor(v[e], 32);
            dw[e] = 0.f;
        }
        if (grp == 0) {
            #pragma unroll
            for (int e = 0; e < NE; ++e) atomicAdd(t.dw + (int64_t)gg * D + e0 + e, v[e]);
        }
    };
    // sum over the 16 lanes of a group, in every lane of it
    auto gsum = [](float v) {
        v += __shfl_xor(v, 8, 16);
        v += __shfl_xor(v, 4, 16);
        v += __shfl_xor(v, 2, 16);
        v += __shfl_xor(v, 1, 16);
        return v;
    };
    for (int g = g0; g < t.Hkv; g += (int)hstep) {
    Vec<float, NE>::load(t.pool_w + (int64_t)g * D + e0, w);
    for (int64_t j = s0; j < t.nodes; j += S) {
        float gk[NE], gv[NE];
        Vec<float, NE>::load(t.gk + ((int64_t)g * tv.node_cap[1] + j) * D + e0, gk);
        if (WR) Vec<float, NE>::load(t.gv + ((int64_t)g * tv.node_cap[1] + j) * D + e0, gv);
        int32_t st0 = 0, st1 = 0;           // BF: the node's staged items
        if (BF) {
            const int32_t *so = t.stage_item + (int64_t)g * t.stage_np + j;
            st0 = __builtin_amdgcn_readfirstlane(so[0]);
            st1 = __builtin_amdgcn_readfirstlane(so[1]);
        }
        const T *xk = static_cast<const T *>(tv.k_cache) + ((int64_t)g * tv.cap + j * b) * D + e0;
        float m = -INFINITY, l = 0.f, Sq = 0.f, r = 0.f, A[NE], B[NE];
        float za[RIF], zq[RIF];             // WR: this group's children's a_c and q_c (one batch)
        #pragma unroll
        for (int e = 0; e < NE; ++e) { A[e] = 0.f; B[e] = 0.f; }
        for (int32_t c0 = grp; c0 < b; c0 += 4 * RIF) {
            float x[RIF][NE];
            #pragma unroll
            for (int u = 0; u < RIF; ++u) {
                const int32_t c = c0 + 4 * u;
                Vec<T, NE>::load(xk + (int64_t)(c < b ? c : b - 1) * D, x[u]);
            }
            #pragma unroll
            for (int u = 0; u < RIF; ++u) {
                const int32_t c = c0 + 4 * u;
                float pa = 0.f, pq = 0.f;
                #pragma unroll
                for (int e = 0; e < NE; ++e) {
                    pa += w[e] * x[u][e];
                    pq += gk[e] * x[u][e];
                }
                pa = t.pool_scale * gsum(pa);
                pq = gsum(pq);
                if (c0 == grp && u == 0) r = __shfl(pq, 0);   // child 0's q, uniform
                if (WR) {
                    za[u] = pa;
                    zq[u] = pq;
                }
                if (c < b) {                                   // uniform within a lane group
                    const float mn = fmaxf(m, pa);
                    const float cs = __expf(m - mn);          // m = -inf on the first row: 0
                    const float p = __expf(pa - mn);
                    const float pd = p * (pq - r);
                    l = l * cs + p;
                    Sq = Sq * cs + pd;
                    #pragma unroll
                    for (int e = 0; e < NE; ++e) {
                        A[e] = A[e] * cs + p * x[u][e];
                        B[e] = B[e] * cs + pd * x[u][e];
                    }
                    m = mn;
                }
            }
        }
        // merge the four lane groups (all hold a row: b >= 4 is not assumed, so guard -inf)
        #pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off), so = __shfl_xor(Sq, off);
            const float mn = fmaxf(m, mo);
            const float ca = m == -INFINITY ? 0.f : __expf(m - mn);
            const float cb = mo == -INFINITY ? 0.f : __expf(mo - mn);
            l = l * ca + lo * cb;
            Sq = Sq * ca + so * cb;
            #pragma unroll
            for (int e = 0; e < NE; ++e) {
                const float ao = __shfl_xor(A[e], off), bo = __shfl_xor(B[e], off);
                A[e] = A[e] * ca + ao * cb;
                B[e] = B[e] * ca + bo * cb;
            }
            m = mn;
        }
        const float il = 1.f / l, sbar = Sq * il;
        if (grp == 0) {                     // every group holds the merged state; count it once
            #pragma unroll
            for (int e = 0; e < NE; ++e) dw[e] += t.pool_scale * (B[e] * il - sbar * A[e] * il);
        }
        if (WR) {                           // the group's children: one batch (b <= 4 * RIF)
            const int64_t row0 = ((int64_t)g * tv.cap + j * b) * D + e0;
            float ov[NE];
            #pragma unroll
            for (int e = 0; e < NE; ++e) ov[e] = gv[e] * (1.f / (float)b);
            #pragma unroll
            for (int u = 0; u < RIF; ++u) {
                const int32_t c = grp + 4 * u;
                if (c < b) {
                    const float al = __expf(za[u] - m) * il;
                    const float dac = t.pool_scale * al * (zq[u] - r - sbar);
                    float ok[NE];
                    #pragma unroll
                    for (int e = 0; e < NE; ++e) ok[e] = al * gk[e] + dac * w[e];
                    if (BF) {
                        float vv[NE];
                        #pragma unroll
                        for (int e = 0; e < NE; ++e) vv[e] = ov[e];
                        for (int32_t it = st0; it < st1; ++it) {
                            float sk[NE], sv[NE];
                            Vec<float, NE>::load(t.stage_k + ((int64_t)it * b + c) * D + e0, sk);
                            Vec<float, NE>::load(t.stage_v + ((int64_t)it * b + c) * D + e0, sv);
                            #pragma unroll
                            for (int e = 0; e < NE; ++e) {
                                ok[e] += sk[e];
                                vv[e] += sv[e];
                            }
                        }
                        Vec<bf16_t, NE>::store(t.dk16 + row0 + (int64_t)c * D, ok);
                        Vec<bf16_t, NE>::store(t.dv16 + row0 + (int64_t)c * D, vv);
                    } else {
                        Vec<float, NE>::store(t.dk + row0 + (int64_t)c * D, ok);
                        Vec<float, NE>::store(t.dv + row0 + (int64_t)c * D, ov);
                    }
                }
            }
        }
    }
    flush(g);
    }
}

template <typename T, int D, bool WR, bool BF>
hipError_t launch_tree_one_t(const TreeView &tv, const BwdTreeArgs &t, hipStream_t s) {
    const int64_t nodes = (int64_t)t.Hkv * t.nodes;
    if (nodes == 0) return hipSuccess;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)bwd_tree_one<T, D, WR, BF>, 256, 0);
    if (e != hipSuccess) return e;
    const int64_t want = (nodes + 3) / 4;
    const int64_t cap = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    const int64_t blocks = want < cap ? want : cap;
    hipLaunchKernelGGL((bwd_tree_one<T, D, WR, BF>), dim3((unsigned)blocks), dim3(256), 0, s, tv, t);
    return hipGetLastError();
}

__global__ void fill_zero(uint4 *p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// rows [r0, r1) of each head of a [H][cap][D] fp32 array, in float4s
__global__ void zero_rows(float4 *p, int32_t H, int64_t cap4, int64_t r0_4, int64_t n4) {
    const int64_t total = (int64_t)H * n4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t h = i / n4;
        p[h * cap4 + r0_4 + (i - h * n4)] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <typename T, int D>
hipError_t launch_rows_t(const TreeView &tv, const BwdArgs &a, const DebugView &dbg, hipStream_t s) {
    const size_t smem = rows_smem<kNW>(a.max_cand, a.k, tv.n_levels, D);
    if (smem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)bwd_rows<T, D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_rows<T, D>), dim3((unsigned)a.rows), dim3(kNW * 64), smem, s, tv, a, dbg);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_tree_t(const TreeView &tv, const BwdTreeArgs &targ, hipStream_t s) {
    const int64_t nodes = (int64_t)targ.Hkv * targ.nodes;
    if (nodes == 0) return hipSuccess;
    // the key cache while it leaves room for two workgroups per CU
    BwdTreeArgs t = targ;
    const size_t cache_bytes = (size_t)4 * t.b * D * sizeof(T);
    t.cache_keys = tree_stats_bytes(t.b) + cache_bytes <= 64 * 1024 ? 1 : 0;
    const size_t smem = tree_stats_bytes(t.b) + (t.cache_keys ? cache_bytes : 0);
    // as many workgroups as are resident at once; each wave then walks its share of nodes
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)bwd_tree<T, D>, 256, smem);
    if (e != hipSuccess) return e;
    const int64_t want = (nodes + 3) / 4;
    const int64_t cap = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    const int64_t blocks = want < cap ? want : cap;
    hipLaunchKernelGGL((bwd_tree<T, D>), dim3((unsigned)blocks), dim3(256), smem, s, tv, t);
    return hipGetLastError();
}

}  // namespace

size_t backward_rows_lds_bytes(int32_t maxc, int32_t k, int32_t nlev, int32_t D) {
    return rows_smem<kNW>(maxc, k, nlev, D);
}

hipError_t launch_zero_rows(float *p, int32_t Hkv, int64_t cap, int64_t r0, int64_t r1, int32_t D, hipStream_t s) {
    if (p == nullptr || r1 <= r0 || Hkv < 1) return hipSuccess;
    const int64_t n4 = (r1 - r0) * D / 4;
    const int64_t total = (int64_t)Hkv * n4;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(zero_rows, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s,
                       reinterpret_cast<float4 *>(p), Hkv, cap * D / 4, r0 * D / 4, n4);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    const int64_t blocks = (n16 + 255) / 256;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                       static_cast<uint4 *>(p), n16);
    return hipGetLastError();
}

hipError_t launch_backward_rows(const TreeView &tv, recsa_dtype st, int32_t D, const BwdArgs &a,
                                const DebugView &dbg, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (st == RECSA_BF16) return D == 128 ? launch_rows_t<bf16_t, 128>(tv, a, dbg, s) : launch_rows_t<bf16_t, 64>(tv, a, dbg, s);
    return D == 128 ? launch_rows_t<float, 128>(tv, a, dbg, s) : launch_rows_t<float, 64>(tv, a, dbg, s);
}

hipError_t launch_backward_tree(const TreeView &tv, recsa_dtype st, int32_t D, const BwdTreeArgs &t,
                                hipStream_t s) {
    // level 1 in one pass: bf16 token gradients with their staged entries (bf16 storage,
    // fanout <= 32), dw only, or the tokens' gradients written (fanout <= 32)
    if (t.level == 1 && t.dk16 != nullptr) {
        if (st != RECSA_BF16 || t.b > 32 || t.write_children == 0 || t.stage_k == nullptr) return hipErrorInvalidValue;
        return D == 128 ? launch_tree_one_t<bf16_t, 128, true, true>(tv, t, s)
                        : launch_tree_one_t<bf16_t, 64, true, true>(tv, t, s);
    }
    if (t.level == 1 && t.dk == nullptr) {
        if (st == RECSA_BF16)
            return D == 128 ? launch_tree_one_t<bf16_t, 128, false, false>(tv, t, s) : launch_tree_one_t<bf16_t, 64, false, false>(tv, t, s);
        return D == 128 ? launch_tree_one_t<float, 128, false, false>(tv, t, s) : launch_tree_one_t<float, 64, false, false>(tv, t, s);
    }
    if (t.level == 1 && t.write_children != 0 && t.dk != nullptr && t.b <= 32) {
        if (st == RECSA_BF16)
            return D == 128 ? launch_tree_one_t<bf16_t, 128, true, false>(tv, t, s) : launch_tree_one_t<bf16_t, 64, true, false>(tv, t, s);
        return D == 128 ? launch_tree_one_t<float, 128, true, false>(tv, t, s) : launch_tree_one_t<float, 64, true, false>(tv, t, s);
    }
    if (st == RECSA_BF16) return D == 128 ? launch_tree_t<bf16_t, 128>(tv, t, s) : launch_tree_t<bf16_t, 64>(tv, t, s);
    return D == 128 ? launch_tree_t<float, 128>(tv, t, s) : launch_tree_t<float, 64>(tv, t, s);
}

}  // namespace recsa
