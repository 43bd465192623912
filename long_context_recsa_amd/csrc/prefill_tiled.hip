// Causal prefill, parent-major, on gfx950 (bf16 storage).
//
// RecSA, abstract: each level above the tokens keeps at most k candidates;
// the summaries of the candidates not kept share one softmax with the exact
// tokens; each entry's RoPE position is its index among its level's
// candidates (the query sits at the level's candidate count n).
//
// A row (one chunk query and one query head) reaches, at level l, the
// children of its parents: the m nodes it kept at level l+1 (ranks 0..m-1,
// ascending) and, when level l has orphans, the partial node N_{l+1} (rank m),
// whose o_l complete children come last.  Candidate i = r*b + c is child c of
// the rank-r parent, so with rotate-half RoPE
//     <rope(q, n), rope(key, i)> = <R((n - r*b) theta) q, R(c theta) key>.
// Rows of one chunk share most parents: at the top every row reads the same
// few nodes, and further down a parent is shared by rows that kept it.  So
// instead of walking each row on its own (which re-reads a parent's children
// once per row), every level is done parent-major:
//   count/scan/scatter  group the level's (row, rank) pairs by (KV head, parent);
//   score   per 16 pairs of one parent: the parent's children are loaded once,
//           rotated by their child offset, and scored against the pairs'
//           rank-rotated queries on bf16 MFMA (fp32 operands split into a bf16
//           high and low part; three products give about 16 correct bits);
//   select  per row: the top-min(k, n) logits become the next level's parents
//           (equal logits: lower index), the others are entries: the row's
//           running max and normaliser absorb them and their logits stay;
//   pv      per 16 pairs of one parent: exp(z - max) of the entries times the
//           children's values (bf16, exact) on MFMA, one partial sum per pair;
// and the partial sums of a level are folded into the row's accumulator when
// the next level is selected (or at the end).  At level 0 the children are
// tokens and every candidate is an entry.
#include <math.h>

#include <algorithm>

#include "recsa_internal.hpp"
#include "select_topk.hpp"

namespace recsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kTile = 16;             // pairs per MFMA tile (the M side)
constexpr int kHistMax = 8192;        // parents per KV head counted in LDS before one global add
constexpr int64_t kRowsPerPass = 1 << 18;

struct RowStat {
    float m_acc;     // the max the accumulator is expressed in
    float m_cur;     // the running max over all entries so far
    float l;         // the running normaliser, in units of m_cur
    int32_t n_keys;  // candidates scored so far
};

struct TP {
    const bf16_t *q;           // [rows][D]
    void *out;                 // [rows][D]
    int32_t out_bf16;
    int32_t Hq, G, Hkv, D;
    int64_t rows;
    int64_t ctx_base;          // n_ctx of row 0's query
    int32_t ctx_step;
    int32_t b, k, zs;          // zs: row stride of z (floats)
    float scale;
    int32_t top;               // highest level any row reaches
    int32_t n_levels;          // levels of the tree (debug layout)
    int64_t length;            // tokens in the tree
    int64_t pw[kMaxLevels + 2];  // b^l
    // workspace
    float *z;                  // [rows][zs]
    int32_t *par[2];           // [rows][k]: parents by level parity
    int32_t *mk[2];            // [rows]: kept parents by level parity
    int32_t *np;               // [rows]: pairs of the last selected level
    int32_t *pairpos;          // [rows][k+1]
    int32_t *counts;           // [nb]
    int32_t *offs;             // [nb+1]
    int32_t *itemoff;          // [nb+1]
    int2 *sorted;              // [pairs]: (row, rank) grouped by parent
    int4 *items;               // (bucket, first pair, pairs, 0)
    int32_t *n_items;
    float *partial;            // [rows][k+1][D]
    float *acc;                // [rows][D]
    RowStat *stat;             // [rows]
};

struct RowLevel {
    int32_t m;       // kept parents
    int32_t o;       // orphans (children of the partial parent)
    int64_t part;    // the partial parent's node id (N_{l+1})
};

__device__ __forceinline__ RowLevel row_level(const TP &a, int64_t row, int l) {
    const int64_t n = a.ctx_base + (row / a.Hq) * a.ctx_step;
    const int64_t up = n / a.pw[l + 1];
    RowLevel r;
    r.m = a.mk[l & 1][row];
    r.o = (int32_t)(n / a.pw[l] - (int64_t)a.b * up);
    r.part = up;
    return r;
}

__device__ __forceinline__ int64_t parent_of(const TP &a, int64_t row, int l, int rank,
                                             const RowLevel &rl) {
    return rank < rl.m ? (int64_t)a.par[l & 1][row * a.k + rank] : rl.part;
}

// keys or values of level l (tokens at l = 0) of KV head g
__device__ __forceinline__ const bf16_t *level_rows(const TreeView &tv, bool values, int l, int g,
                                                    int D) {
    if (l == 0)
        return static_cast<const bf16_t *>(values ? tv.v_cache : tv.k_cache) + (int64_t)g * tv.cap * D;
    return static_cast<const bf16_t *>(values ? tv.val[l] : tv.key[l]) +
           (int64_t)g * tv.node_cap[l] * D;
}

__device__ __forceinline__ float wave_max(float v) {
    #pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    #pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// x ~ hi + lo with both parts bf16 (about 16 significant bits)
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
    #pragma unroll
    for (int v = 0; v < 8; ++v) {
        const __bf16 h = (__bf16)x[v];
        hi[v] = h;
        lo[v] = (__bf16)(x[v] - (float)h);
    }
}

template <int PP>
__device__ __forceinline__ void load_cs(const float2 *p, float *c, float *s) {
    #pragma unroll
    for (int q = 0; q < PP; q += 2) {
        const float4 v = *reinterpret_cast<const float4 *>(p + q);
        c[q] = v.x; s[q] = v.y; c[q + 1] = v.z; s[q + 1] = v.w;
    }
}

// ---------------------------------------------------------------- set-up --
__global__ void tp_init(TP a, DebugView dbg, int64_t nb) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = t; i < a.rows; i += stride) {
        a.stat[i] = RowStat{-INFINITY, -INFINITY, 0.f, 0};
        a.np[i] = 0;
        a.mk[a.top & 1][i] = 0;
        if (dbg.n_keys) dbg.n_keys[i] = 0;
    }
    for (int64_t i = t; i < a.rows * a.D; i += stride) a.acc[i] = 0.f;
    for (int64_t i = t; i < nb; i += stride) a.counts[i] = 0;
    if (dbg.selected)
        for (int64_t i = t; i < a.rows * a.n_levels * a.k; i += stride) dbg.selected[i] = -1;
    if (dbg.kth_gap)
        for (int64_t i = t; i < a.rows * a.n_levels; i += stride) dbg.kth_gap[i] = NAN;
}

// Position of every pair of level l inside its (head, parent) bucket, and the
// bucket sizes.  One block holds rows of one KV head; with few parents it
// counts in LDS first, so a bucket takes one global atomic per block.
__global__ __launch_bounds__(256) void tp_count(TP a, int l, int32_t NP, int use_lds) {
    extern __shared__ int32_t hist[];
    const int g = blockIdx.y;
    const int64_t per_head = a.rows / a.Hq * a.G;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t row = -1;
    if (t < per_head) row = (t / a.G) * a.Hq + (int64_t)g * a.G + (t % a.G);
    if (use_lds) {
        for (int p = threadIdx.x; p < NP; p += blockDim.x) hist[p] = 0;
        __syncthreads();
    }
    RowLevel rl{0, 0, 0};
    int32_t np = 0;
    if (row >= 0) {
        rl = row_level(a, row, l);
        np = rl.m + (rl.o > 0 ? 1 : 0);
    }
    int32_t *pp = a.pairpos + (row >= 0 ? row : 0) * (a.k + 1);
    for (int r = 0; r < np; ++r) {
        const int64_t p = parent_of(a, row, l, r, rl);
        pp[r] = use_lds ? atomicAdd(&hist[p], 1) : atomicAdd(&a.counts[(int64_t)g * NP + p], 1);
    }
    if (use_lds) {
        __syncthreads();
        for (int p = threadIdx.x; p < NP; p += blockDim.x) {
            const int32_t c = hist[p];
            if (c) hist[p] = atomicAdd(&a.counts[(int64_t)g * NP + p], c);
        }
        __syncthreads();
        for (int r = 0; r < np; ++r) pp[r] += hist[parent_of(a, row, l, r, rl)];
    }
}

// Exclusive scans of the bucket sizes (pair offsets) and of their tiles
// (item offsets); clears the sizes for the next level.
__global__ __launch_bounds__(1024) void tp_scan(TP a, int64_t nb) {
    __shared__ int32_t s0[1024], s1[1024];
    const int t = threadIdx.x;
    const int64_t per = (nb + 1023) / 1024;
    const int64_t b0 = t * per, b1 = min(nb, b0 + per);
    int32_t c0 = 0, c1 = 0;
    for (int64_t i = b0; i < b1; ++i) {
        const int32_t c = a.counts[i];
        c0 += c;
        c1 += (c + kTile - 1) / kTile;
    }
    s0[t] = c0;
    s1[t] = c1;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t v0 = t >= off ? s0[t - off] : 0;
        const int32_t v1 = t >= off ? s1[t - off] : 0;
        __syncthreads();
        s0[t] += v0;
        s1[t] += v1;
        __syncthreads();
    }
    int32_t e0 = s0[t] - c0, e1 = s1[t] - c1;
    for (int64_t i = b0; i < b1; ++i) {
        const int32_t c = a.counts[i];
        a.offs[i] = e0;
        a.itemoff[i] = e1;
        e0 += c;
        e1 += (c + kTile - 1) / kTile;
        a.counts[i] = 0;
    }
    if (t == 1023) {
        a.offs[nb] = s0[1023];
        a.itemoff[nb] = s1[1023];
        *a.n_items = s1[1023];
    }
}

// Pairs into bucket order; one item per tile of a bucket.
__global__ __launch_bounds__(256) void tp_scatter(TP a, int l, int32_t NP, int64_t nb) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < a.rows) {
        const int64_t row = t;
        const RowLevel rl = row_level(a, row, l);
        const int32_t np = rl.m + (rl.o > 0 ? 1 : 0);
        const int64_t g = (row % a.Hq) / a.G;
        for (int r = 0; r < np; ++r) {
            const int64_t bkt = g * NP + parent_of(a, row, l, r, rl);
            a.sorted[a.offs[bkt] + a.pairpos[row * (a.k + 1) + r]] = make_int2((int32_t)row, r);
        }
    } else if (t - a.rows < nb) {
        const int64_t bkt = t - a.rows;
        const int32_t o0 = a.offs[bkt], c = a.offs[bkt + 1] - o0, i0 = a.itemoff[bkt];
        for (int32_t s = 0; s < c; s += kTile)
            a.items[i0 + s / kTile] = make_int4((int32_t)bkt, o0 + s, min(kTile, c - s), 0);
    }
}

// ----------------------------------------------------------------- score --
// One wave per item: up to 16 pairs of one parent against its b children.
// MFMA 16x16x32: lane L supplies A row L%16 and B column L%16 for the 8
// k-slots of group L/16.  The k-slots are mapped to dimensions so that a lane
// group owns RoPE pairs [grp*D/8, grp*D/8 + D/8) of both halves: every rotation
// stays inside a lane and each row slice is a contiguous load.
template <int D>
__global__ __launch_bounds__(256) void tp_score(TreeView tv, TP a, int l, int32_t NP) {
    constexpr int H = D / 2, PG = D / 8, KS = D / 32, KS1 = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= *a.n_items) return;
    const int4 it = a.items[item];
    const int g = it.x / NP;
    const int64_t p = it.x % NP;
    const int cnt = it.z;
    const int i16 = lane & 15, grp = lane >> 4;
    const int2 pr = a.sorted[it.y + (i16 < cnt ? i16 : 0)];
    const int64_t row = pr.x;
    const int rank = pr.y;
    const RowLevel rl = row_level(a, row, l);
    const int32_t n = rl.m * a.b + rl.o;
    const int32_t nc = rank < rl.m ? a.b : rl.o;
    const int32_t pos = n - rank * a.b;

    bf16x8 ah[KS], al[KS];
    {
        float q1[PG], q2[PG], c[PG], s[PG], u[D / 4];
        const bf16_t *qr = a.q + row * D;
        Vec<bf16_t, PG>::load(qr + grp * PG, q1);
        Vec<bf16_t, PG>::load(qr + H + grp * PG, q2);
        load_cs<PG>(tv.rope + (int64_t)pos * H + grp * PG, c, s);
        const float live = i16 < cnt ? 1.f : 0.f;
        #pragma unroll
        for (int j = 0; j < PG; ++j) {
            u[j] = live * (q1[j] * c[j] - q2[j] * s[j]);
            u[PG + j] = live * (q2[j] * c[j] + q1[j] * s[j]);
        }
        #pragma unroll
        for (int ks = 0; ks < KS; ++ks) split8(u + 8 * ks, ah[ks], al[ks]);
    }
    static_assert(KS1 * 8 == PG, "first-half slots");

    // the output rows of this lane: pairs 4*grp + v
    int32_t orow[4], orank[4], onc[4];
    #pragma unroll
    for (int v = 0; v < 4; ++v) {
        orow[v] = __shfl((int32_t)row, 4 * grp + v);
        orank[v] = __shfl(rank, 4 * grp + v);
        onc[v] = __shfl(nc, 4 * grp + v);
    }

    const bf16_t *keys = level_rows(tv, false, l, g, D);
    const int64_t nexist = a.length / a.pw[l];
    const int64_t c0 = p * a.b;
    for (int ct = 0; ct < a.b; ct += 16) {
        const int c = ct + i16;
        const bool ok = c < a.b && c0 + c < nexist;
        float k1[PG], k2[PG], cc[PG], ss[PG], kr[D / 4];
        if (ok) {
            const bf16_t *kp = keys + (c0 + c) * D;
            Vec<bf16_t, PG>::load(kp + grp * PG, k1);
            Vec<bf16_t, PG>::load(kp + H + grp * PG, k2);
            load_cs<PG>(tv.rope + (int64_t)c * H + grp * PG, cc, ss);
        } else {
            #pragma unroll
            for (int j = 0; j < PG; ++j) { k1[j] = 0.f; k2[j] = 0.f; cc[j] = 1.f; ss[j] = 0.f; }
        }
        #pragma unroll
        for (int j = 0; j < PG; ++j) {
            kr[j] = k1[j] * cc[j] - k2[j] * ss[j];
            kr[PG + j] = k2[j] * cc[j] + k1[j] * ss[j];
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 bh, bl;
            split8(kr + 8 * ks, bh, bl);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks], bh, acc, 0, 0, 0);
        }
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (4 * grp + v < cnt && c < onc[v])
                a.z[(int64_t)orow[v] * a.zs + orank[v] * a.b + c] = a.scale * acc[v];
        }
    }
}

// ---------------------------------------------------------------- select --
// One wave per row.  Folds the previous level's partial sums into the row's
// accumulator, keeps the top min(k, n) candidates of level l (l >= 1) as the
// next level's parents, and adds this level's entries to the running max and
// normaliser; kept candidates' logits become -inf so the P.V pass skips them.
template <int KT>
__global__ __launch_bounds__(256) void tp_select(TP a, DebugView dbg, int l, int smem_wave) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + w;
    if (row >= a.rows) return;
    unsigned char *base = smem + w * smem_wave;
    unsigned char *scratch = base;                                             // 16-aligned
    float *outv = reinterpret_cast<float *>(base + sel::kScratchBytes);        // [4]
    int32_t *kept = reinterpret_cast<int32_t *>(base + sel::kScratchBytes + 16);
    float *zl = reinterpret_cast<float *>(base + sel::kScratchBytes + 16 + ((a.k * 4 + 15) & ~15));
    uint8_t *flag = reinterpret_cast<uint8_t *>(zl + a.zs);

    RowStat st = a.stat[row];
    const int D = a.D;
    {
        const int npp = a.np[row];
        const float sa = st.m_acc == -INFINITY ? 0.f : __expf(st.m_acc - st.m_cur);
        float *ac = a.acc + row * D;
        const float *pa = a.partial + row * (a.k + 1) * D;
        for (int d = lane; d < D; d += 64) {
            float v = ac[d] * sa;
            for (int r = 0; r < npp; ++r) v += pa[r * D + d];
            ac[d] = v;
        }
        st.m_acc = st.m_cur;
    }
    const RowLevel rl = row_level(a, row, l);
    const int32_t n = rl.m * a.b + rl.o;
    st.n_keys += n;
    float *zr = a.z + row * a.zs;
    int32_t mm = 0;
    float mz = -INFINITY;
    if (n > 0) {
        for (int i = lane; i < n; i += 64) {
            zl[i] = zr[i];
            flag[i] = 0;
        }
        __threadfence_block();
        if (l >= 1) {
            mm = min(a.k, n);
            sel::Cands cd;
            cd.n = n;
            cd.nchild = rl.m * a.b;
            cd.b = a.b;
            cd.top = 0;
            cd.orphan0 = (int32_t)(rl.part * a.b);
            sel::select<KT>(zl, flag, kept, mm, cd, a.par[l & 1] + row * a.k, lane, scratch, outv);
            int32_t *pn = a.par[(l + 1) & 1] + row * a.k;
            for (int r = lane; r < mm; r += 64) pn[r] = kept[r];
            if (dbg.selected)
                for (int r = lane; r < mm; r += 64)
                    dbg.selected[(row * a.n_levels + (l - 1)) * a.k + r] = kept[r];
            if (dbg.kth_gap && lane == 0) dbg.kth_gap[row * a.n_levels + (l - 1)] = outv[1] - outv[2];
            for (int i = lane; i < n; i += 64)
                if (flag[i]) {
                    zr[i] = -INFINITY;
                    zl[i] = -INFINITY;
                }
            __threadfence_block();
        }
        for (int i = lane; i < n; i += 64) mz = fmaxf(mz, zl[i]);
        mz = wave_max(mz);
    }
    if (l >= 1 && lane == 0) a.mk[(l + 1) & 1][row] = mm;
    const float mn = fmaxf(st.m_cur, mz);
    if (mn > -INFINITY && mz > -INFINITY) {
        float s = 0.f;
        for (int i = lane; i < n; i += 64) s += zl[i] == -INFINITY ? 0.f : __expf(zl[i] - mn);
        s = wave_sum(s);
        st.l = (st.m_cur == -INFINITY ? 0.f : st.l * __expf(st.m_cur - mn)) + s;
        st.m_cur = mn;
    }
    if (lane == 0) {
        a.stat[row] = st;
        a.np[row] = rl.m + (rl.o > 0 ? 1 : 0);
    }
}

// -------------------------------------------------------------------- pv --
// One wave per item: sum over the parent's children c of exp(z_c - max) v_c
// for up to 16 pairs.  MFMA 16x16x32 with k = children (lane group grp holds
// children 8*grp .. 8*grp + 7 of each 32) and n = dimensions: lane column L%16
// of tile t is dimension (D/16)*(L%16) + t, so a lane reads D/16 contiguous
// bf16 of each child row and writes D/16 contiguous floats per pair.
template <int D>
__global__ __launch_bounds__(256) void tp_pv(TreeView tv, TP a, int l, int32_t NP) {
    constexpr int NT = D / 16;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= *a.n_items) return;
    const int4 it = a.items[item];
    const int g = it.x / NP;
    const int64_t p = it.x % NP;
    const int cnt = it.z;
    const int i16 = lane & 15, grp = lane >> 4;
    const bool live = i16 < cnt;
    const int2 pr = a.sorted[it.y + (live ? i16 : 0)];
    const int64_t row = pr.x;
    const int rank = pr.y;
    const RowLevel rl = row_level(a, row, l);
    const int32_t nc = live ? (rank < rl.m ? a.b : rl.o) : 0;
    const float M = a.stat[row].m_cur;
    const float *zr = a.z + row * a.zs + rank * a.b;

    int32_t orow[4], orank[4];
    #pragma unroll
    for (int v = 0; v < 4; ++v) {
        orow[v] = __shfl((int32_t)row, 4 * grp + v);
        orank[v] = __shfl(rank, 4 * grp + v);
    }

    const bf16_t *vals = level_rows(tv, true, l, g, D);
    const int64_t nexist = a.length / a.pw[l];
    const int64_t c0 = p * a.b;
    f32x4 acc[NT];
    #pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < a.b; kc += 32) {
        float w[8];
        #pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int c = kc + 8 * grp + v;
            const float zz = c < nc ? zr[c] : -INFINITY;
            w[v] = zz == -INFINITY ? 0.f : __expf(zz - M);
        }
        bf16x8 ph, pl;
        split8(w, ph, pl);
        u16x8 raw[8];
        #pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int c = kc + 8 * grp + v;
            if (c < a.b && c0 + c < nexist) {
                const bf16_t *vp = vals + (c0 + c) * D + NT * i16;
                if constexpr (NT == 8) {
                    const uint4 x = *reinterpret_cast<const uint4 *>(vp);
                    raw[v] = __builtin_bit_cast(u16x8, x);
                } else {
                    const uint2 x = *reinterpret_cast<const uint2 *>(vp);
                    raw[v] = u16x8{(unsigned short)(x.x & 0xFFFF), (unsigned short)(x.x >> 16),
                                   (unsigned short)(x.y & 0xFFFF), (unsigned short)(x.y >> 16),
                                   0, 0, 0, 0};
                }
            } else {
                raw[v] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        #pragma unroll
        for (int t = 0; t < NT; ++t) {
            u16x8 bt;
            #pragma unroll
            for (int v = 0; v < 8; ++v) bt[v] = raw[v][t];
            const bf16x8 bv = __builtin_bit_cast(bf16x8, bt);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bv, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, bv, acc[t], 0, 0, 0);
        }
    }
    #pragma unroll
    for (int v = 0; v < 4; ++v) {
        if (4 * grp + v < cnt) {
            float *dst = a.partial + ((int64_t)orow[v] * (a.k + 1) + orank[v]) * D + NT * i16;
            float o[NT];
            #pragma unroll
            for (int t = 0; t < NT; ++t) o[t] = acc[t][v];
            Vec<float, NT>::store(dst, o);
        }
    }
}

// ----------------------------------------------------------------- final --
__global__ __launch_bounds__(256) void tp_final(TP a, DebugView dbg) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + w;
    if (row >= a.rows) return;
    const RowStat st = a.stat[row];
    const int D = a.D;
    const int npp = a.np[row];
    const float sa = st.m_acc == -INFINITY ? 0.f : __expf(st.m_acc - st.m_cur);
    const float inv = 1.f / st.l;
    const float *ac = a.acc + row * D;
    const float *pa = a.partial + row * (a.k + 1) * D;
    for (int d = lane; d < D; d += 64) {
        float v = ac[d] * sa;
        for (int r = 0; r < npp; ++r) v += pa[r * D + d];
        v *= inv;
        if (a.out_bf16)
            static_cast<bf16_t *>(a.out)[row * D + d] = (bf16_t)f32_to_bf16(v);
        else
            static_cast<float *>(a.out)[row * D + d] = v;
    }
    if (dbg.n_keys && lane == 0) dbg.n_keys[row] = st.n_keys;
}

// ------------------------------------------------------------------ host --
struct Plan {
    int64_t rows;        // rows per pass
    int64_t nb;          // buckets at the widest level
    int32_t zs;
    size_t off_z, off_par0, off_par1, off_mk0, off_mk1, off_np, off_pp, off_cnt, off_offs, off_ioff,
        off_sorted, off_items, off_nitems, off_partial, off_acc, off_stat, total;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

Plan make_plan(int64_t rows, int32_t Hkv, int32_t D, int32_t b, int32_t k, int32_t maxc,
               int64_t capacity) {
    Plan P{};
    P.rows = rows;
    P.nb = (int64_t)Hkv * (capacity / b + 1);
    P.zs = (maxc + 3) / 4 * 4;
    const int64_t pairs = rows * (k + 1);
    const int64_t items = pairs / kTile + P.nb + 1;
    size_t o = 0;
    auto put = [&](size_t bytes) { const size_t at = o; o = up256(o + bytes); return at; };
    P.off_z = put((size_t)rows * P.zs * 4);
    P.off_par0 = put((size_t)rows * k * 4);
    P.off_par1 = put((size_t)rows * k * 4);
    P.off_mk0 = put((size_t)rows * 4);
    P.off_mk1 = put((size_t)rows * 4);
    P.off_np = put((size_t)rows * 4);
    P.off_pp = put((size_t)pairs * 4);
    P.off_cnt = put((size_t)P.nb * 4);
    P.off_offs = put((size_t)(P.nb + 1) * 4);
    P.off_ioff = put((size_t)(P.nb + 1) * 4);
    P.off_sorted = put((size_t)pairs * 8);
    P.off_items = put((size_t)items * 16);
    P.off_nitems = put(16);
    P.off_partial = put((size_t)pairs * D * 4);
    P.off_acc = put((size_t)rows * D * 4);
    P.off_stat = put((size_t)rows * sizeof(RowStat));
    P.total = o;
    return P;
}

int64_t pass_rows(int64_t rows, int32_t Hq) {
    const int64_t cap = kRowsPerPass / Hq * Hq;
    return rows < cap ? rows : (cap > 0 ? cap : Hq);
}

size_t select_smem_wave(int32_t zs, int32_t k) {
    return up256((size_t)sel::kScratchBytes + 16 + ((k * 4 + 15) & ~15) + (size_t)zs * 5);
}

template <int KT>
hipError_t launch_select_t(const TP &a, const DebugView &dbg, int l, int smw, hipStream_t s) {
    const int64_t blocks = (a.rows + 3) / 4;
    const size_t smem = (size_t)smw * 4;
    if (smem > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void *)tp_select<KT>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(tp_select<KT>, dim3((unsigned)blocks), dim3(256), smem, s, a, dbg, l, smw);
    return hipGetLastError();
}

hipError_t launch_select(const TP &a, const DebugView &dbg, int l, int32_t maxc, int smw,
                         hipStream_t s) {
    if (maxc <= 64 * 2) return launch_select_t<2>(a, dbg, l, smw, s);
    if (maxc <= 64 * 5) return launch_select_t<5>(a, dbg, l, smw, s);
    if (maxc <= 64 * 9) return launch_select_t<9>(a, dbg, l, smw, s);
    if (maxc <= 64 * 17) return launch_select_t<17>(a, dbg, l, smw, s);
    return launch_select_t<0>(a, dbg, l, smw, s);
}

template <int D>
hipError_t run_pass(const TreeView &tv, TP a, const DebugView &dbg, int64_t max_ctx, const Plan &P,
                    int32_t maxc, hipStream_t s) {
    const int64_t rows = a.rows;
    {
        const int64_t n = std::max<int64_t>(std::max<int64_t>(rows * D, P.nb), rows * a.n_levels * a.k);
        const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
        hipLaunchKernelGGL(tp_init, dim3((unsigned)blocks), dim3(256), 0, s, a, dbg, P.nb);
    }
    const int smw = (int)select_smem_wave(a.zs, a.k);
    const int64_t per_head = rows / a.Hq * a.G;
    for (int l = a.top; l >= 0; --l) {
        const int32_t NP = (int32_t)(max_ctx / a.pw[l + 1] + 1);
        const int64_t nb = (int64_t)a.Hkv * NP;
        const int use_lds = NP <= kHistMax;
        hipLaunchKernelGGL(tp_count, dim3((unsigned)((per_head + 255) / 256), (unsigned)a.Hkv), dim3(256),
                           use_lds ? (size_t)NP * 4 : 0, s, a, l, NP, use_lds);
        hipLaunchKernelGGL(tp_scan, dim3(1), dim3(1024), 0, s, a, nb);
        hipLaunchKernelGGL(tp_scatter, dim3((unsigned)((rows + nb + 255) / 256)), dim3(256), 0, s, a, l, NP,
                           nb);
        const int64_t pairs = rows * (int64_t)std::min(a.k + 1, (int)NP);
        const int64_t items = pairs / kTile + nb + 1;
        const unsigned ib = (unsigned)((items + 3) / 4);
        hipLaunchKernelGGL(tp_score<D>, dim3(ib), dim3(256), 0, s, tv, a, l, NP);
        hipError_t e = launch_select(a, dbg, l, maxc, smw, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(tp_pv<D>, dim3(ib), dim3(256), 0, s, tv, a, l, NP);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(tp_final, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a, dbg);
    return hipGetLastError();
}

}  // namespace

size_t tiled_workspace_bytes(int64_t rows, int32_t Hq, int32_t Hkv, int32_t D, int32_t b, int32_t k,
                             int32_t maxc, int64_t capacity) {
    return make_plan(pass_rows(rows, Hq), Hkv, D, b, k, maxc, capacity).total;
}

size_t tiled_select_lds_bytes(int32_t maxc, int32_t k) {
    return 4 * select_smem_wave((maxc + 3) / 4 * 4, k);
}

hipError_t launch_prefill_tiled(const TreeView &tv, int32_t D, const DescendArgs &da, int32_t Hkv,
                                int64_t length, int64_t capacity, const DebugView &dbg, void *ws,
                                hipStream_t s) {
    const int64_t per = pass_rows(da.rows, da.Hq);
    const Plan P = make_plan(per, Hkv, D, da.b, da.k, da.max_cand, capacity);
    unsigned char *w = static_cast<unsigned char *>(ws);
    TP a{};
    a.Hq = da.Hq;
    a.G = da.G;
    a.Hkv = Hkv;
    a.D = D;
    a.ctx_step = da.ctx_step;
    a.b = da.b;
    a.k = da.k;
    a.zs = P.zs;
    a.scale = da.scale;
    a.out_bf16 = da.out_bf16;
    a.n_levels = tv.n_levels;
    a.length = length;
    a.z = reinterpret_cast<float *>(w + P.off_z);
    a.par[0] = reinterpret_cast<int32_t *>(w + P.off_par0);
    a.par[1] = reinterpret_cast<int32_t *>(w + P.off_par1);
    a.mk[0] = reinterpret_cast<int32_t *>(w + P.off_mk0);
    a.mk[1] = reinterpret_cast<int32_t *>(w + P.off_mk1);
    a.np = reinterpret_cast<int32_t *>(w + P.off_np);
    a.pairpos = reinterpret_cast<int32_t *>(w + P.off_pp);
    a.counts = reinterpret_cast<int32_t *>(w + P.off_cnt);
    a.offs = reinterpret_cast<int32_t *>(w + P.off_offs);
    a.itemoff = reinterpret_cast<int32_t *>(w + P.off_ioff);
    a.sorted = reinterpret_cast<int2 *>(w + P.off_sorted);
    a.items = reinterpret_cast<int4 *>(w + P.off_items);
    a.n_items = reinterpret_cast<int32_t *>(w + P.off_nitems);
    a.partial = reinterpret_cast<float *>(w + P.off_partial);
    a.acc = reinterpret_cast<float *>(w + P.off_acc);
    a.stat = reinterpret_cast<RowStat *>(w + P.off_stat);
    const size_t esz_q = 2, esz_o = da.out_bf16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < da.rows; r0 += per) {
        const int64_t rows = std::min(per, da.rows - r0);
        const int64_t q0 = r0 / da.Hq;
        a.rows = rows;
        a.q = reinterpret_cast<const bf16_t *>(static_cast<const unsigned char *>(da.q) + r0 * D * esz_q);
        a.out = static_cast<unsigned char *>(da.out) + r0 * D * esz_o;
        a.ctx_base = da.ctx_base + q0 * da.ctx_step;
        const int64_t max_ctx = a.ctx_base + (rows / da.Hq - 1) * da.ctx_step;
        a.top = 0;
        a.pw[0] = 1;
        for (int l = 1; l < kMaxLevels + 2; ++l) {
            a.pw[l] = a.pw[l - 1] <= max_ctx ? a.pw[l - 1] * da.b : a.pw[l - 1];
            if (a.pw[l] <= max_ctx && a.pw[l] > a.pw[l - 1]) a.top = l;
        }
        DebugView d = dbg;
        if (d.selected) d.selected += r0 * tv.n_levels * da.k;
        if (d.kth_gap) d.kth_gap += r0 * tv.n_levels;
        if (d.n_keys) d.n_keys += r0;
        const hipError_t e = D == 128 ? run_pass<128>(tv, a, d, max_ctx, P, da.max_cand, s)
                                      : run_pass<64>(tv, a, d, max_ctx, P, da.max_cand, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace recsa
