// Causal prefill, parent-major, on gfx950 (bf16 storage).
//
// RecSA, abstract (sentences on selection and on RoPE): a level above the tokens
// keeps no more than k of its candidates; every candidate it drops contributes its
// summary to the same softmax that the exact tokens reached at the bottom join;
// the rotary position of an entry is its rank in the candidate list of its level
// (the query sits at the level's candidate count n).
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
//           (equal logits: lower index); the others are entries; kept logits
//           become -inf;
//   pv      per 16 pairs of one parent: the pair's entries as a softmax state
//           of their own (max m, sum l of exp(z - m), and the sum of
//           exp(z - m) times the children's values, bf16 exact, on MFMA);
// At level 0 the children are tokens, every candidate is an entry and nothing
// is selected, so scoring, the pairs' softmax states and P.V are one kernel.
// One last pass merges all pairs' states of a row (as split attention merges
// its splits) into the output.
#include <math.h>

#include <algorithm>

#include "recsa_internal.hpp"
#include "select_topk.hpp"

namespace recsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kTile = 16;               // pairs per MFMA tile (the M side)
constexpr int kMaxFanout = 128;         // children per parent the P.V tiles hold
constexpr int kHistSplit = 4096;        // up to this many parents per head: one LDS count per 256 rows
constexpr int kHistMax = 24576;         // ... and up to this many when a head has kHistRows rows or more
constexpr int64_t kHistRows = 2048;
constexpr int kRange = 2048;            // else: parents per counting block
constexpr int kScanPer = 16;            // bucket sizes per thread in the scans
constexpr int kScanChunk = kScanPer * 256;
constexpr int64_t kRowsPerPass = 1 << 18;   // rows per pass: 8192 queries of 32 heads

struct TP {
    const bf16_t *q;           // [rows][D]
    void *out;                 // [rows][D]
    int32_t out_bf16;
    int32_t Hq, G, Hkv, D;
    int64_t rows;              // rows of this pass
    int64_t rows_cap;          // rows per pass the workspace holds
    int64_t ctx_base;          // n_ctx of row 0's query
    int32_t ctx_step;
    int32_t b, k, zs;          // zs: row stride of z (floats)
    float scale;
    int32_t top;               // highest level any row reaches
    int32_t n_levels;          // levels of the tree (debug layout)
    int32_t lv;                // level slots of the per-level arrays (n_levels + 1)
    int64_t length;            // tokens in the tree
    int64_t pw[kMaxLevels + 2];  // b^l
    // workspace
    float *z;                  // [rows][zs]
    int32_t *par[2];           // [rows][k]: parents by level parity
    int32_t *mk[2];            // [rows]: kept parents by level parity
    int32_t *pairpos;          // [rows][k+1]
    int32_t *counts;           // [nb]
    int32_t *offs;             // [nb+1]
    int32_t *itemoff;          // [nb+1]
    int2 *bsum;                // [nb / kScanChunk + 1]
    int4 *sorted;              // [items][16]: (row, rank, query position, children) by parent
    int4 *items;               // (bucket, 0, pairs, 0)
    int32_t *n_items;
    float *partial;            // [lv][rows_cap][k+1][D]: sum of exp(z - m) v per pair
    float2 *pml;               // [lv][rows_cap][k+1]: (m, sum of exp(z - m)) per pair
    int32_t *nplev;            // [rows][lv]: pairs at each level
    float2 *rowml;             // [rows] (max, sum) of each row's softmax, when not null (backward)
};

// The backward's inputs and outputs for one pass of rows.
struct TB {
    const float *dout;         // [rows][D] fp32
    float *dq;                 // [rows][D] fp32, added to
    float *dk, *dv;            // [Hkv][cap][D] fp32 token gradients, added to (NULL: skipped)
    float *gk[kMaxLevels + 1]; // [Hkv][node_cap][D] fp32 summary gradients (l >= 1), added to
    float *gv[kMaxLevels + 1];
    const float2 *rowml;       // [rows] (max, sum) from the forward
    const float *rowD;         // [rows] <dO, out>
    const int32_t *sel;        // [rows][n_levels][k] kept nodes by level, -1 padded
    int64_t cap;               // token capacity (row stride of a head in dk, dv)
    int64_t node_cap[kMaxLevels + 1];
    BwdTreeArgs tree;          // the tree pass's arguments common to every level (interleaved runs)
    int32_t dq_slots;          // dq shares to per-pair slots, added per level by tb_dq_add (many
                               // rows); else fp32 atomics straight into dq (few rows)
    float *stage_k, *stage_v;  // bf16 token gradients: level 0's items store their sums here,
                               // [items][b][D] fp32, for the tree pass at level 1 to add (NULL: no)
};

struct RowLevel {
    int32_t m;       // kept parents
    int32_t o;       // orphans (children of the partial parent)
    int64_t part;    // the partial parent's node id (N_{l+1})
};

// x / y for 0 <= x < 2^31 and y >= 1 in 32-bit arithmetic (64-bit division is a long
// emulated sequence on the GPU); rows, contexts and node ids all stay below 2^31.
__device__ __forceinline__ uint32_t div32(int64_t x, int64_t y) {
    return y > x ? 0u : (uint32_t)x / (uint32_t)y;
}

__device__ __forceinline__ RowLevel row_level(const TP &a, int64_t row, int l) {
    const int64_t n = a.ctx_base + (int64_t)div32(row, a.Hq) * a.ctx_step;
    const int64_t up = div32(n, a.pw[l + 1]);
    RowLevel r;
    r.m = a.mk[l & 1][row];
    r.o = (int32_t)((int64_t)div32(n, a.pw[l]) - (int64_t)a.b * up);
    r.part = up;
    return r;
}

__device__ __forceinline__ int64_t parent_of(const TP &a, int64_t row, int l, int rank,
                                             const RowLevel &rl) {
    return rank < rl.m ? (int64_t)a.par[l & 1][row * a.k + rank] : rl.part;
}

__device__ __forceinline__ int64_t head_row(const TP &a, int g, int64_t t) {
    const uint32_t q = div32(t, a.G);
    return (int64_t)q * a.Hq + (int64_t)g * a.G + (t - (int64_t)q * a.G);
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

// Exclusive scan of (x, y) over a 256-thread block; `total` gets the block sums.
__device__ __forceinline__ int2 block_scan(int2 v, int2 &total) {
    __shared__ int2 wsum[4];
    const int lane = threadIdx.x & 63, w = wave_id();
    int2 inc = v;
    #pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int yx = __shfl_up(inc.x, o), yy = __shfl_up(inc.y, o);
        if (lane >= o) {
            inc.x += yx;
            inc.y += yy;
        }
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int2 base = make_int2(0, 0);
    total = make_int2(0, 0);
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < w) {
            base.x += wsum[i].x;
            base.y += wsum[i].y;
        }
        total.x += wsum[i].x;
        total.y += wsum[i].y;
    }
    __syncthreads();
    return make_int2(base.x + inc.x - v.x, base.y + inc.y - v.y);
}

// ---------------------------------------------------------------- set-up --
__global__ void tp_init(TP a, DebugView dbg, int64_t nb) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = t; i < a.rows; i += stride) {
        a.mk[a.top & 1][i] = 0;
        if (dbg.n_keys) dbg.n_keys[i] = 0;
    }
    for (int64_t i = t; i < nb; i += stride) a.counts[i] = 0;
    if (dbg.selected)
        for (int64_t i = t; i < a.rows * a.n_levels * a.k; i += stride) dbg.selected[i] = -1;
    if (dbg.kth_gap)
        for (int64_t i = t; i < a.rows * a.n_levels; i += stride) dbg.kth_gap[i] = NAN;
}

// Position of every pair of level l inside its (head, parent) bucket, and the
// bucket sizes.  mode 0 (few parents, or up to kHistMax over at least kHistRows
// rows per head): each block counts 256 rows of one head in LDS, then adds to the
// global sizes (one atomic per parent and block).
// mode 1 (many parents): each block owns a range of kRange parents of one head,
// counts the pairs of all of the head's rows that fall in it, and stores the
// sizes of its range; no global atomics.
__global__ __launch_bounds__(1024) void tp_count(TP a, int l, int32_t NP, int mode) {
    extern __shared__ int32_t hist[];
    const int g = blockIdx.y;
    const int64_t per_head = a.rows / a.Hq * a.G;
    if (mode == 1) {
        const int64_t p0 = (int64_t)blockIdx.x * kRange;
        const int32_t np_blk = (int32_t)min<int64_t>(kRange, NP - p0);
        for (int p = threadIdx.x; p < np_blk; p += blockDim.x) hist[p] = 0;
        __syncthreads();
        for (int64_t t = threadIdx.x; t < per_head; t += blockDim.x) {
            const int64_t row = head_row(a, g, t);
            const RowLevel rl = row_level(a, row, l);
            const int32_t np = rl.m + (rl.o > 0 ? 1 : 0);
            int32_t *pp = a.pairpos + row * (a.k + 1);
            for (int r = 0; r < np; ++r) {
                const int64_t p = parent_of(a, row, l, r, rl) - p0;
                if (p >= 0 && p < np_blk) pp[r] = atomicAdd(&hist[p], 1);
            }
        }
        __syncthreads();
        for (int p = threadIdx.x; p < np_blk; p += blockDim.x) a.counts[(int64_t)g * NP + p0 + p] = hist[p];
        return;
    }
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int p = threadIdx.x; p < NP; p += blockDim.x) hist[p] = 0;
    __syncthreads();
    int64_t row = -1;
    RowLevel rl{0, 0, 0};
    int32_t np = 0;
    if (t < per_head) {
        row = head_row(a, g, t);
        rl = row_level(a, row, l);
        np = rl.m + (rl.o > 0 ? 1 : 0);
    }
    int32_t *pp = a.pairpos + (row >= 0 ? row : 0) * (a.k + 1);
    for (int r = 0; r < np; ++r) pp[r] = atomicAdd(&hist[parent_of(a, row, l, r, rl)], 1);
    __syncthreads();
    #pragma unroll 4
    for (int p = threadIdx.x; p < NP; p += blockDim.x) {
        const int32_t c = hist[p];
        if (c) hist[p] = atomicAdd(&a.counts[(int64_t)g * NP + p], c);
    }
    __syncthreads();
    for (int r = 0; r < np; ++r) pp[r] += hist[parent_of(a, row, l, r, rl)];
}

// Exclusive scans of the bucket sizes (pair offsets) and of their tiles (item
// offsets) in three steps: per-chunk sums, a scan of the chunk sums, per-chunk
// scans; the last step also clears the sizes for the next level.
__device__ __forceinline__ void scan_load(const TP &a, int64_t nb, int64_t e0, int32_t *c) {
    if (e0 + kScanPer <= nb) {
        #pragma unroll
        for (int i = 0; i < kScanPer; i += 4) {
            const int4 v = *reinterpret_cast<const int4 *>(a.counts + e0 + i);
            c[i] = v.x; c[i + 1] = v.y; c[i + 2] = v.z; c[i + 3] = v.w;
        }
    } else {
        #pragma unroll
        for (int i = 0; i < kScanPer; ++i) c[i] = e0 + i < nb ? a.counts[e0 + i] : 0;
    }
}

__global__ __launch_bounds__(256) void tp_scan_sums(TP a, int64_t nb) {
    const int64_t e0 = (int64_t)blockIdx.x * kScanChunk + threadIdx.x * kScanPer;
    int32_t c[kScanPer];
    scan_load(a, nb, e0, c);
    int2 v = make_int2(0, 0);
    #pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        v.x += c[i];
        v.y += (c[i] + kTile - 1) / kTile;
    }
    int2 total;
    block_scan(v, total);
    if (threadIdx.x == 0) a.bsum[blockIdx.x] = total;
}

__global__ __launch_bounds__(256) void tp_scan_chunks(TP a, int64_t nb, int64_t nchunks) {
    int2 carry = make_int2(0, 0);
    for (int64_t c0 = 0; c0 < nchunks; c0 += 256) {
        const int64_t i = c0 + threadIdx.x;
        const int2 v = i < nchunks ? a.bsum[i] : make_int2(0, 0);
        int2 total;
        const int2 ex = block_scan(v, total);
        if (i < nchunks) a.bsum[i] = make_int2(carry.x + ex.x, carry.y + ex.y);
        carry.x += total.x;
        carry.y += total.y;
    }
    if (threadIdx.x == 0) {
        a.offs[nb] = carry.x;
        a.itemoff[nb] = carry.y;
        *a.n_items = carry.y;
    }
}

__global__ __launch_bounds__(256) void tp_scan_write(TP a, int64_t nb) {
    const int64_t e0 = (int64_t)blockIdx.x * kScanChunk + threadIdx.x * kScanPer;
    int32_t c[kScanPer];
    scan_load(a, nb, e0, c);
    int2 v = make_int2(0, 0);
    #pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        v.x += c[i];
        v.y += (c[i] + kTile - 1) / kTile;
    }
    int2 total;
    int2 ex = block_scan(v, total);
    const int2 base = a.bsum[blockIdx.x];
    ex.x += base.x;
    ex.y += base.y;
    for (int i = 0; i < kScanPer && e0 + i < nb; ++i) {
        a.offs[e0 + i] = ex.x;
        a.itemoff[e0 + i] = ex.y;
        ex.x += c[i];
        ex.y += (c[i] + kTile - 1) / kTile;
        a.counts[e0 + i] = 0;
    }
}

// Both scans in one workgroup, chunk after chunk with a carry: for few buckets
// (every level above the tokens) one launch instead of three.
constexpr int64_t kScanSmall = 4 * kScanChunk;

__global__ __launch_bounds__(256) void tp_scan_small(TP a, int64_t nb) {
    int2 carry = make_int2(0, 0);
    for (int64_t base = 0; base < nb; base += kScanChunk) {
        const int64_t e0 = base + threadIdx.x * kScanPer;
        int32_t c[kScanPer];
        scan_load(a, nb, e0, c);
        int2 v = make_int2(0, 0);
        #pragma unroll
        for (int i = 0; i < kScanPer; ++i) {
            v.x += c[i];
            v.y += (c[i] + kTile - 1) / kTile;
        }
        int2 total;
        int2 ex = block_scan(v, total);
        ex.x += carry.x;
        ex.y += carry.y;
        for (int i = 0; i < kScanPer && e0 + i < nb; ++i) {
            a.offs[e0 + i] = ex.x;
            a.itemoff[e0 + i] = ex.y;
            ex.x += c[i];
            ex.y += (c[i] + kTile - 1) / kTile;
            a.counts[e0 + i] = 0;
        }
        carry.x += total.x;
        carry.y += total.y;
    }
    if (threadIdx.x == 0) {
        a.offs[nb] = carry.x;
        a.itemoff[nb] = carry.y;
        *a.n_items = carry.y;
    }
}

// Pairs into bucket order, each with what scoring needs: (row, rank, the
// query's RoPE position n - rank*b, the parent's children in the row's view);
// one item per tile of a bucket.
__global__ __launch_bounds__(256) void tp_scatter(TP a, DebugView dbg, int l, int32_t NP, int64_t nb) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < a.rows) {
        const int64_t row = t;
        const RowLevel rl = row_level(a, row, l);
        const int32_t np = rl.m + (rl.o > 0 ? 1 : 0);
        const int32_t n = rl.m * a.b + rl.o;
        const int64_t g = div32(row - (int64_t)div32(row, a.Hq) * a.Hq, a.G);
        a.nplev[row * a.lv + l] = np;
        if (dbg.n_keys) dbg.n_keys[row] += n;
        for (int r = 0; r < np; ++r) {
            const int64_t bkt = g * NP + parent_of(a, row, l, r, rl);
            a.sorted[(int64_t)a.itemoff[bkt] * kTile + a.pairpos[row * (a.k + 1) + r]] =
                make_int4((int32_t)row, r, n - r * a.b, r < rl.m ? a.b : rl.o);
        }
    } else if (t - a.rows < nb) {
        const int64_t bkt = t - a.rows;
        const int32_t c = a.offs[bkt + 1] - a.offs[bkt], i0 = a.itemoff[bkt];
        for (int32_t s = 0; s < c; s += kTile)
            a.items[i0 + s / kTile] = make_int4((int32_t)bkt, 0, min(kTile, c - s), 0);
        for (int32_t s = c; s % kTile != 0; ++s)
            a.sorted[(int64_t)i0 * kTile + s] = make_int4(0, 0, 0, 0);
    }
}

// ----------------------------------------------------------------- items --
// An item is a tile of up to 16 pairs of one (KV head, parent) bucket; its
// pairs are sorted[16 i .. 16 i + 15] (unused slots: row 0, rank 0, position
// 0, no children).  The kernels over items run persistent waves that fetch the
// next item's records while working on the current one, and issue every load
// of an item before its arithmetic.
//
// MFMA 16x16x32 (bf16 in, fp32 accumulate): lane L supplies A row L%16 and B
// column L%16 for the 8 k-slots of lane group grp = L/16, and gets D rows
// 4*grp .. 4*grp + 3 of column L%16.
struct Item {
    int g;          // KV head
    int64_t p;      // parent node
    int cnt;        // pairs
    int4 pr;        // this lane's pair (L%16): row, rank, query position, children
    int32_t orow[4], orank[4], onc[4];   // pairs 4*grp + v, the D rows of this lane
    int64_t idx;    // the item's index in the level's item list
};

template <typename F>
__device__ __forceinline__ void for_items(const TP &a, int32_t NP, int lane, F &&body) {
    const int64_t n = *a.n_items;
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    int64_t item = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_id();
    if (item >= n) return;
    const int i16 = lane & 15, grp = lane >> 4;
    int4 rec = a.items[item];
    int4 pr = a.sorted[item * kTile + i16];
    for (;;) {
        const int64_t next = item + nw;
        int4 rn = rec, pn = pr;
        if (next < n) {
            rn = a.items[next];
            pn = a.sorted[next * kTile + i16];
        }
        Item it;
        it.idx = item;
        const int32_t bkt = __builtin_amdgcn_readfirstlane(rec.x);   // uniform over the wave
        // (the division runs on the vector unit; bring the uniform results back to scalars)
        it.g = __builtin_amdgcn_readfirstlane(bkt / NP);
        it.p = __builtin_amdgcn_readfirstlane(bkt % NP);
        it.cnt = __builtin_amdgcn_readfirstlane(rec.z);
        it.pr = pr;
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
            it.orow[v] = __shfl(pr.x, 4 * grp + v);
            it.orank[v] = __shfl(pr.y, 4 * grp + v);
            it.onc[v] = __shfl(pr.w, 4 * grp + v);
        }
        body(it);
        if (next >= n) break;
        item = next;
        rec = rn;
        pr = pn;
    }
}

// cos/sin of child offsets 0..b-1 into LDS, rows padded by two pairs against bank conflicts
constexpr int crot_stride(int D) { return D / 2 + 2; }

__device__ __forceinline__ void load_crot(const TreeView &tv, int b, int D, float2 *crot) {
    const int H = D / 2;
    for (int i = threadIdx.x; i < b * H; i += blockDim.x) crot[(i / H) * (H + 2) + i % H] = tv.rope[i];
    __syncthreads();
}

// Query slices of this lane's pair: k-slot (ks, v) of lane group grp is dimension
// grp*D/8 + 8*ks + v for ks < D/64 and its RoPE partner (+ D/2) at ks + D/64, so
// rotations stay inside a lane and row slices are contiguous.
template <int D>
struct QRaw {
    uint4 q[2 * (D / 64)];
    float4 cs[4 * (D / 64)];
};

template <int D>
__device__ __forceinline__ void load_query(const TreeView &tv, const TP &a, const Item &it, int lane,
                                           QRaw<D> &r) {
    constexpr int H = D / 2, PG = D / 8, KS1 = D / 64;
    const int grp = lane >> 4;
    const bf16_t *qr = a.q + (int64_t)it.pr.x * D + grp * PG;
    const float4 *cs = reinterpret_cast<const float4 *>(tv.rope + (int64_t)it.pr.z * H + grp * PG);
    #pragma unroll
    for (int pc = 0; pc < KS1; ++pc) {
        r.q[2 * pc] = *reinterpret_cast<const uint4 *>(qr + 8 * pc);
        r.q[2 * pc + 1] = *reinterpret_cast<const uint4 *>(qr + H + 8 * pc);
        #pragma unroll
        for (int u = 0; u < 4; ++u) r.cs[4 * pc + u] = cs[4 * pc + u];
    }
}

__device__ __forceinline__ void unpack8(uint4 x, float *f) {
    f[0] = bf16_to_f32(x.x & 0xFFFFu); f[1] = bf16_to_f32(x.x >> 16);
    f[2] = bf16_to_f32(x.y & 0xFFFFu); f[3] = bf16_to_f32(x.y >> 16);
    f[4] = bf16_to_f32(x.z & 0xFFFFu); f[5] = bf16_to_f32(x.z >> 16);
    f[6] = bf16_to_f32(x.w & 0xFFFFu); f[7] = bf16_to_f32(x.w >> 16);
}

// rotate (x1, x2) by the 8 (cos, sin) pairs in cs and split to bf16
__device__ __forceinline__ void rotate_split(uint4 a1, uint4 a2, const float4 *cs, bf16x8 &h1, bf16x8 &l1,
                                             bf16x8 &h2, bf16x8 &l2) {
    float x1[8], x2[8], r1[8], r2[8];
    unpack8(a1, x1);
    unpack8(a2, x2);
    #pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float4 v = cs[u];
        r1[2 * u] = x1[2 * u] * v.x - x2[2 * u] * v.y;
        r2[2 * u] = x2[2 * u] * v.x + x1[2 * u] * v.y;
        r1[2 * u + 1] = x1[2 * u + 1] * v.z - x2[2 * u + 1] * v.w;
        r2[2 * u + 1] = x2[2 * u + 1] * v.z + x1[2 * u + 1] * v.w;
    }
    split8(r1, h1, l1);
    split8(r2, h2, l2);
}

// (Slots past the item's pairs rotate row 0's query: their rows of every product are
// dropped by the consumers' masks, so they need no zeroing.)
template <int D>
__device__ __forceinline__ void query_operands(const QRaw<D> &r, const Item &it, int lane, bf16x8 *ah,
                                               bf16x8 *al) {
    constexpr int KS1 = D / 64;
    #pragma unroll
    for (int pc = 0; pc < KS1; ++pc)
        rotate_split(r.q[2 * pc], r.q[2 * pc + 1], &r.cs[4 * pc], ah[pc], al[pc], ah[pc + KS1],
                     al[pc + KS1]);
}

// Key slices of children 32*kk + 16*t + L%16 (t = 0, 1) in the same k-slot layout.
template <int D>
struct KRaw {
    uint4 k[2][2 * (D / 64)];
};

template <int D>
__device__ __forceinline__ void load_keys(const bf16_t *keys, int64_t c0, int64_t nexist, int b, int kk,
                                          int lane, KRaw<D> &r) {
    constexpr int H = D / 2, PG = D / 8, KS1 = D / 64;
    const int i16 = lane & 15, grp = lane >> 4;
    // a uniform base (the parent's first child, or the last node when it has none) and
    // 32-bit byte offsets: the loads take a scalar base; lanes past the children read
    // the base row
    const char *kb = reinterpret_cast<const char *>(keys + (c0 < nexist ? c0 : nexist - 1) * D);
    #pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int c = 32 * kk + 16 * t + i16;
        const bool ok = c < b && c0 + c < nexist;
        const uint32_t off = ((ok ? (uint32_t)c * D : 0u) + grp * PG) * (uint32_t)sizeof(bf16_t);
        #pragma unroll
        for (int pc = 0; pc < KS1; ++pc) {
            r.k[t][2 * pc] = *reinterpret_cast<const uint4 *>(kb + off + 16 * pc);
            r.k[t][2 * pc + 1] = *reinterpret_cast<const uint4 *>(kb + off + 2 * H + 16 * pc);
        }
    }
}

// Logits (unscaled) of pairs 4*grp + v against child 32*kk + 16*t + L%16.
template <int D>
__device__ __forceinline__ f32x4 score_tile(const KRaw<D> &r, int t, const float2 *crot, int64_t c0,
                                            int64_t nexist, int b, int kk, int lane, const bf16x8 *ah,
                                            const bf16x8 *al) {
    constexpr int PG = D / 8, KS1 = D / 64;
    const int i16 = lane & 15, grp = lane >> 4;
    const int c = 32 * kk + 16 * t + i16;
    const bool ok = c < b && c0 + c < nexist;
    // a missing child's column is scored against the base row and dropped by every
    // consumer's mask (c < the pair's children), so it needs no zeroing
    const float4 *cs = reinterpret_cast<const float4 *>(crot + (ok ? c : 0) * crot_stride(D) + grp * PG);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int pc = 0; pc < KS1; ++pc) {
        float4 c4[4];
        #pragma unroll
        for (int u = 0; u < 4; ++u) c4[u] = cs[4 * pc + u];
        bf16x8 h1, l1, h2, l2;
        rotate_split(r.k[t][2 * pc], r.k[t][2 * pc + 1], c4, h1, l1, h2, l2);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[pc], h1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[pc], l1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[pc], h1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[pc + KS1], h2, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[pc + KS1], l2, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[pc + KS1], h2, acc, 0, 0, 0);
    }
    return acc;
}

// Value slices of children 32*kk + 8*grp + v: lane column L%16 of output tile
// t is dimension (D/16)*(L%16) + t, so a lane reads D/16 contiguous bf16 per child.
template <int D>
struct VRaw {
    uint4 v[8];     // D/16 bf16 of each child (upper half unused for D = 64)
};

template <int D>
__device__ __forceinline__ void load_values(const bf16_t *vals, int64_t c0, int64_t nexist, int b, int kk,
                                            int lane, VRaw<D> &r) {
    constexpr int NT = D / 16;
    const int i16 = lane & 15, grp = lane >> 4;
    const char *vb = reinterpret_cast<const char *>(vals + (c0 < nexist ? c0 : nexist - 1) * D);
    #pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int c = 32 * kk + 8 * grp + v;
        const bool ok = c < b && c0 + c < nexist;
        const bf16_t *vp = reinterpret_cast<const bf16_t *>(
            vb + ((ok ? (uint32_t)c * D : 0u) + NT * i16) * (uint32_t)sizeof(bf16_t));
        uint4 x;
        if constexpr (NT == 8) {
            x = *reinterpret_cast<const uint4 *>(vp);
        } else {
            const uint2 y = *reinterpret_cast<const uint2 *>(vp);
            x = make_uint4(y.x, y.y, 0u, 0u);
        }
        r.v[v] = x;     // a missing child's P weight is 0, and its row here is the base row's
    }
}

template <int D>
__device__ __forceinline__ void pv_accumulate(const VRaw<D> &r, const float *w, f32x4 *acc) {
    constexpr int NT = D / 16;
    bf16x8 ph, pl;
    split8(w, ph, pl);
    #pragma unroll
    for (int t = 0; t < NT; ++t) {
        u16x8 bt;
        #pragma unroll
        for (int v = 0; v < 8; ++v) {
            const uint32_t word = t < 2 ? r.v[v].x : t < 4 ? r.v[v].y : t < 6 ? r.v[v].z : r.v[v].w;
            bt[v] = (unsigned short)((t & 1) ? (word >> 16) : (word & 0xFFFFu));
        }
        const bf16x8 bv = __builtin_bit_cast(bf16x8, bt);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bv, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, bv, acc[t], 0, 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void pv_store(const TP &a, const Item &it, int lane, const f32x4 *acc, float *slice) {
    constexpr int NT = D / 16;
    const int i16 = lane & 15, grp = lane >> 4;
    #pragma unroll
    for (int v = 0; v < 4; ++v) {
        if (4 * grp + v < it.cnt) {
            float *dst = slice + ((int64_t)it.orow[v] * (a.k + 1) + it.orank[v]) * D + NT * i16;
            float o[NT];
            #pragma unroll
            for (int t = 0; t < NT; ++t) o[t] = acc[t][v];
            Vec<float, NT>::store(dst, o);
        }
    }
}

// exp(z - m) of this lane's children given their logits (-inf: not an entry),
// with m and l reduced over the pair's four lane groups; lane group 0 stores (m, l).
template <int KC>
__device__ __forceinline__ void pair_softmax(const TP &a, const Item &it, int l, int lane, float (*w)[8]) {
    float m = -INFINITY;
    #pragma unroll
    for (int kk = 0; kk < KC; ++kk)
        #pragma unroll
        for (int v = 0; v < 8; ++v) m = fmaxf(m, w[kk][v]);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    float sum = 0.f;
    #pragma unroll
    for (int kk = 0; kk < KC; ++kk)
        #pragma unroll
        for (int v = 0; v < 8; ++v) {
            const float e = w[kk][v] == -INFINITY ? 0.f : __expf(w[kk][v] - m);
            w[kk][v] = e;
            sum += e;
        }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    if (lane < 16 && lane < it.cnt)
        a.pml[((int64_t)l * a.rows_cap + it.pr.x) * (a.k + 1) + it.pr.y] = make_float2(m, sum);
}

// ----------------------------------------------------------------- score --
// Level l >= 1: each item's pairs against the parent's children; logits to z.
template <int D, int KC>
__global__ __launch_bounds__(256) void tp_score(TreeView tv, TP a, int l, int32_t NP) {
    extern __shared__ __align__(16) unsigned char smem[];
    float2 *crot = reinterpret_cast<float2 *>(smem);
    load_crot(tv, a.b, D, crot);
    const int lane = threadIdx.x & 63;
    const int64_t nexist = a.length / a.pw[l];
    for_items(a, NP, lane, [&](const Item &it) {
        const bf16_t *keys = level_rows(tv, false, l, it.g, D);
        const int64_t c0 = it.p * a.b;
        QRaw<D> qr;
        KRaw<D> kr;
        load_query<D>(tv, a, it, lane, qr);
        load_keys<D>(keys, c0, nexist, a.b, 0, lane, kr);
        bf16x8 ah[D / 32], al[D / 32];
        query_operands<D>(qr, it, lane, ah, al);
        #pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            if (kk > 0) load_keys<D>(keys, c0, nexist, a.b, kk, lane, kr);
            #pragma unroll
            for (int t = 0; t < 2; ++t) {
                const f32x4 acc = score_tile<D>(kr, t, crot, c0, nexist, a.b, kk, lane, ah, al);
                const int c = 32 * kk + 16 * t + (lane & 15);
                #pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (c < it.onc[v])
                        a.z[(int64_t)it.orow[v] * a.zs + it.orank[v] * a.b + c] = a.scale * acc[v];
            }
        }
    });
}

// ---------------------------------------------------------------- select --
// One wave per row: keeps the top min(k, n) candidates of level l (l >= 1) as
// the next level's parents; kept candidates' logits become -inf so the P.V
// pass skips them.
template <int KT>
__device__ __forceinline__ void select_row(const TP &a, const DebugView &dbg, int l, int64_t row, int lane,
                                           unsigned char *scratch, float *outv, int32_t *kept,
                                           int32_t *parl, uint8_t *flag) {
    RowLevel rl = row_level(a, row, l);
    rl.m = __builtin_amdgcn_readfirstlane(rl.m);        // uniform over the wave (one row)
    const int32_t n = rl.m * a.b + rl.o;
    const int32_t mm = min(a.k, n);
    if (lane == 0) a.mk[(l + 1) & 1][row] = mm;
    if (n == 0) return;
    float *zr = a.z + row * a.zs;
    const int32_t *par = a.par[l & 1] + row * a.k;
    for (int r = lane; r < rl.m; r += 64) parl[r] = par[r];
    for (int i = 4 * lane; i < n; i += 256) *reinterpret_cast<uint32_t *>(flag + i) = 0u;
    sel::wave_fence();
    sel::Cands cd;
    cd.n = n;
    cd.nchild = rl.m * a.b;
    cd.b = a.b;
    cd.bmul = sel::fanout_magic((uint32_t)a.b);
    cd.top = 0;
    cd.orphan0 = (int32_t)(rl.part * a.b);
    sel::select<KT>(zr, flag, kept, mm, cd, parl, lane, scratch, outv);
    int32_t *pn = a.par[(l + 1) & 1] + row * a.k;
    for (int r = lane; r < mm; r += 64) pn[r] = kept[r];
    if (dbg.selected)
        for (int r = lane; r < mm; r += 64) dbg.selected[(row * a.n_levels + (l - 1)) * a.k + r] = kept[r];
    if (dbg.kth_gap && lane == 0) dbg.kth_gap[row * a.n_levels + (l - 1)] = outv[1] - outv[2];
    for (int i = lane; i < n; i += 64)
        if (flag[i]) zr[i] = -INFINITY;
}

// A row's inputs to the selection, loaded ahead: its kept-parent count, this lane's
// parent (rank lane) and its logits lane, lane + 64, ... (the whole padded row; the
// slots past the row's candidates are masked once their number is known).
template <int KT>
struct SelIn {
    int32_t m, par;
    float z[KT];
};

template <int KT>
__device__ __forceinline__ void sel_fetch(const TP &a, int l, int64_t row, int lane, SelIn<KT> &f) {
    f.m = a.mk[l & 1][row];
    f.par = lane < a.k ? a.par[l & 1][row * a.k + lane] : 0;
    const float *zr = a.z + row * a.zs;
    #pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int32_t i = lane + 64 * t;
        f.z[t] = i < a.zs ? zr[i] : 0.f;
    }
}

// select_row with its inputs already in registers (KT > 0)
template <int KT>
__device__ __forceinline__ void select_row_in(const TP &a, const DebugView &dbg, int l, int64_t row, int lane,
                                              const SelIn<KT> &f, unsigned char *scratch, float *outv,
                                              int32_t *kept, int32_t *parl, uint8_t *flag) {
    const int64_t nctx = a.ctx_base + (int64_t)div32(row, a.Hq) * a.ctx_step;
    const int64_t up = div32(nctx, a.pw[l + 1]);
    RowLevel rl;
    rl.m = __builtin_amdgcn_readfirstlane(f.m);
    rl.o = (int32_t)((int64_t)div32(nctx, a.pw[l]) - (int64_t)a.b * up);
    rl.part = up;
    const int32_t n = rl.m * a.b + rl.o;
    const int32_t mm = min(a.k, n);
    if (lane == 0) a.mk[(l + 1) & 1][row] = mm;
    if (n == 0) return;
    float *zr = a.z + row * a.zs;
    const int32_t *par = a.par[l & 1] + row * a.k;
    // ranks below 64 come from the prefetch; only wider budgets load the rest here
    // (a load waited on here would also wait for the next row's prefetch)
    if (lane < rl.m) parl[lane] = f.par;
    for (int r = lane + 64; r < rl.m; r += 64) parl[r] = par[r];
    for (int i = 4 * lane; i < n; i += 256) *reinterpret_cast<uint32_t *>(flag + i) = 0u;
    sel::wave_fence();
    sel::Cands cd;
    cd.n = n;
    cd.nchild = rl.m * a.b;
    cd.b = a.b;
    cd.bmul = sel::fanout_magic((uint32_t)a.b);
    cd.top = 0;
    cd.orphan0 = (int32_t)(rl.part * a.b);
    uint32_t kk[KT];
    #pragma unroll
    for (int t = 0; t < KT; ++t) kk[t] = lane + 64 * t < n ? sel::ordered_bits(f.z[t]) : 0u;
    sel::select_from_keys<KT>(kk, zr, flag, kept, mm, cd, parl, lane, scratch, outv);
    int32_t *pn = a.par[(l + 1) & 1] + row * a.k;
    for (int r = lane; r < mm; r += 64) pn[r] = kept[r];
    if (dbg.selected)
        for (int r = lane; r < mm; r += 64) dbg.selected[(row * a.n_levels + (l - 1)) * a.k + r] = kept[r];
    if (dbg.kth_gap && lane == 0) dbg.kth_gap[row * a.n_levels + (l - 1)] = outv[1] - outv[2];
    for (int i = lane; i < n; i += 64)
        if (flag[i]) zr[i] = -INFINITY;
}

// Persistent waves over rows; with the keys in registers (KT > 0) each wave loads the
// next row's inputs before selecting the current row, so the loads' latency hides
// behind the selection.
template <int KT>
__global__ __launch_bounds__(256) void tp_select(TP a, DebugView dbg, int l, int smem_wave) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int w = wave_id(), lane = threadIdx.x & 63;
    const int kq = (a.k * 4 + 15) & ~15;
    unsigned char *base = smem + w * smem_wave;
    unsigned char *scratch = base;                                             // 16-aligned
    float *outv = reinterpret_cast<float *>(base + sel::kScratchBytes);        // [4]
    int32_t *kept = reinterpret_cast<int32_t *>(base + sel::kScratchBytes + 16);
    int32_t *parl = reinterpret_cast<int32_t *>(base + sel::kScratchBytes + 16 + kq);
    uint8_t *flag = base + sel::kScratchBytes + 16 + 2 * kq;
    const int64_t stride = (int64_t)gridDim.x * 4;
    int64_t row = (int64_t)blockIdx.x * 4 + w;
    if constexpr (KT == 0) {
        for (; row < a.rows; row += stride) select_row<KT>(a, dbg, l, row, lane, scratch, outv, kept, parl, flag);
    } else {
        if (row >= a.rows) return;
        // every row's inputs arrive in nxt and are copied to cur at the top of its
        // iteration (the one wait for them), so nothing in the selection waits on a
        // load; the next row's loads are then in flight during the selection
        SelIn<KT> cur, nxt;
        sel_fetch<KT>(a, l, row, lane, nxt);
        for (;;) {
            cur = nxt;
            const int64_t next = row + stride;
            if (next < a.rows) sel_fetch<KT>(a, l, next, lane, nxt);
            select_row_in<KT>(a, dbg, l, row, lane, cur, scratch, outv, kept, parl, flag);
            if (next >= a.rows) break;
            row = next;
        }
    }
}

// -------------------------------------------------------------------- pv --
// Level l >= 1: each pair's entries (children whose logits are not -inf) as a
// softmax state: (m, l) to pml, sum exp(z - m) v to the level's partial slice.
template <int D, int KC>
__global__ __launch_bounds__(256) void tp_pv(TreeView tv, TP a, int l, int32_t NP) {
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4;
    const int64_t nexist = a.length / a.pw[l];
    float *slice = a.partial + (int64_t)l * a.rows_cap * (a.k + 1) * D;
    for_items(a, NP, lane, [&](const Item &it) {
        const bf16_t *vals = level_rows(tv, true, l, it.g, D);
        const int64_t c0 = it.p * a.b;
        const int32_t nc = (lane & 15) < it.cnt ? it.pr.w : 0;
        const float *zr = a.z + (int64_t)it.pr.x * a.zs + it.pr.y * a.b;
        float w[KC][8];
        #pragma unroll
        for (int kk = 0; kk < KC; ++kk)
            #pragma unroll
            for (int v = 0; v < 8; ++v) {
                const int c = 32 * kk + 8 * grp + v;
                const float zz = zr[c < nc ? c : 0];
                w[kk][v] = c < nc ? zz : -INFINITY;
            }
        VRaw<D> vr;
        load_values<D>(vals, c0, nexist, a.b, 0, lane, vr);
        pair_softmax<KC>(a, it, l, lane, w);
        f32x4 acc[D / 16];
        #pragma unroll
        for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        #pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            if (kk > 0) load_values<D>(vals, c0, nexist, a.b, kk, lane, vr);
            pv_accumulate<D>(vr, w[kk], acc);
        }
        pv_store<D>(a, it, lane, acc, slice);
    });
}

// Level l >= 1, fanout <= 32: the same per pair, over runs of RUN consecutive
// items per wave.  A bucket's items are consecutive, so a run mostly shares one
// parent: every item's logits are loaded at the run's start and the parent's
// values once per parent, so a run waits on memory about twice instead of once
// per item.  Long runs suit many items; with few, they leave waves idle.
constexpr int64_t kLongRunRows = 16384;   // rows per pass from which runs are 8 items long

__device__ __forceinline__ Item make_item(int4 rec, int4 pr, int32_t NP, int grp) {
    Item it;
    const int32_t bkt = __builtin_amdgcn_readfirstlane(rec.x);
    it.g = __builtin_amdgcn_readfirstlane(bkt / NP);
    it.p = __builtin_amdgcn_readfirstlane(bkt % NP);
    it.cnt = __builtin_amdgcn_readfirstlane(rec.z);
    it.pr = pr;
    #pragma unroll
    for (int v = 0; v < 4; ++v) {
        it.orow[v] = __shfl(pr.x, 4 * grp + v);
        it.orank[v] = __shfl(pr.y, 4 * grp + v);
        it.onc[v] = __shfl(pr.w, 4 * grp + v);
    }
    return it;
}

template <int D, int KC, int kRun>
__global__ __launch_bounds__(256) void tp_pv_runs(TreeView tv, TP a, int l, int32_t NP) {
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, i16 = lane & 15;
    const int64_t nexist = a.length / a.pw[l];
    float *slice = a.partial + (int64_t)l * a.rows_cap * (a.k + 1) * D;
    const int64_t n = *a.n_items;
    const int64_t nruns = (n + kRun - 1) / kRun;
    // a rank's logits start 16-byte aligned (zs is a multiple of 4), and the 32 KC slots
    // the lane groups read from the last rank's start (k b) lie inside the row
    const bool vec_z = (a.b & 3) == 0 && a.k * a.b + 32 * KC <= a.zs;
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    // each run's item records (bucket and pair count, uniform; this lane's pair)
    struct Recs {
        int32_t bkt[kRun], cnt[kRun];
        int4 pr[kRun];
    };
    auto fetch = [&](int64_t run, Recs &r) {
        const int64_t i0 = run * kRun;
        #pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const int64_t i = i0 + u < n ? i0 + u : i0;
            const int4 rec = a.items[i];
            r.bkt[u] = __builtin_amdgcn_readfirstlane(rec.x);
            r.cnt[u] = __builtin_amdgcn_readfirstlane(rec.z);
            r.pr[u] = a.sorted[i * kTile + i16];
        }
    };
    int64_t run = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_id();
    if (run >= nruns) return;
    Recs cur, nxt;
    fetch(run, cur);
    for (;;) {
        const int64_t next = run + nw;
        if (next < nruns) fetch(next, nxt);        // the next run's records, ahead of this run's loads
        const int64_t i0 = run * kRun;
        const int nit = (int)__builtin_amdgcn_readfirstlane((int32_t)min<int64_t>(kRun, n - i0));
        const int32_t *bkt = cur.bkt, *cnt = cur.cnt;
        const int4 *pr = cur.pr;
        float w[kRun][KC][8];
        #pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const int32_t nc = (u < nit && i16 < cnt[u]) ? pr[u].w : 0;
            const float *zr = a.z + (int64_t)pr[u].x * a.zs;
            #pragma unroll
            for (int kk = 0; kk < KC; ++kk) {
                const int32_t seg = pr[u].y * a.b + 32 * kk + 8 * grp;   // this lane's 8 logits in the row
                float zz[8];
                if (vec_z) {
                    // two 16-byte loads (the slots past the children read the row's next
                    // logits, which the mask below drops)
                    const float4 x0 = *reinterpret_cast<const float4 *>(zr + seg);
                    const float4 x1 = *reinterpret_cast<const float4 *>(zr + seg + 4);
                    zz[0] = x0.x; zz[1] = x0.y; zz[2] = x0.z; zz[3] = x0.w;
                    zz[4] = x1.x; zz[5] = x1.y; zz[6] = x1.z; zz[7] = x1.w;
                } else {
                    #pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        const int c = 32 * kk + 8 * grp + v;
                        zz[v] = zr[c < nc ? pr[u].y * a.b + c : 0];
                    }
                }
                #pragma unroll
                for (int v = 0; v < 8; ++v) w[u][kk][v] = 32 * kk + 8 * grp + v < nc ? zz[v] : -INFINITY;
            }
        }
        VRaw<D> vr[KC];
        int32_t held = -1;                  // the bucket whose values vr holds
        #pragma unroll
        for (int u = 0; u < kRun; ++u) {
            if (u < nit) {
                const Item it = make_item(make_int4(bkt[u], 0, cnt[u], 0), pr[u], NP, grp);
                if (bkt[u] != held) {
                    const bf16_t *vals = level_rows(tv, true, l, it.g, D);
                    #pragma unroll
                    for (int kk = 0; kk < KC; ++kk) load_values<D>(vals, it.p * a.b, nexist, a.b, kk, lane, vr[kk]);
                    held = bkt[u];
                }
                pair_softmax<KC>(a, it, l, lane, w[u]);
                f32x4 acc[D / 16];
                #pragma unroll
                for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                #pragma unroll
                for (int kk = 0; kk < KC; ++kk) pv_accumulate<D>(vr[kk], w[u][kk], acc);
                pv_store<D>(a, it, lane, acc, slice);
            }
        }
        if (next >= nruns) break;
        run = next;
        cur = nxt;
    }
}

// tp_score over runs of kRun consecutive items: the items of one (head, parent)
// bucket are consecutive, so a run mostly scores one parent's children, and those
// keys are loaded once per parent rather than once per item (at the upper levels a
// parent has tens of items, and re-reading its keys from L2 bounds the kernel).
template <int D, int KC, int kRun>
__global__ __launch_bounds__(256) void tp_score_runs(TreeView tv, TP a, int l, int32_t NP) {
    extern __shared__ __align__(16) unsigned char smem[];
    float2 *crot = reinterpret_cast<float2 *>(smem);
    load_crot(tv, a.b, D, crot);
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, i16 = lane & 15;
    const int64_t nexist = a.length / a.pw[l];
    const int64_t n = *a.n_items;
    const int64_t nruns = (n + kRun - 1) / kRun;
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    struct Recs {
        int32_t bkt[kRun], cnt[kRun];
        int4 pr[kRun];
    };
    auto fetch = [&](int64_t run, Recs &r) {
        const int64_t i0 = run * kRun;
        #pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const int64_t i = i0 + u < n ? i0 + u : i0;
            const int4 rec = a.items[i];
            r.bkt[u] = __builtin_amdgcn_readfirstlane(rec.x);
            r.cnt[u] = __builtin_amdgcn_readfirstlane(rec.z);
            r.pr[u] = a.sorted[i * kTile + i16];
        }
    };
    int64_t run = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_id();
    if (run >= nruns) return;
    Recs cur, nxt;
    fetch(run, cur);
    for (;;) {
        const int64_t next = run + nw;
        if (next < nruns) fetch(next, nxt);
        const int64_t i0 = run * kRun;
        const int nit = (int)__builtin_amdgcn_readfirstlane((int32_t)min<int64_t>(kRun, n - i0));
        KRaw<D> kr[KC];
        int32_t held = -1;                  // the bucket whose keys kr holds
        #pragma unroll
        for (int u = 0; u < kRun; ++u) {
            if (u < nit) {
                const Item it = make_item(make_int4(cur.bkt[u], 0, cur.cnt[u], 0), cur.pr[u], NP, grp);
                const int64_t c0 = it.p * a.b;
                QRaw<D> qr;
                load_query<D>(tv, a, it, lane, qr);
                if (cur.bkt[u] != held) {
                    const bf16_t *keys = level_rows(tv, false, l, it.g, D);
                    #pragma unroll
                    for (int kk = 0; kk < KC; ++kk) load_keys<D>(keys, c0, nexist, a.b, kk, lane, kr[kk]);
                    held = cur.bkt[u];
                }
                bf16x8 ah[D / 32], al[D / 32];
                query_operands<D>(qr, it, lane, ah, al);
                #pragma unroll
                for (int kk = 0; kk < KC; ++kk) {
                    #pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4 acc = score_tile<D>(kr[kk], t, crot, c0, nexist, a.b, kk, lane, ah, al);
                        const int c = 32 * kk + 16 * t + i16;
                        #pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (c < it.onc[v])
                                a.z[(int64_t)it.orow[v] * a.zs + it.orank[v] * a.b + c] = a.scale * acc[v];
                    }
                }
            }
        }
        if (next >= nruns) break;
        run = next;
        cur = nxt;
    }
}

// ---------------------------------------------------------------- attend --
// Level 0: each item's pairs against the parent's tokens, the pairs' softmax
// states and P.V in one pass; the logits go through LDS from the score tile's
// layout (pair rows 4*grp + v) to the P.V operand's (pair row L%16).
template <int D, int KC>
__global__ __launch_bounds__(256) void tp_attend(TreeView tv, TP a, int32_t NP) {
    extern __shared__ __align__(16) unsigned char smem[];
    float2 *crot = reinterpret_cast<float2 *>(smem);
    load_crot(tv, a.b, D, crot);
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int i16 = lane & 15, grp = lane >> 4;
    constexpr int ZS = 32 * KC + 1;
    float *zw = reinterpret_cast<float *>(smem + (size_t)a.b * crot_stride(D) * sizeof(float2)) +
                wv * kTile * ZS;
    const int64_t nexist = a.length;
    for_items(a, NP, lane, [&](const Item &it) {
        const bf16_t *keys = level_rows(tv, false, 0, it.g, D);
        const bf16_t *vals = level_rows(tv, true, 0, it.g, D);
        const int64_t c0 = it.p * a.b;
        QRaw<D> qr;
        KRaw<D> kr;
        VRaw<D> vr;
        load_query<D>(tv, a, it, lane, qr);
        load_keys<D>(keys, c0, nexist, a.b, 0, lane, kr);
        load_values<D>(vals, c0, nexist, a.b, 0, lane, vr);
        bf16x8 ah[D / 32], al[D / 32];
        query_operands<D>(qr, it, lane, ah, al);
        #pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            if (kk > 0) load_keys<D>(keys, c0, nexist, a.b, kk, lane, kr);
            #pragma unroll
            for (int t = 0; t < 2; ++t) {
                const f32x4 acc = score_tile<D>(kr, t, crot, c0, nexist, a.b, kk, lane, ah, al);
                const int c = 32 * kk + 16 * t + i16;
                #pragma unroll
                for (int v = 0; v < 4; ++v) zw[(4 * grp + v) * ZS + c] = c < it.onc[v] ? a.scale * acc[v] : -INFINITY;
            }
        }
        sel::wave_fence();      // the tile is this wave's: no wait for its loads in flight
        float w[KC][8];
        #pragma unroll
        for (int kk = 0; kk < KC; ++kk)
            #pragma unroll
            for (int v = 0; v < 8; ++v) w[kk][v] = zw[i16 * ZS + 32 * kk + 8 * grp + v];
        sel::wave_fence();
        pair_softmax<KC>(a, it, 0, lane, w);
        f32x4 acc[D / 16];
        #pragma unroll
        for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        #pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            if (kk > 0) load_values<D>(vals, c0, nexist, a.b, kk, lane, vr);
            pv_accumulate<D>(vr, w[kk], acc);
        }
        pv_store<D>(a, it, lane, acc, a.partial);
    });
}

// ------------------------------------------------------------- backward --
// Gradients of <dO, out> with the selection of the forward held fixed, per
// (KV head, parent) item of up to 16 pairs: the pairs' logits against the
// parent's children (score_tile) and dp = <dO, v> (dot_tile) on MFMA; then per
// chunk of 32 children, with p = e^(z - M) / L (0 for kept or missing
// children) and dz = s p (dp - D):
//   dV_c += sum_pairs p dO,  dK_c += R(-c) sum_pairs dz U  (U = R(n - r b) q),
//   dq += R(-(n - r b)) sum_c dz R(c) k_c,
// summed over the item's pairs in registers first, so each (child, dim) takes
// one atomic add per item rather than one per pair.  In that phase lane j holds
// the RoPE pair (j, j + D/2) of every pair of the item and the wave walks the
// children, so each atomic instruction covers consecutive dimensions of one
// child (two cache lines) instead of one dimension of 64 children.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// <dO, v> of pairs 4*grp + v against child 32*kk + 16*t + L%16: values in the keys'
// k-slot layout (bf16, exact as the B operand), dO split into bf16 hi + lo.
template <int D>
__device__ __forceinline__ f32x4 dot_tile(const KRaw<D> &r, int t, const bf16x8 *dh, const bf16x8 *dl) {
    constexpr int KS1 = D / 64;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int pc = 0; pc < KS1; ++pc) {
        const bf16x8 v1 = __builtin_bit_cast(bf16x8, r.k[t][2 * pc]);
        const bf16x8 v2 = __builtin_bit_cast(bf16x8, r.k[t][2 * pc + 1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dh[pc], v1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dl[pc], v1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dh[pc + KS1], v2, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dl[pc + KS1], v2, acc, 0, 0, 0);
    }
    return acc;
}

template <int D>
__host__ __device__ constexpr size_t tb_wave_lds() {
    return (size_t)32 * D * 2 + (size_t)2 * 32 * kTile * 4 + (size_t)kTile * 4 * 4;
}

// ST: level 0 with bf16 token gradients (the items' sums go to the staging buffer)
template <int D, int KC, bool ST>
__global__ __launch_bounds__(256) void tb_item(TreeView tv, TP a, TB t, int l, int32_t NP) {
    constexpr int H = D / 2, PG = D / 8, KS1 = D / 64;
    constexpr int SUB = 64 / H;                  // children per step of the wave (1 at D = 128, 2 at D = 64)
    extern __shared__ __align__(16) unsigned char smem[];
    float2 *crot = reinterpret_cast<float2 *>(smem);
    load_crot(tv, a.b, D, crot);
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int i16 = lane & 15, grp = lane >> 4;
    const int j = lane % H, sb = lane / H;       // the lane's RoPE pair (j, j + H) and child sub-step
    unsigned char *wb = smem + (size_t)a.b * crot_stride(D) * sizeof(float2) + (size_t)wv * tb_wave_lds<D>();
    uint16_t *Kb = reinterpret_cast<uint16_t *>(wb);                  // [32][D] the chunk's keys (bf16)
    float *Pt = reinterpret_cast<float *>(Kb + 32 * D);               // [32 children][16 pairs]
    float *dZt = Pt + 32 * kTile;                                     // [32][16]
    uint32_t *kmask = reinterpret_cast<uint32_t *>(dZt + 32 * kTile); // [16][4] kept children bits
    const int64_t nexist = a.length / a.pw[l];
    const int32_t b = a.b;
    // ST: the tokens' gradients go to the item's own rows of the staging buffer, every
    // child of the parent stored (zeros included), no atomics and nothing read
    constexpr bool staged = ST;
    const bool grads_here = l > 0 || t.dk != nullptr || staged;
    for_items(a, NP, lane, [&](const Item &it) {
        // a bucket of one item is the only writer of its parent's children's gradients in
        // this launch: it reads, adds and stores them instead of adding with atomics
        // (~280 G float atomics/s across the chip, which the token level's ~1 G adds per
        // 4096-query chunk would wait on)
        const int64_t bkt = (int64_t)it.g * NP + it.p;
        const bool excl = grads_here && !staged &&
                          __builtin_amdgcn_readfirstlane(a.itemoff[bkt + 1] - a.itemoff[bkt]) == 1;
        const bf16_t *keys = level_rows(tv, false, l, it.g, D);
        const bf16_t *vals = level_rows(tv, true, l, it.g, D);
        const int64_t c0 = it.p * b;
        wave_sync();                        // the previous item's LDS reads are done
        // queries rotated to their rank position (the score's A operand)
        QRaw<D> qr;
        load_query<D>(tv, a, it, lane, qr);
        bf16x8 ah[D / 32], al[D / 32];
        query_operands<D>(qr, it, lane, ah, al);
        // dO of the pairs split into the A operand of <dO, v>
        bf16x8 dh[D / 32], dl[D / 32];
        {
            const float live = i16 < it.cnt ? 1.f : 0.f;
            const float *dp = t.dout + (int64_t)it.pr.x * D;
            #pragma unroll
            for (int pc = 0; pc < KS1; ++pc) {
                float x1[8], x2[8];
                #pragma unroll
                for (int v = 0; v < 8; v += 4) {
                    const float4 y1 = *reinterpret_cast<const float4 *>(dp + grp * PG + 8 * pc + v);
                    const float4 y2 = *reinterpret_cast<const float4 *>(dp + H + grp * PG + 8 * pc + v);
                    x1[v] = live * y1.x; x1[v + 1] = live * y1.y; x1[v + 2] = live * y1.z; x1[v + 3] = live * y1.w;
                    x2[v] = live * y2.x; x2[v + 1] = live * y2.y; x2[v + 2] = live * y2.z; x2[v + 3] = live * y2.w;
                }
                split8(x1, dh[pc], dl[pc]);
                split8(x2, dh[pc + KS1], dl[pc + KS1]);
            }
        }
        // children of the parent that a pair's row kept at this level (they are not entries)
        if (grp == 0) {
            uint32_t m4[4] = {0u, 0u, 0u, 0u};
            if (l >= 1 && i16 < it.cnt) {
                const int32_t *ks = t.sel + ((int64_t)it.pr.x * a.n_levels + (l - 1)) * a.k;
                for (int r = 0; r < a.k; ++r) {
                    const int32_t id = ks[r];
                    const int64_t c = (int64_t)id - c0;
                    if (id >= 0 && c >= 0 && c < b) m4[c >> 5] |= 1u << (c & 31);
                }
            }
            #pragma unroll
            for (int u = 0; u < 4; ++u) kmask[i16 * 4 + u] = m4[u];
        }
        // per D-row pair (4*grp + v): the row's softmax statistics
        float Mv[4], Lv[4], Dv[4];
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
            const bool ok = 4 * grp + v < it.cnt;
            const float2 ml = ok ? t.rowml[it.orow[v]] : make_float2(0.f, 1.f);
            Mv[v] = ml.x;
            Lv[v] = 1.f / ml.y;
            Dv[v] = ok ? t.rowD[it.orow[v]] : 0.f;
        }
        wave_sync();
        // dq of every pair of the item in the children's frame, dimensions (j, j + H)
        float dq1[kTile], dq2[kTile];
        #pragma unroll
        for (int pr = 0; pr < kTile; ++pr) { dq1[pr] = 0.f; dq2[pr] = 0.f; }
        for (int kk = 0; kk < KC; ++kk) {
            KRaw<D> kr, vr;
            load_keys<D>(keys, c0, nexist, b, kk, lane, kr);
            load_keys<D>(vals, c0, nexist, b, kk, lane, vr);
            // the chunk's keys to LDS (bf16), for dq
            #pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                #pragma unroll
                for (int pc = 0; pc < KS1; ++pc) {
                    *reinterpret_cast<uint4 *>(Kb + (16 * tt + i16) * D + grp * PG + 8 * pc) = kr.k[tt][2 * pc];
                    *reinterpret_cast<uint4 *>(Kb + (16 * tt + i16) * D + H + grp * PG + 8 * pc) = kr.k[tt][2 * pc + 1];
                }
            // p and dz of pairs 4*grp .. 4*grp + 3 against child 32*kk + cc, to [cc][pair]
            #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const f32x4 zt = score_tile<D>(kr, tt, crot, c0, nexist, b, kk, lane, ah, al);
                const f32x4 pt = dot_tile<D>(vr, tt, dh, dl);
                const int cc = 16 * tt + i16;
                const int c = 32 * kk + cc;
                float pe4[4], dz4[4];
                #pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int pr = 4 * grp + v;
                    const bool kept = (kmask[pr * 4 + (c >> 5)] >> (c & 31)) & 1u;
                    const bool ok = pr < it.cnt && c < it.onc[v] && !kept;
                    pe4[v] = ok ? __expf(a.scale * zt[v] - Mv[v]) * Lv[v] : 0.f;
                    dz4[v] = a.scale * pe4[v] * (pt[v] - Dv[v]);
                }
                *reinterpret_cast<float4 *>(Pt + cc * kTile + 4 * grp) = make_float4(pe4[0], pe4[1], pe4[2], pe4[3]);
                *reinterpret_cast<float4 *>(dZt + cc * kTile + 4 * grp) = make_float4(dz4[0], dz4[1], dz4[2], dz4[3]);
            }
            wave_sync();
            // per child: dV, dK (one atomic add per dimension) and its share of dq
            {
                // every pair's rotated query U = R((n - r b) theta) q and dO in dimensions
                // (j, j + H), straight from memory (the same products as the score's operand)
                float u1[kTile], u2[kTile], o1[kTile], o2[kTile];
                #pragma unroll
                for (int pr = 0; pr < kTile; ++pr) {
                    const int row = __builtin_amdgcn_readlane(it.pr.x, pr);
                    const int pos = __builtin_amdgcn_readlane(it.pr.z, pr);
                    const bf16_t *qp = a.q + (int64_t)row * D;
                    const float x1 = bf16_to_f32(qp[j]), x2 = bf16_to_f32(qp[H + j]);
                    const float2 cs = tv.rope[(int64_t)pos * H + j];
                    u1[pr] = x1 * cs.x - x2 * cs.y;
                    u2[pr] = x2 * cs.x + x1 * cs.y;
                    const bool live = pr < it.cnt;
                    o1[pr] = live ? t.dout[(int64_t)row * D + j] : 0.f;
                    o2[pr] = live ? t.dout[(int64_t)row * D + H + j] : 0.f;
                }
                const int nc = b - 32 * kk < 32 ? b - 32 * kk : 32;      // children in this chunk
                // exclusive bucket: this lane's old dV, dK values of the child kAhead steps
                // ahead are loaded before the current child's arithmetic, to hide their latency
                auto grad_rows = [&](int c, float *&gk, float *&gv) {
                    if (staged) {
                        gk = t.stage_k + (it.idx * b + c) * D;
                        gv = t.stage_v + (it.idx * b + c) * D;
                        return;
                    }
                    gk = l == 0 ? t.dk + ((int64_t)it.g * t.cap + c0 + c) * D
                                : t.gk[l] + ((int64_t)it.g * t.node_cap[l] + c0 + c) * D;
                    gv = l == 0 ? t.dv + ((int64_t)it.g * t.cap + c0 + c) * D
                                : t.gv[l] + ((int64_t)it.g * t.node_cap[l] + c0 + c) * D;
                };
                auto fetch_old = [&](int cc, float *o) {
                    const int c = 32 * kk + cc;
                    if (cc < nc && c0 + c < nexist) {
                        float *gk, *gv;
                        grad_rows(c, gk, gv);
                        o[0] = gv[j];
                        o[1] = gv[H + j];
                        o[2] = gk[j];
                        o[3] = gk[H + j];
                    }
                };
                constexpr int kAhead = 2;
                float ring[kAhead][4];
                #pragma unroll
                for (int u = 0; u < kAhead; ++u) {
                    #pragma unroll
                    for (int q = 0; q < 4; ++q) ring[u][q] = 0.f;
                    if (excl) fetch_old(u * SUB + sb, ring[u]);
                }
                for (int s0 = 0; s0 < nc; s0 += SUB) {
                    float cur[4];
                    #pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        cur[q] = ring[0][q];
                        #pragma unroll
                        for (int u = 0; u + 1 < kAhead; ++u) ring[u][q] = ring[u + 1][q];
                    }
                    if (excl) fetch_old(s0 + kAhead * SUB + sb, ring[kAhead - 1]);
                    const int cc = s0 + sb;
                    const bool inb = cc < nc;
                    const int ccl = inb ? cc : 0;
                    const int c = 32 * kk + ccl;
                    float pv[kTile], dz[kTile];
                    #pragma unroll
                    for (int q4 = 0; q4 < kTile / 4; ++q4) {
                        const float4 x = *reinterpret_cast<const float4 *>(Pt + ccl * kTile + 4 * q4);
                        const float4 y = *reinterpret_cast<const float4 *>(dZt + ccl * kTile + 4 * q4);
                        pv[4 * q4] = x.x; pv[4 * q4 + 1] = x.y; pv[4 * q4 + 2] = x.z; pv[4 * q4 + 3] = x.w;
                        dz[4 * q4] = y.x; dz[4 * q4 + 1] = y.y; dz[4 * q4 + 2] = y.z; dz[4 * q4 + 3] = y.w;
                    }
                    bool any = false;
                    #pragma unroll
                    for (int pr = 0; pr < kTile; ++pr) {
                        if (!inb) { pv[pr] = 0.f; dz[pr] = 0.f; }
                        any = any || pv[pr] != 0.f || dz[pr] != 0.f;
                    }
                    float v1 = 0.f, v2 = 0.f, k1 = 0.f, k2 = 0.f;
                    #pragma unroll
                    for (int pr = 0; pr < kTile; ++pr) {
                        v1 += pv[pr] * o1[pr];
                        v2 += pv[pr] * o2[pr];
                        k1 += dz[pr] * u1[pr];
                        k2 += dz[pr] * u2[pr];
                    }
                    const float2 cs = crot[c * crot_stride(D) + j];         // (cos, sin) of c theta_j
                    if ((staged ? inb : any) && grads_here && c0 + c < nexist) {
                        float *gk, *gv;
                        grad_rows(c, gk, gv);
                        const float dk1 = k1 * cs.x + k2 * cs.y, dk2 = k2 * cs.x - k1 * cs.y;   // R(-c theta)
                        if (excl || staged) {
                            gv[j] = cur[0] + v1;
                            gv[H + j] = cur[1] + v2;
                            gk[j] = cur[2] + dk1;
                            gk[H + j] = cur[3] + dk2;
                        } else {
                            atomicAdd(gv + j, v1);
                            atomicAdd(gv + H + j, v2);
                            atomicAdd(gk + j, dk1);
                            atomicAdd(gk + H + j, dk2);
                        }
                    }
                    const float x1 = bf16_to_f32(Kb[ccl * D + j]), x2 = bf16_to_f32(Kb[ccl * D + H + j]);
                    const float r1 = x1 * cs.x - x2 * cs.y, r2 = x2 * cs.x + x1 * cs.y;   // R(c theta) k_c
                    #pragma unroll
                    for (int pr = 0; pr < kTile; ++pr) {
                        dq1[pr] += dz[pr] * r1;
                        dq2[pr] += dz[pr] * r2;
                    }
                }
            }
            wave_sync();                    // the next chunk rewrites Kb, Pt and dZt
        }
        // dq share of each pair, R(-(n - r b) theta) of the sums.  With many rows, to the
        // pair's own slot (row, rank) of the forward's per-pair buffer, free once its
        // output is merged: plain stores, which tb_dq_add then adds to the rows' dq (an
        // atomic add per dimension and pair would wait on the chip's atomic rate); with
        // few rows, atomics (no extra launch)
        if (SUB == 2) {
            #pragma unroll
            for (int pr = 0; pr < kTile; ++pr) {
                dq1[pr] += __shfl_xor(dq1[pr], 32);
                dq2[pr] += __shfl_xor(dq2[pr], 32);
            }
        }
        #pragma unroll
        for (int pr = 0; pr < kTile; ++pr) {
            if (pr < it.cnt) {
                const int row = __builtin_amdgcn_readlane(it.pr.x, pr);
                const int rank = __builtin_amdgcn_readlane(it.pr.y, pr);
                const int pos = __builtin_amdgcn_readlane(it.pr.z, pr);
                if (sb == 0) {
                    const float2 r = tv.rope[(int64_t)pos * H + j];
                    const float x1 = dq1[pr] * r.x + dq2[pr] * r.y, x2 = dq2[pr] * r.x - dq1[pr] * r.y;
                    if (t.dq_slots) {
                        float *slot = a.partial + ((int64_t)row * (a.k + 1) + rank) * D;
                        slot[j] = x1;
                        slot[H + j] = x2;
                    } else {
                        float *dq = t.dq + (int64_t)row * D;
                        atomicAdd(dq + j, x1);
                        atomicAdd(dq + H + j, x2);
                    }
                }
            }
        }
    });
}

// dq of each row += the dq shares tb_item stored for its pairs of level l (slots
// (row, rank) for rank < the row's pairs at l); one thread per (row, 4 dimensions).
__global__ __launch_bounds__(256) void tb_dq_add(TP a, float *dq, int l) {
    const int D4 = a.D / 4;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.rows * D4;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = div32(t, D4);
        const int j = (int)(t - row * D4);
        const int np = a.nplev[row * a.lv + l];
        const float4 *src = reinterpret_cast<const float4 *>(a.partial) + row * (a.k + 1) * D4 + j;
        float4 *dst = reinterpret_cast<float4 *>(dq) + row * D4 + j;
        float4 v = *dst;
        for (int r = 0; r < np; ++r) {
            const float4 x = src[(int64_t)r * D4];
            v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
        }
        *dst = v;
    }
}

// Staged bf16 token gradients of tokens [n1 * b, length) of head blockIdx.x, the
// children of the partial level-1 parent n1 (all tokens when n1 = 0): the sums of
// the staged items of their bucket (head, parent n1), zeros when no row reads them.
__global__ __launch_bounds__(256) void tb_stage_tail(const int32_t *itemoff, const float *sk, const float *sv,
                                                     bf16_t *dk16, bf16_t *dv16, int64_t cap, int32_t b,
                                                     int32_t D, int32_t NP0, int64_t n1, int64_t length) {
    const int g = blockIdx.x;
    const int64_t bkt = (int64_t)g * NP0 + n1;
    const int32_t i0 = itemoff[bkt], i1 = itemoff[bkt + 1];
    const int32_t ntok = (int32_t)(length - n1 * b);
    const int32_t D4 = D / 4;
    for (int32_t x = threadIdx.x; x < ntok * D4; x += blockDim.x) {
        const int32_t c = x / D4, e = (x - c * D4) * 4;
        float k[4] = {0.f, 0.f, 0.f, 0.f}, v[4] = {0.f, 0.f, 0.f, 0.f};
        for (int32_t it = i0; it < i1; ++it) {
            const float4 a = *reinterpret_cast<const float4 *>(sk + ((int64_t)it * b + c) * D + e);
            const float4 w = *reinterpret_cast<const float4 *>(sv + ((int64_t)it * b + c) * D + e);
            k[0] += a.x; k[1] += a.y; k[2] += a.z; k[3] += a.w;
            v[0] += w.x; v[1] += w.y; v[2] += w.z; v[3] += w.w;
        }
        const int64_t o = ((int64_t)g * cap + n1 * b + c) * D + e;
        Vec<bf16_t, 4>::store(dk16 + o, k);
        Vec<bf16_t, 4>::store(dv16 + o, v);
    }
}

// The kept nodes of level l + 1 (the parents of level l) from the forward's record.
__global__ void tb_parents(TP a, const int32_t *sel, int l) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= a.rows) return;
    int32_t m = 0;
    if (l < a.top) {
        const int32_t *ks = sel + (row * a.n_levels + l) * a.k;
        for (int r = 0; r < a.k; ++r) {
            const int32_t id = ks[r];
            if (id >= 0) a.par[l & 1][row * a.k + m++] = id;
        }
    }
    a.mk[l & 1][row] = m;
}

// <dO, out> per row.
__global__ void tb_rowdot(const float *dout, const float *out, float *rowD, int64_t rows, int D) {
    const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    float v = 0.f;
    for (int j = lane; j < D; j += 64) v += dout[row * D + j] * out[row * D + j];
    #pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) rowD[row] = v;
}

// ----------------------------------------------------------------- final --
// Merges every pair state (m, l, acc) of a row: with M the largest m,
// out = sum exp(m - M) acc / sum exp(m - M) l.  One thread per (row, 4 dimensions).
__device__ __forceinline__ void final_one(const TP &a, int64_t t, int D4) {
    const int64_t row = div32(t, D4);
    const int j = (int)(t - row * D4);
    const int64_t pslice = a.rows_cap * (a.k + 1);
    float M = -INFINITY;
    for (int l = 0; l <= a.top; ++l) {
        const int np = a.nplev[row * a.lv + l];
        const float2 *ml = a.pml + l * pslice + row * (a.k + 1);
        for (int r = 0; r < np; ++r) M = fmaxf(M, ml[r].x);
    }
    float L = 0.f;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 *base = reinterpret_cast<const float4 *>(a.partial) + row * (a.k + 1) * D4 + j;
    for (int l = 0; l <= a.top; ++l) {
        const int np = a.nplev[row * a.lv + l];
        const float2 *ml = a.pml + l * pslice + row * (a.k + 1);
        const float4 *pa = base + l * pslice * D4;
        // branch-free, so the loads of several pairs are in flight together (a pair
        // without entries has m = -inf and a zero sum: weight 0)
        #pragma unroll 8
        for (int r = 0; r < np; ++r) {
            const float2 s = ml[r];
            // the pair states are read once: nontemporal
            const f32x4 xv = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(pa + r * D4));
            const float4 x = make_float4(xv[0], xv[1], xv[2], xv[3]);
            const float e = s.x == -INFINITY ? 0.f : __expf(s.x - M);
            L += e * s.y;
            v.x += e * x.x; v.y += e * x.y; v.z += e * x.z; v.w += e * x.w;
        }
    }
    const float inv = 1.f / L;
    if (a.rowml != nullptr && j == 0) a.rowml[row] = make_float2(M, L);
    const float o[4] = {v.x * inv, v.y * inv, v.z * inv, v.w * inv};
    if (a.out_bf16)
        Vec<bf16_t, 4>::store(static_cast<bf16_t *>(a.out) + row * a.D + 4 * j, o);
    else
        Vec<float, 4>::store(static_cast<float *>(a.out) + row * a.D + 4 * j, o);
}

__global__ __launch_bounds__(256) void tp_final(TP a) {
    const int D4 = a.D / 4;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.rows * D4;
         t += (int64_t)gridDim.x * blockDim.x)
        final_one(a, t, D4);
}

// ------------------------------------------------------------------ host --
struct Plan {
    int64_t rows;        // rows per pass
    int64_t nb;          // buckets at the widest level
    int32_t zs, lv;
    size_t off_z, off_par0, off_par1, off_mk0, off_mk1, off_pp, off_cnt, off_offs, off_ioff, off_bsum,
        off_sorted, off_items, off_nitems, off_partial, off_pml, off_nplev, total;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

Plan make_plan(int64_t rows, int32_t Hkv, int32_t D, int32_t b, int32_t k, int32_t maxc,
               int64_t capacity, int32_t n_levels) {
    Plan P{};
    P.rows = rows;
    P.nb = (int64_t)Hkv * (capacity / b + 1);
    P.zs = (maxc + 3) / 4 * 4;
    P.lv = n_levels + 1;
    const int64_t pairs = rows * (k + 1);
    const int64_t items = pairs / kTile + P.nb + 1;
    size_t o = 0;
    auto put = [&](size_t bytes) { const size_t at = o; o = up256(o + bytes); return at; };
    P.off_z = put((size_t)rows * P.zs * 4);
    P.off_par0 = put((size_t)rows * k * 4);
    P.off_par1 = put((size_t)rows * k * 4);
    P.off_mk0 = put((size_t)rows * 4);
    P.off_mk1 = put((size_t)rows * 4);
    P.off_pp = put((size_t)pairs * 4);
    P.off_cnt = put((size_t)P.nb * 4);
    P.off_offs = put((size_t)(P.nb + 1) * 4);
    P.off_ioff = put((size_t)(P.nb + 1) * 4);
    P.off_bsum = put((size_t)(P.nb / kScanChunk + 1) * 8);
    P.off_sorted = put((size_t)items * kTile * 16);
    P.off_items = put((size_t)items * 16);
    P.off_nitems = put(16);
    P.off_partial = put((size_t)P.lv * pairs * D * 4);
    P.off_pml = put((size_t)P.lv * pairs * 8);
    P.off_nplev = put((size_t)rows * P.lv * 4);
    P.total = o;
    return P;
}

int64_t pass_rows(int64_t rows, int32_t Hq) {
    const int64_t cap = kRowsPerPass / Hq * Hq;
    return rows < cap ? rows : (cap > 0 ? cap : Hq);
}

size_t select_smem_wave(int32_t zs, int32_t k) {
    return up256((size_t)sel::kScratchBytes + 16 + 2 * (size_t)((k * 4 + 15) & ~15) + (size_t)zs);
}

// Blocks for a persistent launch over `blocks` blocks' worth of items: as many
// as fit on the device at once (at most `blocks`).
hipError_t persistent_grid(const void *kern, size_t smem, unsigned blocks, unsigned &grid) {
    int dev = 0, cus = 0, per = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && smem > 64 * 1024)
        e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, 256, smem);
    if (e != hipSuccess) return e;
    const int64_t fit = (int64_t)std::max(per, 1) * std::max(cus, 1);
    grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(blocks, fit));
    return hipSuccess;
}

template <int KT>
hipError_t launch_select_t(const TP &a, const DebugView &dbg, int l, int smw, hipStream_t s) {
    const size_t smem = (size_t)smw * 4;
    unsigned grid;
    const hipError_t e = persistent_grid((const void *)tp_select<KT>, smem, (unsigned)((a.rows + 3) / 4), grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tp_select<KT>, dim3(grid), dim3(256), smem, s, a, dbg, l, smw);
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

hipError_t launch_count(const TP &a, int l, int32_t NP, hipStream_t s) {
    const int64_t per_head = a.rows / a.Hq * a.G;
    // a block clears and scans the whole histogram, which pays for itself only over
    // enough rows; with few rows and many parents, blocks own ranges of parents instead
    if (NP <= kHistSplit || (NP <= kHistMax && per_head >= kHistRows)) {
        if ((size_t)NP * 4 > 64 * 1024) {
            const hipError_t e =
                hipFuncSetAttribute((const void *)tp_count, hipFuncAttributeMaxDynamicSharedMemorySize, NP * 4);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(tp_count, dim3((unsigned)((per_head + 255) / 256), (unsigned)a.Hkv), dim3(256),
                           (size_t)NP * 4, s, a, l, NP, 0);
    } else {
        hipLaunchKernelGGL(tp_count, dim3((unsigned)((NP + kRange - 1) / kRange), (unsigned)a.Hkv),
                           dim3(1024), (size_t)kRange * 4, s, a, l, NP, 1);
    }
    return hipGetLastError();
}

// The pairs of level l grouped by (KV head, parent) into items of up to 16.
hipError_t bucket_level(const TP &a, const DebugView &dbg, int l, int32_t NP, hipStream_t s) {
    const int64_t nb = (int64_t)a.Hkv * NP;
    const int64_t nchunks = (nb + kScanChunk - 1) / kScanChunk;
    hipError_t e;
    if ((e = launch_count(a, l, NP, s)) != hipSuccess) return e;
    if (nb <= kScanSmall) {
        hipLaunchKernelGGL(tp_scan_small, dim3(1), dim3(256), 0, s, a, nb);
    } else {
        hipLaunchKernelGGL(tp_scan_sums, dim3((unsigned)nchunks), dim3(256), 0, s, a, nb);
        hipLaunchKernelGGL(tp_scan_chunks, dim3(1), dim3(256), 0, s, a, nb, nchunks);
        hipLaunchKernelGGL(tp_scan_write, dim3((unsigned)nchunks), dim3(256), 0, s, a, nb);
    }
    hipLaunchKernelGGL(tp_scatter, dim3((unsigned)((a.rows + nb + 255) / 256)), dim3(256), 0, s, a, dbg, l, NP,
                       nb);
    return hipGetLastError();
}

template <int D, int KC>
hipError_t run_pass(const TreeView &tv, TP a, const DebugView &dbg, int64_t max_ctx, const Plan &P,
                    int32_t maxc, hipStream_t s) {
    const int64_t rows = a.rows;
    {
        const int64_t n = std::max<int64_t>(std::max<int64_t>(rows, P.nb), rows * a.n_levels * a.k);
        const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
        hipLaunchKernelGGL(tp_init, dim3((unsigned)blocks), dim3(256), 0, s, a, dbg, P.nb);
    }
    const int smw = (int)select_smem_wave(a.zs, a.k);
    hipError_t e;
    for (int l = a.top; l >= 0; --l) {
        const int32_t NP = (int32_t)(max_ctx / a.pw[l + 1] + 1);
        const int64_t nb = (int64_t)a.Hkv * NP;
        if ((e = bucket_level(a, dbg, l, NP, s)) != hipSuccess) return e;
        const int64_t pairs = rows * (int64_t)std::min(a.k + 1, (int)NP);
        const int64_t items = pairs / kTile + nb + 1;
        const unsigned ib = (unsigned)((items + 3) / 4);
        const size_t crot_bytes = (size_t)a.b * crot_stride(D) * sizeof(float2);
        if (l == 0) {
            const size_t sm = crot_bytes + (size_t)4 * kTile * (32 * KC + 1) * sizeof(float);
            unsigned grid;
            if ((e = persistent_grid((const void *)tp_attend<D, KC>, sm, ib, grid)) != hipSuccess) return e;
            hipLaunchKernelGGL((tp_attend<D, KC>), dim3(grid), dim3(256), sm, s, tv, a, NP);
        } else {
            unsigned grid;
            if constexpr (KC <= 2) {
                constexpr int kR = 4;
                const unsigned rb = (unsigned)((items / kR + 1 + 3) / 4);
                if ((e = persistent_grid((const void *)tp_score_runs<D, KC, kR>, crot_bytes, rb, grid)) !=
                    hipSuccess)
                    return e;
                hipLaunchKernelGGL((tp_score_runs<D, KC, kR>), dim3(grid), dim3(256), crot_bytes, s, tv, a, l, NP);
            } else {
                if ((e = persistent_grid((const void *)tp_score<D, KC>, crot_bytes, ib, grid)) != hipSuccess)
                    return e;
                hipLaunchKernelGGL((tp_score<D, KC>), dim3(grid), dim3(256), crot_bytes, s, tv, a, l, NP);
            }
            if ((e = launch_select(a, dbg, l, maxc, smw, s)) != hipSuccess) return e;
            if constexpr (KC == 1) {
                if (rows >= kLongRunRows) {
                    const unsigned rb = (unsigned)((items / 8 + 1 + 3) / 4);
                    if ((e = persistent_grid((const void *)tp_pv_runs<D, 1, 8>, 0, rb, grid)) != hipSuccess) return e;
                    hipLaunchKernelGGL((tp_pv_runs<D, 1, 8>), dim3(grid), dim3(256), 0, s, tv, a, l, NP);
                } else {
                    const unsigned rb = (unsigned)((items / 4 + 1 + 3) / 4);
                    if ((e = persistent_grid((const void *)tp_pv_runs<D, 1, 4>, 0, rb, grid)) != hipSuccess) return e;
                    hipLaunchKernelGGL((tp_pv_runs<D, 1, 4>), dim3(grid), dim3(256), 0, s, tv, a, l, NP);
                }
            } else if constexpr (KC == 2) {
                // two chunks of children per item: runs of 2 items keep 2 waves per SIMD
                const unsigned rb = (unsigned)((items / 2 + 1 + 3) / 4);
                if ((e = persistent_grid((const void *)tp_pv_runs<D, 2, 2>, 0, rb, grid)) != hipSuccess) return e;
                hipLaunchKernelGGL((tp_pv_runs<D, 2, 2>), dim3(grid), dim3(256), 0, s, tv, a, l, NP);
            } else {
                if ((e = persistent_grid((const void *)tp_pv<D, KC>, 0, ib, grid)) != hipSuccess) return e;
                hipLaunchKernelGGL((tp_pv<D, KC>), dim3(grid), dim3(256), 0, s, tv, a, l, NP);
            }
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        unsigned grid;
        if ((e = persistent_grid((const void *)tp_final, 0, (unsigned)((rows * (D / 4) + 255) / 256), grid)) !=
            hipSuccess)
            return e;
        hipLaunchKernelGGL(tp_final, dim3(grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

size_t tiled_backward_lds_bytes(int32_t D, int32_t b) {
    return (size_t)b * crot_stride(D) * sizeof(float2) +
           4 * (D == 128 ? tb_wave_lds<128>() : tb_wave_lds<64>());
}

namespace {

// Backward of one pass of rows: the forward (recording the selections and each row's
// softmax statistics), <dO, out>, then per level from the top the same buckets and
// tb_item.  With `tree` (one pass of rows) the tree pass runs between the levels: after
// level l's items it writes level l - 1's gradients (the tokens' at l = 1), which
// level l - 1's items then add to, so no gradient is read back and only the top level
// and the children past each level's last complete node need clearing.
template <int D, int KC>
hipError_t run_backward_pass(const TreeView &tv, TP a, TB t, float *out, float *kth_gap, int64_t max_ctx,
                             const Plan &P, int32_t maxc, bool tree, hipStream_t s) {
    hipError_t e;
    t.dq_slots = a.rows >= kLongRunRows ? 1 : 0;
    {
        DebugView fd{};
        fd.selected = const_cast<int32_t *>(t.sel);
        fd.kth_gap = kth_gap;
        a.out = out;
        a.out_bf16 = 0;
        if ((e = run_pass<D, KC>(tv, a, fd, max_ctx, P, maxc, s)) != hipSuccess) return e;
        hipLaunchKernelGGL(tb_rowdot, dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0, s, t.dout, out,
                           const_cast<float *>(t.rowD), a.rows, D);
    }
    // bf16 token gradients (staged): level 0's items run before the tree pass at level 1
    // and leave their sums in the staging buffer, which that pass adds as it writes each
    // token row once; tokens past the last complete level-1 node get theirs from
    // tb_stage_tail.  Needs one pass of rows (the tree pass interleaved).
    const bool staged = tree && t.tree.dk16 != nullptr;
    if (staged && t.stage_k == nullptr) return hipErrorInvalidValue;
    if (tree && a.top >= 1) {
        const int64_t ntop = a.length / a.pw[a.top];
        if ((e = launch_zero_rows(t.gk[a.top], a.Hkv, t.node_cap[a.top], 0, ntop, D, s)) != hipSuccess) return e;
        if ((e = launch_zero_rows(t.gv[a.top], a.Hkv, t.node_cap[a.top], 0, ntop, D, s)) != hipSuccess) return e;
    } else if (tree && t.dk != nullptr) {
        // no level above the tokens (fewer than b tokens): no tree pass writes them
        if ((e = launch_zero_rows(t.dk, a.Hkv, t.cap, 0, a.length, D, s)) != hipSuccess) return e;
        if ((e = launch_zero_rows(t.dv, a.Hkv, t.cap, 0, a.length, D, s)) != hipSuccess) return e;
    }
    const DebugView none{};
    const size_t lds = tiled_backward_lds_bytes(D, a.b);
    TB t0 = t;                              // level 0's items: to the staging buffer when staged
    if (staged) {
        t0.dk = nullptr;
        t0.dv = nullptr;
    } else {
        t0.stage_k = nullptr;
        t0.stage_v = nullptr;
    }
    auto items = [&](int l) -> hipError_t {
        const int32_t NP = (int32_t)(max_ctx / a.pw[l + 1] + 1);
        const int64_t nb = (int64_t)a.Hkv * NP;
        hipLaunchKernelGGL(tb_parents, dim3((unsigned)((a.rows + 255) / 256)), dim3(256), 0, s, a, t.sel, l);
        hipError_t r;
        if ((r = bucket_level(a, none, l, NP, s)) != hipSuccess) return r;
        const int64_t pairs = a.rows * (int64_t)std::min(a.k + 1, (int)NP);
        const int64_t n_items = pairs / kTile + nb + 1;
        unsigned grid;
        const bool st = staged && l == 0;
        const void *fn = st ? (const void *)tb_item<D, KC, true> : (const void *)tb_item<D, KC, false>;
        if ((r = persistent_grid(fn, lds, (unsigned)((n_items + 3) / 4), grid)) != hipSuccess) return r;
        if (st)
            hipLaunchKernelGGL((tb_item<D, KC, true>), dim3(grid), dim3(256), lds, s, tv, a, t0, l, NP);
        else
            hipLaunchKernelGGL((tb_item<D, KC, false>), dim3(grid), dim3(256), lds, s, tv, a, l == 0 ? t0 : t, l, NP);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        if (t.dq_slots) {
            unsigned dg;
            if ((r = persistent_grid((const void *)tb_dq_add, 0, (unsigned)((a.rows * (D / 4) + 255) / 256), dg)) !=
                hipSuccess)
                return r;
            hipLaunchKernelGGL(tb_dq_add, dim3(dg), dim3(256), 0, s, a, t.dq, l);
        }
        return hipSuccess;
    };
    // the staged tokens past the last complete level-1 node (all tokens when there is no
    // level above them): the items of their bucket (head g, parent length / b) summed
    auto stage_tail = [&]() -> hipError_t {
        const int64_t n1 = a.length / a.b;
        if (n1 * a.b >= a.length) return hipSuccess;
        const int32_t NP0 = (int32_t)(max_ctx / a.pw[1] + 1);
        hipLaunchKernelGGL(tb_stage_tail, dim3((unsigned)a.Hkv), dim3(256), 0, s, a.itemoff, t.stage_k,
                           t.stage_v, t.tree.dk16, t.tree.dv16, t.cap, a.b, D, NP0, n1, a.length);
        return hipGetLastError();
    };
    for (int l = a.top; l >= 0; --l) {
        if (staged && l == 0 && a.top >= 1) break;   // level 0 ran before the tree pass at 1
        if ((e = items(l)) != hipSuccess) return e;
        if (staged && l == 0) {
            if ((e = stage_tail()) != hipSuccess) return e;
        }
        if (tree && l >= 1) {
            BwdTreeArgs tt = t.tree;
            tt.level = l;
            tt.nodes = a.length / a.pw[l];
            tt.gk = t.gk[l];
            tt.gv = t.gv[l];
            tt.gk_child = l >= 2 ? t.gk[l - 1] : nullptr;
            tt.gv_child = l >= 2 ? t.gv[l - 1] : nullptr;
            tt.dk = t.dk;
            tt.dv = t.dv;
            tt.write_children = 1;
            if (staged && l == 1) {
                if ((e = items(0)) != hipSuccess) return e;
                tt.stage_k = t.stage_k;
                tt.stage_v = t.stage_v;
                tt.stage_item = a.itemoff;
                tt.stage_np = (int32_t)(max_ctx / a.pw[1] + 1);
            } else {
                tt.dk16 = nullptr;
                tt.dv16 = nullptr;
            }
            if ((e = launch_backward_tree(tv, RECSA_BF16, D, tt, s)) != hipSuccess) return e;
            // children past the last complete node of level l have no parent to write them
            const int64_t under = tt.nodes * a.b;
            if (l >= 2) {
                const int64_t nc = a.length / a.pw[l - 1];
                if ((e = launch_zero_rows(t.gk[l - 1], a.Hkv, t.node_cap[l - 1], under, nc, D, s)) != hipSuccess)
                    return e;
                if ((e = launch_zero_rows(t.gv[l - 1], a.Hkv, t.node_cap[l - 1], under, nc, D, s)) != hipSuccess)
                    return e;
            } else if (staged) {
                if ((e = stage_tail()) != hipSuccess) return e;
            } else if (t.dk != nullptr) {
                if ((e = launch_zero_rows(t.dk, a.Hkv, t.cap, under, a.length, D, s)) != hipSuccess) return e;
                if ((e = launch_zero_rows(t.dv, a.Hkv, t.cap, under, a.length, D, s)) != hipSuccess) return e;
            }
        }
    }
    return hipSuccess;
}

template <int D>
hipError_t run_backward_pass_d(const TreeView &tv, const TP &a, const TB &t, float *out, float *kth_gap,
                               int64_t max_ctx, const Plan &P, int32_t maxc, bool tree, hipStream_t s) {
    switch ((a.b + 31) / 32) {
        case 1: return run_backward_pass<D, 1>(tv, a, t, out, kth_gap, max_ctx, P, maxc, tree, s);
        case 2: return run_backward_pass<D, 2>(tv, a, t, out, kth_gap, max_ctx, P, maxc, tree, s);
        case 3: return run_backward_pass<D, 3>(tv, a, t, out, kth_gap, max_ctx, P, maxc, tree, s);
        default: return run_backward_pass<D, 4>(tv, a, t, out, kth_gap, max_ctx, P, maxc, tree, s);
    }
}

template <int D>
hipError_t run_pass_d(const TreeView &tv, const TP &a, const DebugView &dbg, int64_t max_ctx,
                      const Plan &P, int32_t maxc, hipStream_t s) {
    switch ((a.b + 31) / 32) {
        case 1: return run_pass<D, 1>(tv, a, dbg, max_ctx, P, maxc, s);
        case 2: return run_pass<D, 2>(tv, a, dbg, max_ctx, P, maxc, s);
        case 3: return run_pass<D, 3>(tv, a, dbg, max_ctx, P, maxc, s);
        default: return run_pass<D, 4>(tv, a, dbg, max_ctx, P, maxc, s);
    }
}

}  // namespace

size_t tiled_workspace_bytes(int64_t rows, int32_t Hq, int32_t Hkv, int32_t D, int32_t b, int32_t k,
                             int32_t maxc, int64_t capacity, int32_t n_levels) {
    return make_plan(pass_rows(rows, Hq), Hkv, D, b, k, maxc, capacity, n_levels).total;
}

int32_t tiled_max_fanout() { return kMaxFanout; }

size_t tiled_select_lds_bytes(int32_t maxc, int32_t k) {
    return 4 * select_smem_wave((maxc + 3) / 4 * 4, k);
}

namespace {

TP make_tp(const TreeView &tv, int32_t D, const DescendArgs &da, int32_t Hkv, int64_t length, const Plan &P,
           void *ws) {
    unsigned char *w = static_cast<unsigned char *>(ws);
    TP a{};
    a.Hq = da.Hq;
    a.G = da.G;
    a.Hkv = Hkv;
    a.D = D;
    a.rows_cap = P.rows;
    a.ctx_step = da.ctx_step;
    a.b = da.b;
    a.k = da.k;
    a.zs = P.zs;
    a.lv = P.lv;
    a.scale = da.scale;
    a.out_bf16 = da.out_bf16;
    a.n_levels = tv.n_levels;
    a.length = length;
    a.z = reinterpret_cast<float *>(w + P.off_z);
    a.par[0] = reinterpret_cast<int32_t *>(w + P.off_par0);
    a.par[1] = reinterpret_cast<int32_t *>(w + P.off_par1);
    a.mk[0] = reinterpret_cast<int32_t *>(w + P.off_mk0);
    a.mk[1] = reinterpret_cast<int32_t *>(w + P.off_mk1);
    a.pairpos = reinterpret_cast<int32_t *>(w + P.off_pp);
    a.counts = reinterpret_cast<int32_t *>(w + P.off_cnt);
    a.offs = reinterpret_cast<int32_t *>(w + P.off_offs);
    a.itemoff = reinterpret_cast<int32_t *>(w + P.off_ioff);
    a.bsum = reinterpret_cast<int2 *>(w + P.off_bsum);
    a.sorted = reinterpret_cast<int4 *>(w + P.off_sorted);
    a.items = reinterpret_cast<int4 *>(w + P.off_items);
    a.n_items = reinterpret_cast<int32_t *>(w + P.off_nitems);
    a.partial = reinterpret_cast<float *>(w + P.off_partial);
    a.pml = reinterpret_cast<float2 *>(w + P.off_pml);
    a.nplev = reinterpret_cast<int32_t *>(w + P.off_nplev);
    return a;
}

// The pass's first row r0 onwards: queries, context lengths and the level powers.
int64_t set_pass(TP &a, const DescendArgs &da, int64_t r0, int64_t rows, int32_t D) {
    const int64_t q0 = r0 / da.Hq;
    a.rows = rows;
    a.q = reinterpret_cast<const bf16_t *>(static_cast<const unsigned char *>(da.q) + r0 * D * 2);
    a.ctx_base = da.ctx_base + q0 * da.ctx_step;
    const int64_t max_ctx = a.ctx_base + (rows / da.Hq - 1) * da.ctx_step;
    a.top = 0;
    a.pw[0] = 1;
    for (int l = 1; l < kMaxLevels + 2; ++l) {
        a.pw[l] = a.pw[l - 1] <= max_ctx ? a.pw[l - 1] * da.b : a.pw[l - 1];
        if (a.pw[l] <= max_ctx && a.pw[l] > a.pw[l - 1]) a.top = l;
    }
    return max_ctx;
}

// The backward's own buffers after the forward's plan: out [rows][D] fp32, the
// selections [rows][n_levels][k], (max, sum) and <dO, out> per row.
struct BwdPlan {
    size_t off_out, off_sel, off_ml, off_rowD, off_stk, off_stv, total;
};

// Items of level 0 (the staging buffer's rows of b children): at most one per 16 pairs
// plus one per non-empty bucket, and there are at most rows * (k + 1) pairs and
// Hkv * (capacity / b + 1) buckets.
int64_t stage_items(int64_t rows, int32_t k, int32_t Hkv, int32_t b, int64_t capacity) {
    const int64_t pairs = rows * (k + 1);
    const int64_t nb = (int64_t)Hkv * (capacity / b + 1);
    return (pairs + kTile - 1) / kTile + std::min(pairs, nb);
}

// stage: bf16 token gradients, with the staging buffers [items][b][D] fp32 for k and v
BwdPlan make_bwd_plan(const Plan &P, int32_t D, int32_t k, int32_t n_levels, bool stage, int32_t Hkv,
                      int32_t b, int64_t capacity) {
    BwdPlan B{};
    size_t o = P.total;
    auto put = [&](size_t bytes) { const size_t at = o; o = up256(o + bytes); return at; };
    B.off_out = put((size_t)P.rows * D * 4);
    B.off_sel = put((size_t)P.rows * (n_levels > 0 ? n_levels : 1) * k * 4);
    B.off_ml = put((size_t)P.rows * 8);
    B.off_rowD = put((size_t)P.rows * 4);
    if (stage) {
        const size_t bytes = (size_t)stage_items(P.rows, k, Hkv, b, capacity) * b * D * 4;
        B.off_stk = put(bytes);
        B.off_stv = put(bytes);
    }
    B.total = o;
    return B;
}

}  // namespace

size_t tiled_backward_workspace_bytes(int64_t rows, int32_t Hq, int32_t Hkv, int32_t D, int32_t b, int32_t k,
                                      int32_t maxc, int64_t capacity, int32_t n_levels, bool bf16_grads) {
    const Plan P = make_plan(pass_rows(rows, Hq), Hkv, D, b, k, maxc, capacity, n_levels);
    return make_bwd_plan(P, D, k, n_levels, bf16_grads, Hkv, b, capacity).total;
}

bool tiled_backward_one_pass(int64_t rows, int32_t Hq) { return pass_rows(rows, Hq) >= rows; }

hipError_t launch_backward_tiled(const TreeView &tv, int32_t D, const DescendArgs &da, int32_t Hkv,
                                 int64_t length, int64_t capacity, const BwdArgs &ba, int32_t *dbg_selected,
                                 float *dbg_kth_gap, const BwdTreeArgs *tree, void *ws, hipStream_t s) {
    const int64_t per = pass_rows(da.rows, da.Hq);
    if (tree != nullptr && per < da.rows) return hipErrorInvalidValue;   // interleaving needs one pass
    const Plan P = make_plan(per, Hkv, D, da.b, da.k, da.max_cand, capacity, tv.n_levels);
    const bool staged = tree != nullptr && tree->dk16 != nullptr;
    const BwdPlan B = make_bwd_plan(P, D, da.k, tv.n_levels, staged, Hkv, da.b, capacity);
    unsigned char *w = static_cast<unsigned char *>(ws);
    TP a = make_tp(tv, D, da, Hkv, length, P, ws);
    a.rowml = reinterpret_cast<float2 *>(w + B.off_ml);
    float *out = reinterpret_cast<float *>(w + B.off_out);
    TB t{};
    t.dk = ba.dk;
    t.dv = ba.dv;
    for (int l = 0; l <= kMaxLevels; ++l) {
        t.gk[l] = ba.gk[l];
        t.gv[l] = ba.gv[l];
        t.node_cap[l] = tv.node_cap[l];
    }
    t.cap = tv.cap;
    if (tree != nullptr) t.tree = *tree;
    t.rowml = a.rowml;
    t.rowD = reinterpret_cast<const float *>(w + B.off_rowD);
    t.sel = reinterpret_cast<const int32_t *>(w + B.off_sel);
    if (staged) {
        t.stage_k = reinterpret_cast<float *>(w + B.off_stk);
        t.stage_v = reinterpret_cast<float *>(w + B.off_stv);
    }
    for (int64_t r0 = 0; r0 < da.rows; r0 += per) {
        const int64_t rows = std::min(per, da.rows - r0);
        const int64_t max_ctx = set_pass(a, da, r0, rows, D);
        t.dout = ba.dout + r0 * D;
        t.dq = ba.dq + r0 * D;
        float *kth = dbg_kth_gap != nullptr ? dbg_kth_gap + r0 * tv.n_levels : nullptr;
        const bool il = tree != nullptr;
        const hipError_t e = D == 128 ? run_backward_pass_d<128>(tv, a, t, out, kth, max_ctx, P, da.max_cand, il, s)
                                      : run_backward_pass_d<64>(tv, a, t, out, kth, max_ctx, P, da.max_cand, il, s);
        if (e != hipSuccess) return e;
        if (dbg_selected != nullptr && tv.n_levels > 0) {
            const hipError_t c = hipMemcpyAsync(dbg_selected + r0 * tv.n_levels * da.k, t.sel,
                                                (size_t)rows * tv.n_levels * da.k * 4, hipMemcpyDeviceToDevice, s);
            if (c != hipSuccess) return c;
        }
    }
    return hipSuccess;
}

hipError_t launch_prefill_tiled(const TreeView &tv, int32_t D, const DescendArgs &da, int32_t Hkv,
                                int64_t length, int64_t capacity, const DebugView &dbg, void *ws,
                                hipStream_t s) {
    const int64_t per = pass_rows(da.rows, da.Hq);
    const Plan P = make_plan(per, Hkv, D, da.b, da.k, da.max_cand, capacity, tv.n_levels);
    TP a = make_tp(tv, D, da, Hkv, length, P, ws);
    const size_t esz_o = da.out_bf16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < da.rows; r0 += per) {
        const int64_t rows = std::min(per, da.rows - r0);
        const int64_t max_ctx = set_pass(a, da, r0, rows, D);
        a.out = static_cast<unsigned char *>(da.out) + r0 * D * esz_o;
        DebugView d = dbg;
        if (d.selected) d.selected += r0 * tv.n_levels * da.k;
        if (d.kth_gap) d.kth_gap += r0 * tv.n_levels;
        if (d.n_keys) d.n_keys += r0;
        const hipError_t e = D == 128 ? run_pass_d<128>(tv, a, d, max_ctx, P, da.max_cand, s)
                                      : run_pass_d<64>(tv, a, d, max_ctx, P, da.max_cand, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace recsa
