// Internal definitions shared by the RecSA host library and its gfx950 kernels.
#pragma once
#include <stddef.h>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "recsa.h"

namespace recsa {

constexpr int kMaxLevels = 32;     // b >= 2 and capacity < 2^31 give at most 31 levels

using bf16_t = uint16_t;           // bf16 bit pattern

// Everything a kernel needs to find the cache, the tree and the RoPE table.
struct TreeView {
    const void *k_cache;
    const void *v_cache;
    int64_t cap;                        // token capacity (row stride of a head)
    void *key[kMaxLevels + 1];          // key[l]: [Hkv][node_cap[l]][D] store type (l >= 1)
    void *val[kMaxLevels + 1];          // val[l]: same, subtree means in store type
    float *mean[kMaxLevels + 1];        // fp32 subtree means (bf16 storage only; else null)
    int64_t node_cap[kMaxLevels + 1];
    const float2 *rope;                 // [rope_rows][D/2] (cos, sin) of pos * theta_j
    int32_t rope_rows;
    int32_t n_levels;
};

struct DebugView {
    int32_t *selected;   // [rows][n_levels][k]
    float *kth_gap;      // [rows][n_levels]
    int32_t *n_keys;     // [rows]
};

// Index of the calling wave in its workgroup, as a scalar: the compiler does not treat
// threadIdx.x / 64 as wave-uniform by itself, and branches and addresses built from
// it would otherwise run on the vector unit under exec masks.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---- storage conversions ---------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);            // round to nearest, ties to even (finite inputs)
    return u >> 16;
}

// Load N consecutive elements of type T starting at p (N*sizeof(T) in {4, 8, 16, 32}
// bytes, naturally aligned) and widen them to fp32.
template <typename T, int N> struct Vec;

template <int N> struct Vec<float, N> {
    __device__ __forceinline__ static void load(const float *p, float *out) {
        if constexpr (N == 1) {
            out[0] = p[0];
        } else if constexpr (N == 2) {
            float2 v = *reinterpret_cast<const float2 *>(p);
            out[0] = v.x; out[1] = v.y;
        } else {
            #pragma unroll
            for (int i = 0; i < N; i += 4) {
                float4 v = *reinterpret_cast<const float4 *>(p + i);
                out[i] = v.x; out[i + 1] = v.y; out[i + 2] = v.z; out[i + 3] = v.w;
            }
        }
    }
    __device__ __forceinline__ static void store(float *p, const float *in) {
        if constexpr (N == 1) {
            p[0] = in[0];
        } else if constexpr (N == 2) {
            *reinterpret_cast<float2 *>(p) = make_float2(in[0], in[1]);
        } else {
            #pragma unroll
            for (int i = 0; i < N; i += 4)
                *reinterpret_cast<float4 *>(p + i) = make_float4(in[i], in[i + 1], in[i + 2], in[i + 3]);
        }
    }
};

template <int N> struct Vec<bf16_t, N> {
    __device__ __forceinline__ static void load(const bf16_t *p, float *out) {
        if constexpr (N == 2) {
            uint32_t v = *reinterpret_cast<const uint32_t *>(p);
            out[0] = bf16_to_f32(v & 0xFFFFu); out[1] = bf16_to_f32(v >> 16);
        } else if constexpr (N == 4) {
            uint2 v = *reinterpret_cast<const uint2 *>(p);
            out[0] = bf16_to_f32(v.x & 0xFFFFu); out[1] = bf16_to_f32(v.x >> 16);
            out[2] = bf16_to_f32(v.y & 0xFFFFu); out[3] = bf16_to_f32(v.y >> 16);
        } else {
            static_assert(N % 8 == 0, "bf16 vector width");
            #pragma unroll
            for (int i = 0; i < N; i += 8) {
                uint4 v = *reinterpret_cast<const uint4 *>(p + i);
                out[i + 0] = bf16_to_f32(v.x & 0xFFFFu); out[i + 1] = bf16_to_f32(v.x >> 16);
                out[i + 2] = bf16_to_f32(v.y & 0xFFFFu); out[i + 3] = bf16_to_f32(v.y >> 16);
                out[i + 4] = bf16_to_f32(v.z & 0xFFFFu); out[i + 5] = bf16_to_f32(v.z >> 16);
                out[i + 6] = bf16_to_f32(v.w & 0xFFFFu); out[i + 7] = bf16_to_f32(v.w >> 16);
            }
        }
    }
    __device__ __forceinline__ static void store(bf16_t *p, const float *in) {
        if constexpr (N == 2) {
            *reinterpret_cast<uint32_t *>(p) = f32_to_bf16(in[0]) | (f32_to_bf16(in[1]) << 16);
        } else if constexpr (N == 4) {
            *reinterpret_cast<uint2 *>(p) = make_uint2(f32_to_bf16(in[0]) | (f32_to_bf16(in[1]) << 16),
                                                       f32_to_bf16(in[2]) | (f32_to_bf16(in[3]) << 16));
        } else {
            static_assert(N % 8 == 0, "bf16 vector width");
            #pragma unroll
            for (int i = 0; i < N; i += 8)
                *reinterpret_cast<uint4 *>(p + i) =
                    make_uint4(f32_to_bf16(in[i + 0]) | (f32_to_bf16(in[i + 1]) << 16),
                               f32_to_bf16(in[i + 2]) | (f32_to_bf16(in[i + 3]) << 16),
                               f32_to_bf16(in[i + 4]) | (f32_to_bf16(in[i + 5]) << 16),
                               f32_to_bf16(in[i + 6]) | (f32_to_bf16(in[i + 7]) << 16));
        }
    }
};

// ---- launchers (defined in the kernel translation units) --------------------
hipError_t launch_rope_table(float2 *table, int32_t rows, int32_t D, double base, hipStream_t s);

hipError_t launch_scatter(const TreeView &tv, recsa_dtype st, int32_t Hkv, int32_t D,
                          const void *k_new, const void *v_new, int64_t at, int64_t n,
                          hipStream_t s);

// Summarize level-`level` nodes [n0, n1) of every KV head from level level-1.
hipError_t launch_level(const TreeView &tv, recsa_dtype st, int32_t Hkv, int32_t D, int32_t b,
                        int32_t level, int64_t n0, int64_t n1, const float *pool_w,
                        float pool_scale, bool keys_only, hipStream_t s);

constexpr int kInlineSeqs = 32;    // sequences whose table travels in the kernel arguments

// One sequence of a multi-sequence decode: its cache, its tree (same layout as the
// others'), its pooler vectors (unused by the descent) and its length.  The layout is
// recsa_tree_desc's, so a caller's descriptor array is copied to the device as it is.
struct SeqEntry {
    const void *k_cache;
    const void *v_cache;
    const void *tree;
    const float *pool_w;
    int64_t length;
};
static_assert(sizeof(SeqEntry) == sizeof(recsa_tree_desc), "SeqEntry mirrors recsa_tree_desc");
static_assert(offsetof(SeqEntry, tree) == offsetof(recsa_tree_desc, tree), "SeqEntry mirrors recsa_tree_desc");
static_assert(offsetof(SeqEntry, length) == offsetof(recsa_tree_desc, length), "SeqEntry mirrors recsa_tree_desc");

struct DescendArgs {
    const void *q;             // [rows / Hq][Hq][D]
    void *out;                 // same shape, out dtype
    int64_t rows;              // queries * Hq
    int32_t Hq, G;             // query heads, query heads per KV head
    int32_t gs;                // query heads per row: 1, or G when a group shares its selection
    int64_t ctx_base;          // n_ctx of query 0
    int32_t ctx_step;          // n_ctx of query i = ctx_base + i * ctx_step
    int32_t b, k;
    int32_t max_cand;          // largest candidate count of any level
    float scale;
    int32_t out_bf16;
    // multi-sequence decode: query i reads sequence i, at n_ctx = its length; the
    // TreeView describes sequence 0 and the others are found by byte offsets from it.
    // The table is inline for up to kInlineSeqs sequences, else in device memory.
    const SeqEntry *seqs;
    int32_t n_inline;
    SeqEntry seq_inline[kInlineSeqs];
};

hipError_t launch_descend(const TreeView &tv, recsa_dtype st, int32_t D, const DescendArgs &a,
                          const DebugView &dbg, hipStream_t s);

// ---- backward (selection held fixed) -------------------------------------------
struct BwdArgs {
    const void *q;             // [rows / Hq][Hq][D] store type
    const float *dout;         // same shape, fp32
    float *dq;                 // same shape, fp32 (written)
    float *dk, *dv;            // [Hkv][cap][D] fp32 token gradients (added to)
    int32_t phase;             // 0: every entry; 1: summaries and dq only; 2: token entries only (no dq)
    float *gk[kMaxLevels + 1]; // gk[l], gv[l]: [Hkv][node_cap[l]][D] fp32 summary gradients (l >= 1)
    float *gv[kMaxLevels + 1];
    int64_t rows;              // queries * Hq
    int32_t Hq, G;
    int64_t ctx_base;          // n_ctx of query 0
    int32_t ctx_step;          // n_ctx of query i = ctx_base + i * ctx_step
    int32_t b, k;
    int32_t max_cand;
    float scale;
};

struct BwdTreeArgs {
    int32_t level;             // the nodes' level (>= 1); children are level - 1
    int32_t Hkv;
    int64_t nodes;             // complete nodes of that level
    int32_t b;
    float pool_scale;
    const float *pool_w;       // [Hkv][D]
    const float *gk, *gv;      // the level's gradients
    float *gk_child, *gv_child;  // level - 1's (level >= 2)
    float *dk, *dv;            // token gradients (level 1)
    int32_t write_children;    // write the children's gradients (tokens' dk, dv at level 1), not add
                               // to them; children of nodes without gradient get zeros
    float *dw;                 // [Hkv][D] (added to)
    int32_t cache_keys;        // set by the launch: the children's keys stay in LDS between passes
    // bf16 token gradients (level 1, fanout <= 32; instead of dk, dv): each token row is
    // written once, its tree part plus the rows' own entries, which level 0's items left
    // as per-item sums in fp32 (stage_k, stage_v [items][b][D]; the items of the bucket
    // (head g, level-1 node j) are stage_item[g * stage_np + j] .. [.. + 1] - 1)
    bf16_t *dk16, *dv16;
    const float *stage_k, *stage_v;
    const int32_t *stage_item;
    int32_t stage_np;
};

// ---- dense attention (the distillation teacher) ---------------------------------
struct DenseArgs {
    const void *q;             // [B][Hq][D] store type, at position `length`
    void *out;                 // [B][Hq][D] out type
    int32_t out_bf16;
    float *part;               // [Hkv][nspan][B * G][D + 2] per-span (acc, max, sum)
    const void *k_cache, *v_cache;
    int64_t cap;
    int32_t B, Hq, Hkv, G;
    int64_t length;
    int64_t span;              // tokens per span
    int32_t nspan;
    double base;
    float scale;
    float2 *incr;              // bf16 storage: [64][D/2] (cos, sin) of tt * theta_j, filled by the launch
};
// spans of dense attention: at most kDenseMaxSpans over any length (the workspace bound)
constexpr int64_t kDenseMaxSpans = 256;
int64_t dense_span(int64_t length);
hipError_t launch_dense(recsa_dtype st, int32_t D, const DenseArgs &a, hipStream_t s);

hipError_t launch_distill_loss(const float *out, const float *teacher, float *dout, float *loss,
                               int64_t n, int64_t rows, hipStream_t s);
hipError_t launch_distill_update(float *w, float *vel, const float *dw, int64_t n, float lr, float mu,
                                 hipStream_t s);

size_t backward_rows_lds_bytes(int32_t maxc, int32_t k, int32_t nlev, int32_t D);
// parent-major backward (bf16 storage, many rows): the forward again, then per level
// the pairs bucketed by parent and one item kernel; summary gradients to ba.gk / ba.gv
// LDS of the parent-major backward's item kernel (per workgroup of four waves).
size_t tiled_backward_lds_bytes(int32_t D, int32_t b);
// bf16_grads: with the staging buffers of bf16 token gradients (tree->dk16 set)
size_t tiled_backward_workspace_bytes(int64_t rows, int32_t Hq, int32_t Hkv, int32_t D, int32_t b, int32_t k,
                                      int32_t maxc, int64_t capacity, int32_t n_levels, bool bf16_grads);
// tree == NULL: every level's items in each pass of rows (the caller clears the
// gradients and runs the tree pass after); else (one pass of rows only) the tree pass
// runs between the levels with these common arguments, writing each level's children's
// gradients before that level's items add to them: nothing to clear or run after
bool tiled_backward_one_pass(int64_t rows, int32_t Hq);
hipError_t launch_backward_tiled(const TreeView &tv, int32_t D, const DescendArgs &da, int32_t Hkv,
                                 int64_t length, int64_t capacity, const BwdArgs &ba, int32_t *dbg_selected,
                                 float *dbg_kth_gap, const BwdTreeArgs *tree, void *ws, hipStream_t s);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
// zeros rows [r0, r1) of each of Hkv heads of a [Hkv][cap][D] fp32 array
hipError_t launch_zero_rows(float *p, int32_t Hkv, int64_t cap, int64_t r0, int64_t r1, int32_t D, hipStream_t s);
hipError_t launch_backward_rows(const TreeView &tv, recsa_dtype st, int32_t D, const BwdArgs &a,
                                const DebugView &dbg, hipStream_t s);
hipError_t launch_backward_tree(const TreeView &tv, recsa_dtype st, int32_t D, const BwdTreeArgs &t,
                                hipStream_t s);
// a.gs > 1: one selection per (query, KV group), by storage type
hipError_t launch_descend_grouped_bf16(const TreeView &tv, int32_t D, const DescendArgs &a,
                                       const DebugView &dbg, hipStream_t s);
hipError_t launch_descend_grouped_f32(const TreeView &tv, int32_t D, const DescendArgs &a,
                                      const DebugView &dbg, hipStream_t s);

}  // namespace recsa
