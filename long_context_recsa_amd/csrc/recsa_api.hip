// Host side of librecsa: argument validation, the tree buffer's layout, and
// the launches of each ABI call on the caller's stream.  See include/recsa.h
// for the contract of every entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "recsa_internal.hpp"

namespace recsa {
size_t descend_lds_bytes(int32_t maxc, int32_t k, int32_t b, int32_t D, int32_t gs);
int32_t descend_max_candidates();
size_t tiled_workspace_bytes(int64_t rows, int32_t Hq, int32_t Hkv, int32_t D, int32_t b, int32_t k,
                             int32_t maxc, int64_t capacity, int32_t n_levels);
size_t tiled_select_lds_bytes(int32_t maxc, int32_t k);
int32_t tiled_max_fanout();
hipError_t launch_prefill_tiled(const TreeView &tv, int32_t D, const DescendArgs &da, int32_t Hkv,
                                int64_t length, int64_t capacity, const DebugView &dbg, void *ws,
                                hipStream_t s);
}  // namespace recsa

namespace {

using namespace recsa;

thread_local char g_err[512] = "";

recsa_status fail(recsa_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

recsa_status hip_fail(hipError_t e, const char *what) {
    return fail(RECSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int64_t kMaxCapacity = 0x7FFFFFFF;      // node ids and candidate indices are int32
constexpr size_t kMaxLds = 160 * 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t elem_bytes(int32_t dt) { return dt == RECSA_BF16 ? 2 : 4; }

// Prefill of at least this many rows (queries x query heads) over bf16 storage
// runs parent-major (rows grouped by the parents they keep, bf16 MFMA); fewer
// rows, fp32 storage or a fanout above 128 run one workgroup per row.
// params.path = RECSA_PATH_ROWWISE or RECSA_PATH_PARENT_MAJOR fixes one of the two
// (check_path has already refused a parent-major request the path cannot serve).
constexpr int64_t kTiledMinRows = 4096;

bool tiled_possible(const recsa_params *p) {
    return p->store_dtype == RECSA_BF16 && p->fanout_b <= tiled_max_fanout();
}

bool use_tiled(const recsa_params *p, int64_t rows) {
    if (p->path == RECSA_PATH_ROWWISE || !tiled_possible(p)) return false;
    if (p->path == RECSA_PATH_PARENT_MAJOR) return true;
    return rows >= kTiledMinRows;
}

// The backward's parent-major path: the same storage and fanout conditions as the
// forward's, its own threshold.  It runs the forward again with its bucket
// set-up (a fixed ~0.2 ms at 524K tokens), so the row-wise backward stays faster up to
// about 128 rows; from 256 rows on the parent-major one is (1.6-2x at 1024 rows, 19x
// at 131072 rows, 524K tokens, Qwen3-4B layer).
constexpr int64_t kTiledBackwardMinRows = 256;

bool tiled_backward_possible(const recsa_params *p) {
    return tiled_possible(p) && tiled_backward_lds_bytes(p->head_dim, p->fanout_b) <= kMaxLds;
}

bool use_tiled_backward(const recsa_params *p, int64_t rows) {
    if (p->path == RECSA_PATH_ROWWISE || !tiled_backward_possible(p)) return false;
    if (p->path == RECSA_PATH_PARENT_MAJOR) return true;
    return rows >= kTiledBackwardMinRows;
}

struct Layout {
    int32_t n_levels = 0;
    int64_t node_cap[kMaxLevels + 1] = {};
    size_t key_off[kMaxLevels + 1] = {};
    size_t val_off[kMaxLevels + 1] = {};
    size_t mean_off[kMaxLevels + 1] = {};
    bool has_mean[kMaxLevels + 1] = {};
    size_t rope_off = 0;
    int32_t rope_rows = 0;
    int64_t max_cand = 0;
    size_t total = 0;
};

recsa_status check_params(const recsa_params *p) {
    if (p == nullptr) return fail(RECSA_ERR_INVALID_ARG, "params is NULL");
    if (p->n_kv_heads < 1) return fail(RECSA_ERR_INVALID_ARG, "n_kv_heads must be >= 1");
    if (p->n_q_heads < p->n_kv_heads || p->n_q_heads % p->n_kv_heads != 0)
        return fail(RECSA_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(RECSA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
    if (p->fanout_b < 2) return fail(RECSA_ERR_INVALID_ARG, "fanout_b must be >= 2");
    if (p->budget_k < 1) return fail(RECSA_ERR_INVALID_ARG, "budget_k must be >= 1");
    if (p->store_dtype != RECSA_FP32 && p->store_dtype != RECSA_BF16)
        return fail(RECSA_ERR_INVALID_ARG, "store_dtype must be RECSA_FP32 or RECSA_BF16");
    if (p->out_dtype != RECSA_FP32 && p->out_dtype != RECSA_BF16)
        return fail(RECSA_ERR_INVALID_ARG, "out_dtype must be RECSA_FP32 or RECSA_BF16");
    if (p->path != RECSA_PATH_AUTO && p->path != RECSA_PATH_ROWWISE &&
        p->path != RECSA_PATH_PARENT_MAJOR)
        return fail(RECSA_ERR_INVALID_ARG, "path must be a recsa_path value");
    if (!(p->rope_base > 0.0) || !isfinite(p->rope_base))
        return fail(RECSA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
    if (!isfinite(p->softmax_scale) || !isfinite(p->pool_scale))
        return fail(RECSA_ERR_INVALID_ARG, "scales must be finite");
    if (p->capacity < 1 || p->capacity > kMaxCapacity)
        return fail(RECSA_ERR_INVALID_ARG, "capacity must be in [1, 2^31 - 1]");
    return RECSA_OK;
}

// Requires valid params.
Layout make_layout(const recsa_params *p) {
    Layout L;
    const int64_t b = p->fanout_b, D = p->head_dim;
    const size_t es = elem_bytes(p->store_dtype);
    int64_t n = p->capacity / b;
    while (n >= 1 && L.n_levels < kMaxLevels) {
        ++L.n_levels;
        L.node_cap[L.n_levels] = n;
        n /= b;
    }
    size_t off = 0;
    for (int l = 1; l <= L.n_levels; ++l) {
        const size_t arr = (size_t)p->n_kv_heads * (size_t)L.node_cap[l] * (size_t)D;
        L.key_off[l] = off;
        off = align_up(off + arr * es);
        L.val_off[l] = off;
        off = align_up(off + arr * es);
        // fp32 running means feed the next level's values when storage rounds to bf16
        L.has_mean[l] = (p->store_dtype == RECSA_BF16) && (l < L.n_levels);
        if (L.has_mean[l]) {
            L.mean_off[l] = off;
            off = align_up(off + arr * sizeof(float));
        }
    }
    const int64_t kb = (int64_t)p->budget_k * b + b - 1;
    L.max_cand = kb < p->capacity ? kb : p->capacity;
    // positions 0..max_cand, and at least 0..max(64, b): the descent also reads the
    // rotation of every child offset c < b
    int64_t rows = L.max_cand > 64 ? L.max_cand : 64;
    if (rows < b) rows = b;
    L.rope_rows = (int32_t)(rows + 1);
    L.rope_off = off;
    off = align_up(off + (size_t)L.rope_rows * (size_t)(D / 2) * sizeof(float2));
    L.total = off;
    return L;
}

recsa_status check_limits(const recsa_params *p, const Layout &L) {
    // the descent addresses one KV head's rows with 32-bit byte offsets
    if ((uint64_t)p->capacity * (uint64_t)p->head_dim * elem_bytes(p->store_dtype) > 0xFFFFFFFFull)
        return fail(RECSA_ERR_UNSUPPORTED, "one KV head's cache must be under 4 GiB (capacity %lld)",
                    (long long)p->capacity);
    if (L.max_cand > descend_max_candidates())
        return fail(RECSA_ERR_UNSUPPORTED,
                    "a level can hold %lld candidates (min(capacity, k*b + b - 1)); at most %d "
                    "are supported",
                    (long long)L.max_cand, descend_max_candidates());
    if (descend_lds_bytes((int32_t)L.max_cand, p->budget_k, p->fanout_b, p->head_dim, 1) > kMaxLds)
        return fail(RECSA_ERR_UNSUPPORTED, "budget_k and fanout_b need more LDS than a CU has");
    return RECSA_OK;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

recsa_status check_desc(const recsa_params *p, const recsa_tree_desc *d) {
    if (d == nullptr) return fail(RECSA_ERR_INVALID_ARG, "tree descriptor is NULL");
    if (d->k_cache == nullptr || d->v_cache == nullptr || d->tree == nullptr ||
        d->pool_w == nullptr)
        return fail(RECSA_ERR_INVALID_ARG, "k_cache, v_cache, tree and pool_w must be non-NULL");
    if (!aligned(d->k_cache, 16) || !aligned(d->v_cache, 16) || !aligned(d->pool_w, 16))
        return fail(RECSA_ERR_INVALID_ARG, "k_cache, v_cache and pool_w must be 16-byte aligned");
    if (!aligned(d->tree, kAlign)) return fail(RECSA_ERR_INVALID_ARG, "tree must be 256-byte aligned");
    if (d->length < 0 || d->length > p->capacity)
        return fail(RECSA_ERR_CAPACITY, "length %lld outside [0, capacity]", (long long)d->length);
    return RECSA_OK;
}

TreeView make_view(const recsa_params *p, const recsa_tree_desc *d, const Layout &L) {
    TreeView tv{};
    char *base = static_cast<char *>(d->tree);
    tv.k_cache = d->k_cache;
    tv.v_cache = d->v_cache;
    tv.cap = p->capacity;
    tv.n_levels = L.n_levels;
    for (int l = 1; l <= L.n_levels; ++l) {
        tv.key[l] = base + L.key_off[l];
        tv.val[l] = base + L.val_off[l];
        tv.mean[l] = L.has_mean[l] ? reinterpret_cast<float *>(base + L.mean_off[l]) : nullptr;
        tv.node_cap[l] = L.node_cap[l];
    }
    tv.rope = reinterpret_cast<const float2 *>(base + L.rope_off);
    tv.rope_rows = L.rope_rows;
    return tv;
}

// Summarize every node that is complete at new_len and was not at old_len (keys_only:
// the summary keys alone, the means being those stored already).
recsa_status grow_levels(const recsa_params *p, const recsa_tree_desc *d, const Layout &L,
                         const TreeView &tv, int64_t old_len, int64_t new_len, hipStream_t s,
                         bool keys_only = false) {
    int64_t pw = 1;
    for (int l = 1; l <= L.n_levels; ++l) {
        pw *= p->fanout_b;
        const int64_t n0 = old_len / pw, n1 = new_len / pw;
        if (n1 == 0) break;
        if (n1 > n0) {
            hipError_t e = launch_level(tv, (recsa_dtype)p->store_dtype, p->n_kv_heads,
                                        p->head_dim, p->fanout_b, l, n0, n1, d->pool_w,
                                        p->pool_scale, keys_only, s);
            if (e != hipSuccess) return hip_fail(e, "tree level launch");
        }
    }
    return RECSA_OK;
}

recsa_status run_descend(const recsa_params *p, const recsa_tree_desc *d, const void *q,
                         int64_t n_queries, int64_t ctx_base, int32_t ctx_step, void *out,
                         const recsa_debug *dbg, bool tiled, void *ws, hipStream_t s,
                         bool group_shared = false) {
    recsa_status st = check_params(p);
    if (st != RECSA_OK) return st;
    const Layout L = make_layout(p);
    if ((st = check_limits(p, L)) != RECSA_OK) return st;
    const int32_t G = p->n_q_heads / p->n_kv_heads;
    const int32_t gs = group_shared ? G : 1;
    if (gs != 1 && gs != 2 && gs != 4 && gs != 8)
        return fail(RECSA_ERR_UNSUPPORTED,
                    "a shared selection is built for groups of 1, 2, 4 or 8 query heads (got %d)",
                    (int)G);
    if (descend_lds_bytes((int32_t)L.max_cand, p->budget_k, p->fanout_b, p->head_dim, gs) > kMaxLds)
        return fail(RECSA_ERR_UNSUPPORTED,
                    "budget_k and fanout_b need more LDS than a CU has for %d heads per row", (int)gs);
    if ((st = check_desc(p, d)) != RECSA_OK) return st;
    if (q == nullptr || out == nullptr) return fail(RECSA_ERR_INVALID_ARG, "q and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(out, 16))
        return fail(RECSA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
    const int64_t rows = n_queries * p->n_q_heads;
    if (rows > 0x7FFFFFFF) return fail(RECSA_ERR_INVALID_ARG, "too many rows in one call");
    const TreeView tv = make_view(p, d, L);
    DescendArgs a{};
    a.q = q;
    a.out = out;
    a.rows = rows;
    a.Hq = p->n_q_heads;
    a.G = G;
    a.gs = gs;
    a.ctx_base = ctx_base;
    a.ctx_step = ctx_step;
    a.b = p->fanout_b;
    a.k = p->budget_k;
    a.max_cand = (int32_t)L.max_cand;
    a.scale = p->softmax_scale;
    a.out_bf16 = p->out_dtype == RECSA_BF16;
    DebugView dv{};
    if (dbg != nullptr) {
        dv.selected = dbg->selected;
        dv.kth_gap = dbg->kth_gap;
        dv.n_keys = dbg->n_keys;
    }
    if (tiled) {
        if (ws == nullptr || !aligned(ws, 256))
            return fail(RECSA_ERR_INVALID_ARG,
                        "this prefill (%lld rows) needs a 256-byte aligned workspace of "
                        "recsa_workspace_bytes(params, %lld) bytes",
                        (long long)rows, (long long)rows);
        if (tiled_select_lds_bytes((int32_t)L.max_cand, p->budget_k) > kMaxLds)
            return fail(RECSA_ERR_UNSUPPORTED, "selection of %lld candidates needs too much LDS",
                        (long long)L.max_cand);
        hipError_t e = launch_prefill_tiled(tv, p->head_dim, a, p->n_kv_heads, d->length, p->capacity,
                                            dv, ws, s);
        if (e != hipSuccess) return hip_fail(e, "tiled prefill launch");
        return RECSA_OK;
    }
    hipError_t e = launch_descend(tv, (recsa_dtype)p->store_dtype, p->head_dim, a, dv, s);
    if (e != hipSuccess) return hip_fail(e, "descend launch");
    return RECSA_OK;
}

// bf16 token gradients: the parent-major backward in one pass of rows, with the tree
// pass at level 1 in one pass over each node's children (fanout <= 32)
bool bf16_grads_possible(const recsa_params *p) {
    return p->path != RECSA_PATH_ROWWISE && tiled_backward_possible(p) && p->fanout_b <= 32;
}

size_t backward_grad_bytes(const recsa_params *p, const Layout &L) {
    size_t total = 0;
    for (int l = 1; l <= L.n_levels; ++l)
        total += 2 * align_up((size_t)p->n_kv_heads * (size_t)L.node_cap[l] * (size_t)p->head_dim * sizeof(float));
    return total;
}

size_t backward_ws_bytes(const recsa_params *p, int64_t max_rows, bool bf16_grads) {
    if (check_params(p) != RECSA_OK || max_rows < 0) return 0;
    if (bf16_grads && !bf16_grads_possible(p)) return 0;
    const Layout L = make_layout(p);
    size_t total = backward_grad_bytes(p, L);
    if (bf16_grads || use_tiled_backward(p, max_rows))
        total += tiled_backward_workspace_bytes(max_rows, p->n_q_heads, p->n_kv_heads, p->head_dim, p->fanout_b,
                                                p->budget_k, (int32_t)L.max_cand, p->capacity, L.n_levels,
                                                bf16_grads);
    return total;
}

// d_k, d_v: fp32, or bf16 with bf16_grads
recsa_status run_backward(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                          int64_t n_q, int32_t causal, const float *d_out, float *d_q, void *d_k,
                          void *d_v, bool bf16_grads, float *d_w, const recsa_debug *dbg, void *ws,
                          void *stream) {
    recsa_status st = check_params(p);
    if (st != RECSA_OK) return st;
    const Layout L = make_layout(p);
    if ((st = check_limits(p, L)) != RECSA_OK) return st;
    if ((st = check_desc(p, desc)) != RECSA_OK) return st;
    if (desc->length < 1) return fail(RECSA_ERR_INVALID_ARG, "the backward needs at least one cached token");
    if (p->path == RECSA_PATH_PARENT_MAJOR && !tiled_backward_possible(p))
        return fail(RECSA_ERR_UNSUPPORTED,
                    "the parent-major backward needs bf16 storage, fanout_b <= %d and its item "
                    "kernel's LDS within a CU's", (int)tiled_max_fanout());
    if (bf16_grads && !bf16_grads_possible(p))
        return fail(RECSA_ERR_UNSUPPORTED,
                    "bf16 token gradients need bf16 storage, fanout_b <= 32, the parent-major path "
                    "(path not RECSA_PATH_ROWWISE) and its item kernel's LDS within a CU's");
    if (n_q < 1) return fail(RECSA_ERR_INVALID_ARG, "n_q must be >= 1");
    if (causal != 0 && causal != 1) return fail(RECSA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (causal && n_q > desc->length)
        return fail(RECSA_ERR_INVALID_ARG, "n_q (%lld) exceeds the tree length (%lld)", (long long)n_q,
                    (long long)desc->length);
    const void *ptrs[] = {q, d_out, d_q, d_w};
    for (const void *ptr : ptrs) {
        if (ptr == nullptr) return fail(RECSA_ERR_INVALID_ARG, "q, d_out, d_q and d_w must be non-NULL");
        if (!aligned(ptr, 16)) return fail(RECSA_ERR_INVALID_ARG, "q, d_out, d_q and d_w must be 16-byte aligned");
    }
    if ((d_k == nullptr) != (d_v == nullptr))
        return fail(RECSA_ERR_INVALID_ARG, "d_k and d_v must both be given or both be NULL");
    if (bf16_grads && d_k == nullptr) return fail(RECSA_ERR_INVALID_ARG, "d_k and d_v must be non-NULL");
    if (!aligned(d_k, 16) || !aligned(d_v, 16))
        return fail(RECSA_ERR_INVALID_ARG, "d_k and d_v must be 16-byte aligned");
    const int64_t rows = n_q * p->n_q_heads;
    if (rows > 0x7FFFFFFF) return fail(RECSA_ERR_INVALID_ARG, "too many rows in one call");
    if (bf16_grads && !tiled_backward_one_pass(rows, p->n_q_heads))
        return fail(RECSA_ERR_UNSUPPORTED, "bf16 token gradients take at most one pass of rows (%lld rows given)",
                    (long long)rows);
    const size_t ws_bytes = backward_ws_bytes(p, rows, bf16_grads);
    if (ws_bytes > 0 && (ws == nullptr || !aligned(ws, 256)))
        return fail(RECSA_ERR_INVALID_ARG,
                    bf16_grads ? "the backward needs a 256-byte aligned workspace of "
                                 "recsa_backward_bf16_workspace_bytes() bytes"
                               : "the backward needs a 256-byte aligned workspace of "
                                 "recsa_backward_workspace_bytes() bytes");
    if (backward_rows_lds_bytes((int32_t)L.max_cand, p->budget_k, L.n_levels, p->head_dim) > kMaxLds)
        return fail(RECSA_ERR_UNSUPPORTED, "budget_k and fanout_b need more LDS than a CU has");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const TreeView tv = make_view(p, desc, L);
    BwdArgs a{};
    a.q = q;
    a.dout = d_out;
    a.dq = d_q;
    a.dk = bf16_grads ? nullptr : static_cast<float *>(d_k);
    a.dv = bf16_grads ? nullptr : static_cast<float *>(d_v);
    char *w = static_cast<char *>(ws);
    for (int l = 1; l <= L.n_levels; ++l) {
        const size_t bytes = align_up((size_t)p->n_kv_heads * (size_t)L.node_cap[l] * (size_t)p->head_dim * sizeof(float));
        a.gk[l] = reinterpret_cast<float *>(w);
        a.gv[l] = reinterpret_cast<float *>(w + bytes);
        w += 2 * bytes;
    }
    a.rows = rows;
    a.Hq = p->n_q_heads;
    a.G = p->n_q_heads / p->n_kv_heads;
    a.ctx_base = causal ? desc->length - n_q + 1 : desc->length;
    a.ctx_step = causal ? 1 : 0;
    a.b = p->fanout_b;
    a.k = p->budget_k;
    a.max_cand = (int32_t)L.max_cand;
    a.scale = p->softmax_scale;
    DebugView dv{};
    if (dbg != nullptr) {
        dv.selected = dbg->selected;
        dv.kth_gap = dbg->kth_gap;
        dv.n_keys = nullptr;
    }
    const size_t grad_bytes = backward_grad_bytes(p, L);
    hipError_t e = launch_fill_zero(d_w, (size_t)p->n_kv_heads * p->head_dim * sizeof(float), s);
    if (e != hipSuccess) return hip_fail(e, "gradient clear");
    // Every gradient is written.  Wherever the order allows, the tree pass writes a
    // level's children's gradients before the rows' entries of that child level are
    // added to them, so no gradient is read back:
    //   parent-major in one pass of rows: the tree pass runs between the levels' items;
    //   row-wise: the summaries' entries and dq first (phase 1), the tree pass (the
    //     tokens' gradients written at level 1; above it, added to what the rows left),
    //     then the rows' token entries (phase 2);
    //   parent-major over several passes of rows: everything cleared, then added to.
    const bool tiled = bf16_grads || use_tiled_backward(p, rows);
    const bool tokens = d_k != nullptr && !bf16_grads;
    const bool interleave = tiled && tiled_backward_one_pass(rows, p->n_q_heads);
    const bool split = tokens && !tiled;
    BwdTreeArgs common{};
    common.Hkv = p->n_kv_heads;
    common.b = p->fanout_b;
    common.pool_scale = p->pool_scale;
    common.pool_w = desc->pool_w;
    common.dw = d_w;
    if (bf16_grads) {
        common.dk16 = static_cast<bf16_t *>(d_k);
        common.dv16 = static_cast<bf16_t *>(d_v);
    }
    if (!interleave) {
        e = launch_fill_zero(ws, grad_bytes, s);
        if (e != hipSuccess) return hip_fail(e, "workspace clear");
    }
    if (tiled && tokens && !interleave) {
        e = launch_zero_rows(a.dk, p->n_kv_heads, p->capacity, 0, desc->length, p->head_dim, s);
        if (e == hipSuccess) e = launch_zero_rows(a.dv, p->n_kv_heads, p->capacity, 0, desc->length, p->head_dim, s);
        if (e != hipSuccess) return hip_fail(e, "gradient clear");
    }
    if (tiled) {
        // parent-major: dq is a sum over items
        e = launch_fill_zero(d_q, (size_t)rows * p->head_dim * sizeof(float), s);
        if (e != hipSuccess) return hip_fail(e, "gradient clear");
        DescendArgs da{};
        da.q = q;
        da.out = nullptr;
        da.rows = rows;
        da.Hq = p->n_q_heads;
        da.G = a.G;
        da.gs = 1;
        da.ctx_base = a.ctx_base;
        da.ctx_step = a.ctx_step;
        da.b = a.b;
        da.k = a.k;
        da.max_cand = a.max_cand;
        da.scale = a.scale;
        e = launch_backward_tiled(tv, p->head_dim, da, p->n_kv_heads, desc->length, p->capacity, a,
                                  dbg != nullptr ? dbg->selected : nullptr, dbg != nullptr ? dbg->kth_gap : nullptr,
                                  interleave ? &common : nullptr, static_cast<char *>(ws) + grad_bytes, s);
        if (e != hipSuccess) return hip_fail(e, "tiled backward launch");
        if (interleave) return RECSA_OK;
    } else {
        a.phase = split ? 1 : 0;
        e = launch_backward_rows(tv, (recsa_dtype)p->store_dtype, p->head_dim, a, dv, s);
        if (e != hipSuccess) return hip_fail(e, "backward rows launch");
    }
    // summaries' gradients down the tree, top level first
    int64_t pw = 1;
    int top = 0;
    for (int l = 1; l <= L.n_levels; ++l) {
        pw *= p->fanout_b;
        if (desc->length / pw < 1) break;
        top = l;
    }
    for (int l = top; l >= 1; --l) {
        int64_t pl = 1;
        for (int i = 0; i < l; ++i) pl *= p->fanout_b;
        BwdTreeArgs t = common;
        t.level = l;
        t.nodes = desc->length / pl;
        t.gk = a.gk[l];
        t.gv = a.gv[l];
        t.gk_child = l >= 2 ? a.gk[l - 1] : nullptr;
        t.gv_child = l >= 2 ? a.gv[l - 1] : nullptr;
        t.dk = a.dk;
        t.dv = a.dv;
        t.write_children = split && l == 1 ? 1 : 0;
        e = launch_backward_tree(tv, (recsa_dtype)p->store_dtype, p->head_dim, t, s);
        if (e != hipSuccess) return hip_fail(e, "backward tree launch");
    }
    if (split) {
        // tokens past the last complete level-1 node have no parent to write them
        const int64_t under = desc->length / p->fanout_b * p->fanout_b;
        e = launch_zero_rows(a.dk, p->n_kv_heads, p->capacity, under, desc->length, p->head_dim, s);
        if (e == hipSuccess)
            e = launch_zero_rows(a.dv, p->n_kv_heads, p->capacity, under, desc->length, p->head_dim, s);
        if (e != hipSuccess) return hip_fail(e, "gradient clear");
        // then the rows' own token entries
        a.phase = 2;
        e = launch_backward_rows(tv, (recsa_dtype)p->store_dtype, p->head_dim, a, DebugView{}, s);
        if (e != hipSuccess) return hip_fail(e, "backward rows launch");
    }
    return RECSA_OK;
}

// The sequence table of recsa_decode_multi_noalloc for more than kInlineSeqs
// sequences: file-scope device memory, one copy per GPU, held until the process ends.
// Host code reaches it only through the address hipGetSymbolAddress gives on each
// device (the array's own name is a host-side stand-in).
constexpr int32_t kNoAllocSeqs = 4096;
static __device__ __attribute__((aligned(256))) SeqEntry scratch[kNoAllocSeqs];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The table's device address on the current device, looked up once per device.
hipError_t scratch_address(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// Multi-sequence decode: `table` is device memory for the sequence table when n_seq >
// kInlineSeqs (the caller's workspace or the no-allocation scratch).  With
// validate_only, only the argument checks run.
recsa_status run_multi(const recsa_params *p, const recsa_tree_desc *descs, int32_t n_seq,
                       const void *q, void *out, const recsa_debug *dbg, void *table, hipStream_t s,
                       bool validate_only = false) {
    recsa_status st = check_params(p);
    if (st != RECSA_OK) return st;
    const Layout L = make_layout(p);
    if ((st = check_limits(p, L)) != RECSA_OK) return st;
    if (descs == nullptr || n_seq < 1)
        return fail(RECSA_ERR_INVALID_ARG, "need at least one sequence descriptor");
    for (int32_t i = 0; i < n_seq; ++i) {
        if ((st = check_desc(p, &descs[i])) != RECSA_OK) return st;
        if (descs[i].length < 1)
            return fail(RECSA_ERR_INVALID_ARG, "sequence %d has no cached token", (int)i);
    }
    if (q == nullptr || out == nullptr) return fail(RECSA_ERR_INVALID_ARG, "q and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(out, 16))
        return fail(RECSA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
    if ((int64_t)n_seq * p->n_q_heads > 0x7FFFFFFF)
        return fail(RECSA_ERR_INVALID_ARG, "too many rows in one call");
    if (validate_only) return RECSA_OK;
    DescendArgs a{};
    hipError_t e = hipSuccess;
    if (n_seq <= kInlineSeqs) {
        // the sequence table travels in the kernel arguments
        a.n_inline = n_seq;
        for (int32_t i = 0; i < n_seq; ++i) memcpy(&a.seq_inline[i], &descs[i], sizeof(SeqEntry));
    } else {
        // the caller's descriptors are the table (SeqEntry mirrors recsa_tree_desc); a
        // pageable source is staged before the copy call returns
        e = hipMemcpyAsync(table, descs, (size_t)n_seq * sizeof(SeqEntry), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "sequence table copy");
        a.seqs = static_cast<const SeqEntry *>(table);
    }
    const TreeView tv = make_view(p, &descs[0], L);
    a.q = q;
    a.out = out;
    a.rows = (int64_t)n_seq * p->n_q_heads;
    a.Hq = p->n_q_heads;
    a.G = p->n_q_heads / p->n_kv_heads;
    a.gs = 1;
    a.ctx_base = 0;
    a.ctx_step = 0;
    a.b = p->fanout_b;
    a.k = p->budget_k;
    a.max_cand = (int32_t)L.max_cand;
    a.scale = p->softmax_scale;
    a.out_bf16 = p->out_dtype == RECSA_BF16;
    DebugView dv{};
    if (dbg != nullptr) {
        dv.selected = dbg->selected;
        dv.kth_gap = dbg->kth_gap;
        dv.n_keys = dbg->n_keys;
    }
    e = launch_descend(tv, (recsa_dtype)p->store_dtype, p->head_dim, a, dv, s);
    if (e != hipSuccess) return hip_fail(e, "descend launch");
    return RECSA_OK;
}

// Per-span partial states of dense attention: at most kDenseMaxSpans spans whatever the length.
size_t dense_part_bytes(const recsa_params *p, int32_t batch) {
    return align_up((size_t)p->n_kv_heads * (size_t)kDenseMaxSpans * (size_t)batch *
                    (size_t)(p->n_q_heads / p->n_kv_heads) *
                    (size_t)(p->head_dim + 2) * sizeof(float));
}

}  // namespace

extern "C" {

int32_t recsa_num_levels(const recsa_params *p) {
    if (check_params(p) != RECSA_OK) return -1;
    return make_layout(p).n_levels;
}

size_t recsa_tree_bytes(const recsa_params *p) {
    if (check_params(p) != RECSA_OK) return 0;
    return make_layout(p).total;
}

int64_t recsa_max_candidates(const recsa_params *p) {
    if (check_params(p) != RECSA_OK) return -1;
    return make_layout(p).max_cand;
}

recsa_status recsa_tree_layout(const recsa_params *p, int32_t level, size_t *key_offset,
                               size_t *val_offset, int64_t *node_capacity) {
    recsa_status st = check_params(p);
    if (st != RECSA_OK) return st;
    const Layout L = make_layout(p);
    if (level < 1 || level > L.n_levels)
        return fail(RECSA_ERR_INVALID_ARG, "level %d outside [1, %d]", level, L.n_levels);
    if (key_offset) *key_offset = L.key_off[level];
    if (val_offset) *val_offset = L.val_off[level];
    if (node_capacity) *node_capacity = L.node_cap[level];
    return RECSA_OK;
}

size_t recsa_workspace_bytes(const recsa_params *p, int64_t max_rows) {
    if (check_params(p) != RECSA_OK || max_rows < 1) return 0;
    if (!use_tiled(p, max_rows)) return 0;
    const Layout L = make_layout(p);
    return tiled_workspace_bytes(max_rows, p->n_q_heads, p->n_kv_heads, p->head_dim, p->fanout_b,
                                 p->budget_k, (int32_t)L.max_cand, p->capacity, L.n_levels);
}

recsa_status recsa_build_tree(const recsa_params *p, recsa_tree_desc *desc, int64_t length,
                              void *stream) {
    recsa_status st = check_params(p);
    if (st != RECSA_OK) return st;
    const Layout L = make_layout(p);
    if ((st = check_limits(p, L)) != RECSA_OK) return st;
    if ((st = check_desc(p, desc)) != RECSA_OK) return st;
    if (length < 0 || length > p->capacity)
        return fail(RECSA_ERR_CAPACITY, "length %lld outside [0, capacity]", (long long)length);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const TreeView tv = make_view(p, desc, L);
    hipError_t e = launch_rope_table(const_cast<float2 *>(tv.rope), L.rope_rows, p->head_dim,
                                     p->rope_base, s);
    if (e != hipSuccess) return hip_fail(e, "rope table launch");
    if ((st = grow_levels(p, desc, L, tv, 0, length, s)) != RECSA_OK) return st;
    desc->length = length;
    return RECSA_OK;
}

recsa_status recsa_append(const recsa_params *p, recsa_tree_desc *desc, const void *k_new,
                          const void *v_new, int64_t n_new, void *stream) {
    recsa_status st = check_params(p);
    if (st != RECSA_OK) return st;
    const Layout L = make_layout(p);
    if ((st = check_limits(p, L)) != RECSA_OK) return st;
    if ((st = check_desc(p, desc)) != RECSA_OK) return st;
    if (n_new < 0) return fail(RECSA_ERR_INVALID_ARG, "n_new must be >= 0");
    if (n_new > p->capacity - desc->length)
        return fail(RECSA_ERR_CAPACITY, "append of %lld tokens past capacity (%lld of %lld used)",
                    (long long)n_new, (long long)desc->length, (long long)p->capacity);
    if (n_new == 0) return RECSA_OK;
    if (k_new == nullptr || v_new == nullptr)
        return fail(RECSA_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
    if (!aligned(k_new, 16) || !aligned(v_new, 16))
        return fail(RECSA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const TreeView tv = make_view(p, desc, L);
    hipError_t e = launch_scatter(tv, (recsa_dtype)p->store_dtype, p->n_kv_heads, p->head_dim,
                                  k_new, v_new, desc->length, n_new, s);
    if (e != hipSuccess) return hip_fail(e, "append scatter launch");
    if ((st = grow_levels(p, desc, L, tv, desc->length, desc->length + n_new, s)) != RECSA_OK)
        return st;
    desc->length += n_new;
    return RECSA_OK;
}

recsa_status recsa_decode(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                          int32_t batch, void *out, const recsa_debug *dbg, void *ws,
                          void *stream) {
    (void)ws;
    if (batch < 1) return fail(RECSA_ERR_INVALID_ARG, "batch must be >= 1");
    if (desc != nullptr && desc->length < 1)
        return fail(RECSA_ERR_INVALID_ARG, "decode needs at least one cached token");
    return run_descend(p, desc, q, batch, desc ? desc->length : 0, 0, out, dbg, false, nullptr,
                       static_cast<hipStream_t>(stream));
}

recsa_status recsa_decode_grouped(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                                  int32_t batch, void *out, const recsa_debug *dbg, void *ws,
                                  void *stream) {
    (void)ws;
    if (batch < 1) return fail(RECSA_ERR_INVALID_ARG, "batch must be >= 1");
    if (desc != nullptr && desc->length < 1)
        return fail(RECSA_ERR_INVALID_ARG, "decode needs at least one cached token");
    return run_descend(p, desc, q, batch, desc ? desc->length : 0, 0, out, dbg, false, nullptr,
                       static_cast<hipStream_t>(stream), true);
}

size_t recsa_multi_workspace_bytes(int32_t n_seq) {
    return n_seq > kInlineSeqs ? align_up((size_t)n_seq * sizeof(SeqEntry)) : 0;
}

recsa_status recsa_decode_multi(const recsa_params *p, const recsa_tree_desc *descs, int32_t n_seq,
                                const void *q, void *out, const recsa_debug *dbg, void *ws,
                                void *stream) {
    if (n_seq > kInlineSeqs && (ws == nullptr || !aligned(ws, 16)))
        return fail(RECSA_ERR_INVALID_ARG,
                    "a 16-byte aligned workspace of recsa_multi_workspace_bytes(%d) bytes is needed",
                    (int)n_seq);
    return run_multi(p, descs, n_seq, q, out, dbg, ws, static_cast<hipStream_t>(stream));
}

recsa_status recsa_decode_multi_noalloc(const recsa_params *p, const recsa_tree_desc *descs,
                                        int32_t n_seq, const void *q, void *out,
                                        const recsa_debug *dbg, void *stream) {
    if (n_seq > kNoAllocSeqs)
        return fail(RECSA_ERR_INVALID_ARG,
                    "%d sequences exceed the %d the no-allocation decode's table holds", (int)n_seq,
                    (int)kNoAllocSeqs);
    void *table = nullptr;
    if (n_seq > kInlineSeqs) {
        // validate first, so a refused call touches no HIP state
        recsa_status st = run_multi(p, descs, n_seq, q, out, dbg, nullptr, nullptr, true);
        if (st != RECSA_OK) return st;
        hipError_t e = scratch_address(&table);
        if (e != hipSuccess) return hip_fail(e, "scratch address");
    }
    return run_multi(p, descs, n_seq, q, out, dbg, table, static_cast<hipStream_t>(stream));
}

recsa_status recsa_prefill(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                           int64_t n_q, void *out, const recsa_debug *dbg, void *ws,
                           void *stream) {
    if (n_q < 1) return fail(RECSA_ERR_INVALID_ARG, "n_q must be >= 1");
    if (desc != nullptr && n_q > desc->length)
        return fail(RECSA_ERR_INVALID_ARG, "n_q (%lld) exceeds the tree length (%lld); append first",
                    (long long)n_q, (long long)desc->length);
    if (check_params(p) == RECSA_OK && p->path == RECSA_PATH_PARENT_MAJOR && !tiled_possible(p))
        return fail(RECSA_ERR_UNSUPPORTED,
                    "the parent-major prefill needs bf16 storage and fanout_b <= %d",
                    (int)tiled_max_fanout());
    const bool tiled = check_params(p) == RECSA_OK && use_tiled(p, n_q * p->n_q_heads);
    return run_descend(p, desc, q, n_q, desc ? desc->length - n_q + 1 : 0, 1, out, dbg, tiled, ws,
                       static_cast<hipStream_t>(stream));
}

size_t recsa_backward_workspace_bytes(const recsa_params *p, int64_t max_rows) {
    return backward_ws_bytes(p, max_rows, false);
}

recsa_status recsa_backward(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                            int64_t n_q, int32_t causal, const float *d_out, float *d_q, float *d_k,
                            float *d_v, float *d_w, const recsa_debug *dbg, void *ws, void *stream) {
    return run_backward(p, desc, q, n_q, causal, d_out, d_q, d_k, d_v, false, d_w, dbg, ws, stream);
}

size_t recsa_backward_bf16_workspace_bytes(const recsa_params *p, int64_t max_rows) {
    return backward_ws_bytes(p, max_rows, true);
}

recsa_status recsa_backward_bf16(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                                 int64_t n_q, int32_t causal, const float *d_out, float *d_q, void *d_k,
                                 void *d_v, float *d_w, const recsa_debug *dbg, void *ws, void *stream) {
    return run_backward(p, desc, q, n_q, causal, d_out, d_q, d_k, d_v, true, d_w, dbg, ws, stream);
}

size_t recsa_dense_workspace_bytes(const recsa_params *p, int32_t batch) {
    if (check_params(p) != RECSA_OK || batch < 1) return 0;
    return dense_part_bytes(p, batch) + align_up((size_t)64 * (p->head_dim / 2) * sizeof(float2));
}

recsa_status recsa_dense_decode(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                                int32_t batch, void *out, void *ws, void *stream) {
    recsa_status st = check_params(p);
    if (st != RECSA_OK) return st;
    if ((st = check_desc(p, desc)) != RECSA_OK) return st;
    if (desc->length < 1) return fail(RECSA_ERR_INVALID_ARG, "dense attention needs at least one cached token");
    if (batch < 1) return fail(RECSA_ERR_INVALID_ARG, "batch must be >= 1");
    if (q == nullptr || out == nullptr || ws == nullptr)
        return fail(RECSA_ERR_INVALID_ARG, "q, out and ws must be non-NULL");
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(ws, 16))
        return fail(RECSA_ERR_INVALID_ARG, "q, out and ws must be 16-byte aligned");
    DenseArgs a{};
    a.q = q;
    a.out = out;
    a.out_bf16 = p->out_dtype == RECSA_BF16;
    a.part = static_cast<float *>(ws);
    a.k_cache = desc->k_cache;
    a.v_cache = desc->v_cache;
    a.cap = p->capacity;
    a.B = batch;
    a.Hq = p->n_q_heads;
    a.Hkv = p->n_kv_heads;
    a.G = p->n_q_heads / p->n_kv_heads;
    a.length = desc->length;
    a.span = dense_span(desc->length);
    a.nspan = (int32_t)((desc->length + a.span - 1) / a.span);
    a.base = p->rope_base;
    a.scale = p->softmax_scale;
    a.incr = reinterpret_cast<float2 *>(static_cast<char *>(ws) + dense_part_bytes(p, batch));
    hipError_t e = launch_dense((recsa_dtype)p->store_dtype, p->head_dim, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dense attention launch");
    return RECSA_OK;
}

size_t recsa_distill_workspace_bytes(const recsa_params *p, int32_t batch) {
    if (check_params(p) != RECSA_OK || batch < 1) return 0;
    const size_t rowsD = (size_t)batch * p->n_q_heads * p->head_dim * sizeof(float);
    return 3 * align_up(rowsD) + align_up((size_t)p->n_kv_heads * p->head_dim * sizeof(float)) +
           recsa_backward_workspace_bytes(p, (int64_t)batch * p->n_q_heads);
}

recsa_status recsa_distill_step(const recsa_params *p, recsa_tree_desc *desc, float *pool_w,
                                const void *q, int32_t batch, const float *teacher, float lr,
                                float momentum, float *velocity, float *loss, void *ws, void *stream) {
    recsa_status st = check_params(p);
    if (st != RECSA_OK) return st;
    if ((st = check_desc(p, desc)) != RECSA_OK) return st;
    if (desc->length < 1) return fail(RECSA_ERR_INVALID_ARG, "distillation needs at least one cached token");
    if (batch < 1) return fail(RECSA_ERR_INVALID_ARG, "batch must be >= 1");
    if (pool_w == nullptr || pool_w != desc->pool_w)
        return fail(RECSA_ERR_INVALID_ARG, "pool_w must be the tree descriptor's pooler vectors");
    const void *ptrs[] = {q, teacher, velocity, loss, ws};
    for (const void *ptr : ptrs) {
        if (ptr == nullptr) return fail(RECSA_ERR_INVALID_ARG, "q, teacher, velocity, loss and ws must be non-NULL");
    }
    if (!aligned(q, 16) || !aligned(teacher, 16) || !aligned(velocity, 16) || !aligned(ws, 256))
        return fail(RECSA_ERR_INVALID_ARG,
                    "q, teacher and velocity must be 16-byte aligned and ws 256-byte aligned");
    if (!(lr >= 0.f) || !(momentum >= 0.f && momentum < 1.f))
        return fail(RECSA_ERR_INVALID_ARG, "lr must be >= 0 and momentum in [0, 1)");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t rows = (int64_t)batch * p->n_q_heads;
    const size_t rowsD = (size_t)rows * p->head_dim * sizeof(float);
    char *w = static_cast<char *>(ws);
    float *out = reinterpret_cast<float *>(w);
    float *dout = reinterpret_cast<float *>(w + align_up(rowsD));
    float *dq = reinterpret_cast<float *>(w + 2 * align_up(rowsD));
    float *dw = reinterpret_cast<float *>(w + 3 * align_up(rowsD));
    void *bws = w + 3 * align_up(rowsD) + align_up((size_t)p->n_kv_heads * p->head_dim * sizeof(float));
    // the student: RecSA decode with fp32 output
    recsa_params pf = *p;
    pf.out_dtype = RECSA_FP32;
    if ((st = run_descend(&pf, desc, q, batch, desc->length, 0, out, nullptr, false, nullptr, s)) != RECSA_OK)
        return st;
    hipError_t e = launch_distill_loss(out, teacher, dout, loss, (int64_t)rows * p->head_dim, rows, s);
    if (e != hipSuccess) return hip_fail(e, "distillation loss launch");
    // dloss/dw (written) with the selection fixed; the token gradients are not needed
    if ((st = run_backward(p, desc, q, batch, 0, dout, dq, nullptr, nullptr, false, dw, nullptr, bws, stream)) !=
        RECSA_OK)
        return st;
    e = launch_distill_update(pool_w, velocity, dw, (int64_t)p->n_kv_heads * p->head_dim, lr, momentum, s);
    if (e != hipSuccess) return hip_fail(e, "pooler update launch");
    // every summary key depends on w, no mean does: pool the keys again, level by level
    const Layout L = make_layout(p);
    return grow_levels(p, desc, L, make_view(p, desc, L), 0, desc->length, s, true);
}

const char *recsa_status_string(recsa_status s) {
    switch (s) {
        case RECSA_OK: return "RECSA_OK";
        case RECSA_ERR_INVALID_ARG: return "RECSA_ERR_INVALID_ARG";
        case RECSA_ERR_UNSUPPORTED: return "RECSA_ERR_UNSUPPORTED";
        case RECSA_ERR_CAPACITY: return "RECSA_ERR_CAPACITY";
        case RECSA_ERR_HIP: return "RECSA_ERR_HIP";
    }
    return "RECSA_UNKNOWN_STATUS";
}

const char *recsa_last_error(void) { return g_err; }

}  // extern "C"
