/*
 * recsa.h -- C ABI of the RecSA hot path on one AMD Instinct MI355X (gfx950).
 *
 * RecSA ("Recursive Sparse Attention: Million-Token Length Extrapolation at
 * Logarithmic Cost", arXiv 2611.07232, abstract) puts a tree over the KV
 * cache; a node stands for its whole subtree through a single key and the
 * average of the subtree's token values (abstract, sentence on the tree).  One
 * pooler per layer, the same at every level, makes the keys (sentence on the
 * pooler).  A query walks down the tree and holds on to no more than k
 * candidates per level; each candidate it drops joins, through its summary,
 * the same softmax as the exact tokens it reaches at the bottom (sentence on
 * selection), and an entry's rotary position is its rank in the candidate list
 * of its level (sentence on RoPE).
 *
 * Conventions shared by every call
 *  - All tensors are caller-owned device memory.  The library allocates
 *    nothing, frees nothing and keeps no pointer after a call returns; inputs
 *    are borrowed for the stream-ordered duration of the work it enqueues.
 *    Its one piece of state is the fixed sequence table of
 *    recsa_decode_multi_noalloc (static device memory, one per GPU).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work of a call is enqueued on it; no call synchronizes the device.
 *  - Arguments are validated on the host before any HIP call.  A failure
 *    returns a status other than RECSA_OK, enqueues nothing and leaves the
 *    tree descriptor unchanged; recsa_last_error() then describes it.  Launch
 *    failures return RECSA_ERR_HIP.  Faults inside kernels surface at the
 *    caller's next synchronization.  Nothing throws or aborts.
 *  - Storage: K, V, Q and the tree's summaries are in `store_dtype` (fp32 or
 *    bf16 bit patterns); all arithmetic is fp32.
 *  - Tree shape: level l has N_l = floor(n / b^l) complete nodes over n
 *    tokens (aligned blocks of b^l tokens); only complete nodes have
 *    summaries.  Levels run 1..recsa_num_levels(params) for `capacity` tokens.
 *  - Query head h reads KV head h / (n_q_heads / n_kv_heads).
 */
#ifndef RECSA_H
#define RECSA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define RECSA_API __attribute__((visibility("default")))
#else
#define RECSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RECSA_OK = 0,
    RECSA_ERR_INVALID_ARG = 1,   /* a null/misaligned pointer, a size out of range, bad params */
    RECSA_ERR_UNSUPPORTED = 2,   /* valid but not built for: head_dim, LDS limits */
    RECSA_ERR_CAPACITY = 3,      /* length or append past `capacity` */
    RECSA_ERR_HIP = 4            /* a HIP launch or runtime call failed */
} recsa_status;

typedef enum { RECSA_FP32 = 0, RECSA_BF16 = 1 } recsa_dtype;

/* How recsa_prefill and recsa_backward lay out their work (recsa_params.path).
 * Both layouts compute the same rule; they differ in speed and in the precision
 * of the entry logits (fp32 row-wise, split-bf16 MFMA products of about 16
 * significant bits parent-major).  The choice is part of the params, so a
 * workspace-sizing call and the call that uses the workspace always agree. */
typedef enum {
    RECSA_PATH_AUTO = 0,          /* the library chooses by storage, fanout and row count */
    RECSA_PATH_ROWWISE = 1,       /* one workgroup per row (query x query head) */
    RECSA_PATH_PARENT_MAJOR = 2   /* rows grouped by the parents they keep (bf16 storage,
                                     fanout <= 128; RECSA_ERR_UNSUPPORTED elsewhere) */
} recsa_path;

typedef struct {
    int32_t n_kv_heads;      /* >= 1 */
    int32_t n_q_heads;       /* multiple of n_kv_heads */
    int32_t head_dim;        /* 64 or 128 */
    int32_t fanout_b;        /* tree fanout b >= 2 */
    int32_t budget_k;        /* candidates kept per level, 1 <= k */
    int32_t store_dtype;     /* recsa_dtype of K, V, Q and summaries */
    int32_t out_dtype;       /* recsa_dtype of the attention output */
    int32_t path;            /* recsa_path; RECSA_PATH_AUTO (0) unless a test or a
                                measurement needs one layout */
    double  rope_base;       /* RoPE base (1e6 for the Qwen3 family); > 0 */
    float   softmax_scale;   /* logit scale s, usually 1/sqrt(head_dim) */
    float   pool_scale;      /* pooler logit scale, usually 1/sqrt(head_dim) */
    int64_t capacity;        /* tokens the cache and tree can hold, >= 1 */
} recsa_params;

typedef struct {
    void       *k_cache;     /* [n_kv_heads][capacity][head_dim] store_dtype, pre-RoPE keys */
    void       *v_cache;     /* [n_kv_heads][capacity][head_dim] store_dtype */
    void       *tree;        /* recsa_tree_bytes() bytes, 256-byte aligned; library-defined layout */
    const float *pool_w;     /* [n_kv_heads][head_dim] fp32 pooler vectors */
    int64_t     length;      /* tokens in the tree; written by build/append only */
} recsa_tree_desc;

typedef struct {             /* optional per-row outputs; NULL fields are skipped */
    int32_t *selected;       /* [rows][n_levels][budget_k]: at [r][l-1][:] the node ids kept at
                                level l, ascending, -1 padded (also for levels above the row's top) */
    float   *kth_gap;        /* [rows][n_levels]: z_(m) - z_(m+1) of level l's sorted logits,
                                m = min(k, candidates); NaN when no candidate is left out */
    int32_t *n_keys;         /* [rows]: keys scored over all levels (= entries read + kept nodes) */
} recsa_debug;

/* Levels above the tokens that `capacity` tokens can fill: max{l : capacity / b^l >= 1}.
 * Returns -1 on invalid params. */
RECSA_API int32_t recsa_num_levels(const recsa_params *p);

/* Bytes the `tree` buffer needs (summaries of every level, fp32 running means
 * for bf16 storage, and the RoPE cos/sin table).  0 on invalid params. */
RECSA_API size_t recsa_tree_bytes(const recsa_params *p);

/* Byte offsets inside `tree` of level l's key and value arrays (each
 * [n_kv_heads][nodes][head_dim] store_dtype) and that level's node capacity.
 * Level 1..recsa_num_levels().  For inspection and tests. */
RECSA_API recsa_status recsa_tree_layout(const recsa_params *p, int32_t level, size_t *key_offset,
                               size_t *val_offset, int64_t *node_capacity);

/* Largest number of candidates any level can hold for these params
 * (min(capacity, k*b + b - 1)); RoPE positions run 0..this value. */
RECSA_API int64_t recsa_max_candidates(const recsa_params *p);

/* Workspace bytes recsa_decode/recsa_prefill need for `max_rows` rows (queries x
 * query heads): 0 for decode and for calls that run one workgroup per row; a
 * bf16-storage prefill of at least 4096 rows with fanout <= 128 runs
 * parent-major (rows grouped by the parents they keep) and needs this much
 * device memory, 256-byte aligned, passed as `ws`.  `ws` may be NULL when this
 * is 0.  0 on invalid params. */
RECSA_API size_t recsa_workspace_bytes(const recsa_params *p, int64_t max_rows);

/* Build the tree over the first `length` tokens already stored in
 * k_cache/v_cache (tree, sentence on the tree; pooler, sentence on the pooler):
 * every complete node at every level gets its pooled key
 *   alpha_c = softmax_c(pool_scale * pool_w[g] . child_key_c),  key = sum_c alpha_c child_key_c
 * (children are tokens at level 1 and the stored level l-1 keys above) and
 * its value = mean of the subtree's token values.  Also fills the RoPE table.
 * Sets desc->length = length.  0 <= length <= capacity. */
RECSA_API recsa_status recsa_build_tree(const recsa_params *p, recsa_tree_desc *desc, int64_t length,
                              void *stream);

/* Append n_new tokens (k_new, v_new: [n_new][n_kv_heads][head_dim] store_dtype,
 * token-major) after desc->length and summarize every node that became
 * complete, lowest level first.  Existing nodes are not touched.
 * desc->length += n_new.  The tree must have been built (any length). */
RECSA_API recsa_status recsa_append(const recsa_params *p, recsa_tree_desc *desc, const void *k_new,
                          const void *v_new, int64_t n_new, void *stream);

/* Decode: `batch` queries q[batch][n_q_heads][head_dim] (store_dtype, pre-RoPE),
 * each attending to all desc->length tokens (sentence on selection; sentence on RoPE):
 * per level from the top, every candidate i is scored
 *   z_i = softmax_scale * <rope(q, n), rope(key_i, i)>,  n = the level's candidate count,
 * the min(k, n) best are kept (equal logits: lower candidate index), every
 * other candidate becomes a softmax entry with its summary value, and the
 * kept nodes' children followed by the level's orphan nodes (children of the
 * partial parent) become the next level's candidates.  At level 0 every
 * candidate token (the kept nodes' tokens, then the partial tail) is an entry
 * with its exact value.  out[batch][n_q_heads][head_dim] (out_dtype) is the
 * softmax over all entries.  RoPE is rotate-half: pair (i, i + head_dim/2)
 * turns by pos * rope_base^(-2i/head_dim).  `dbg` may be NULL. */
RECSA_API recsa_status recsa_decode(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                          int32_t batch, void *out, const recsa_debug *dbg, void *ws,
                          void *stream);

/* Decode with one selection per (query, KV group) instead of per query head:
 * the G = n_q_heads / n_kv_heads heads h = g*G .. g*G + G - 1 that read KV
 * head g descend together.  Per level the group's score of a candidate is the
 * sum of the G heads' logits z_i (the logit of the summed query, since RoPE
 * and the inner product are linear); the min(k, n) best by that score are
 * kept (equal scores: lower candidate index), for all G heads.  Each head's
 * softmax runs over the shared entries with its own logits, so each key and
 * value row is read once per group rather than once per head.  This is a
 * variant, not the RecSA rule (which selects per head): per-group top-k is
 * the selection of MiniMax Sparse Attention (its abstract, on the search-results
 * page for "coarse attention block"); summing the heads' logits is this
 * library's reading of how a group scores.  q, out, ws, stream: as in
 * recsa_decode.  `dbg` rows are i * n_kv_heads + g, and kth_gap is that of
 * the group score.  G must be 1, 2, 4 or 8 (RECSA_ERR_UNSUPPORTED otherwise);
 * with G = 1 the result is recsa_decode's. */
RECSA_API recsa_status recsa_decode_grouped(const recsa_params *p, const recsa_tree_desc *desc,
                                  const void *q, int32_t batch, void *out,
                                  const recsa_debug *dbg, void *ws, void *stream);

/* Workspace bytes recsa_decode_multi needs for n_seq sequences (device memory):
 * 0 for up to 32 sequences, whose table travels with the launch. */
RECSA_API size_t recsa_multi_workspace_bytes(int32_t n_seq);

/* Decode for n_seq sequences at once (a serving batch): sequence i has its own
 * cache and tree, described by descs[i] (host array, same params for all,
 * each with length >= 1; read before the call returns), and one query
 * q[i][n_q_heads][head_dim] at its own position descs[i].length, with the
 * same per-level rule as recsa_decode.  out[i][n_q_heads][head_dim].  `ws`:
 * recsa_multi_workspace_bytes(n_seq) bytes of device memory, 16-byte aligned,
 * which the call fills with the sequence table on `stream` (may be NULL when
 * that is 0).  `dbg` may be NULL (rows are i * n_q_heads + h). */
RECSA_API recsa_status recsa_decode_multi(const recsa_params *p, const recsa_tree_desc *descs,
                                int32_t n_seq, const void *q, void *out, const recsa_debug *dbg,
                                void *ws, void *stream);

/* recsa_decode_multi for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call with no workspace argument.  For more than 32 sequences the sequence
 * table goes to a fixed table inside the library instead of a caller workspace:
 * device memory of 4096 entries (160 KB) per GPU, held from the first such call on
 * that GPU (the device current at the call) until the process ends.  At most 4096
 * sequences (RECSA_ERR_INVALID_ARG beyond).  The call allocates nothing and frees
 * nothing.  Every such call on one GPU shares that table: calls whose work overlaps
 * on one GPU (other streams, other threads) race and must be ordered by the caller.
 * Arguments, results and errors otherwise as recsa_decode_multi. */
RECSA_API recsa_status recsa_decode_multi_noalloc(const recsa_params *p, const recsa_tree_desc *descs,
                                        int32_t n_seq, const void *q, void *out,
                                        const recsa_debug *dbg, void *stream);

/* Causal prefill of the last n_q tokens of the tree (append them first):
 * q[n_q][n_q_heads][head_dim]; query j sits at token L0 + j, L0 = length - n_q,
 * and attends to tokens [0, L0 + j] through the tree of that prefix (complete
 * nodes only), with the same per-level rule as recsa_decode.
 * out[n_q][n_q_heads][head_dim].  `ws`: see recsa_workspace_bytes(p, n_q * n_q_heads)
 * (RECSA_ERR_INVALID_ARG when it is needed and NULL).  `dbg` may be NULL. */
RECSA_API recsa_status recsa_prefill(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                           int64_t n_q, void *out, const recsa_debug *dbg, void *ws,
                           void *stream);

/* Workspace bytes recsa_backward needs for up to `max_rows` rows (n_q *
 * n_q_heads; device memory, 256-byte aligned): fp32 gradients of every level's
 * summary keys and values, and, for bf16 storage and at least 256 rows (fanout
 * <= 128, and the item kernel's LDS within a CU's), the parent-major path's
 * buffers: the forward's buckets, its output, selections and per-row softmax
 * statistics.  0 on invalid params. */
RECSA_API size_t recsa_backward_workspace_bytes(const recsa_params *p, int64_t max_rows);

/* Backward of the attention output with the selection held fixed (the method
 * is trained end to end: abstract, sentence on evaluation).  For the rows of
 * recsa_decode (causal = 0: n_q queries at position desc->length) or of
 * recsa_prefill (causal = 1: the last n_q tokens' queries, causal), given
 * d_out = dL/d out [n_q][n_q_heads][head_dim] fp32, computes with the kept
 * sets of the forward rule held fixed (selection is piecewise constant; only
 * the softmax entries carry gradient):
 *   d_q [n_q][n_q_heads][head_dim] fp32, written;
 *   d_k, d_v [n_kv_heads][capacity][head_dim] fp32, WRITTEN for tokens
 *     [0, length) (rows from length on are not touched): entries' direct
 *     gradients plus those reaching summaries, pushed down the tree (a summary
 *     value is its subtree's mean; a summary key is the pooler over its stored
 *     children's keys); both NULL to skip the token gradients (d_w and d_q are
 *     still computed);
 *   d_w [n_kv_heads][head_dim] fp32, written: the pooler vectors' gradient.
 * Nothing is added to what the buffers held: a caller accumulating over calls
 * adds the results itself.  The summaries' gradients reach the tokens first
 * (written, so the tokens' gradients are never read back), then the rows' own
 * token entries are added (fp32 atomics, or read-add-store where one work
 * item owns a node's tokens); with more than one pass of rows on the
 * parent-major path (over 262144 rows) the tokens' gradients are cleared
 * first and added to instead.
 * Rounding a summary to store_dtype passes the gradient through unchanged.
 * Entry logits, softmax and the selection are recomputed as in the forward.
 * Sums over rows use fp32 atomics, so low-order bits depend on their order.
 * bf16 storage with at least 256 rows runs parent-major (as recsa_prefill
 * does): the forward again, recording the selections and each row's softmax
 * statistics, then per level the pairs (row, parent) grouped by parent, each
 * group of up to 16 pairs adding one summed gradient per child rather than one
 * per row.  Its entry logits come from the prefill's split-bf16 products (about
 * 16 significant bits), so a row whose k-th and (k+1)-th logits lie closer than
 * that may keep another candidate than the row-wise path keeps.
 * q: as the forward's, store_dtype.  ws: recsa_backward_workspace_bytes(p,
 * n_q * n_q_heads) bytes, 256-byte aligned (may be NULL when that is 0).  dbg (may be NULL): selected
 * and kth_gap as recsa_decode reports them (n_keys is not written). */
RECSA_API recsa_status recsa_backward(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                            int64_t n_q, int32_t causal, const float *d_out, float *d_q,
                            float *d_k, float *d_v, float *d_w, const recsa_debug *dbg, void *ws,
                            void *stream);

/* Workspace bytes recsa_backward_bf16 needs for up to `max_rows` rows: those of the
 * parent-major backward plus two fp32 staging buffers of
 * (ceil(max_rows * (budget_k + 1) / 16) + min(max_rows * (budget_k + 1),
 *  n_kv_heads * (capacity / fanout_b + 1))) * fanout_b * head_dim floats each.
 * 0 on invalid params or where recsa_backward_bf16 is unsupported. */
RECSA_API size_t recsa_backward_bf16_workspace_bytes(const recsa_params *p, int64_t max_rows);

/* recsa_backward with the tokens' gradients in bf16 (the cache's storage type), for
 * training loops that keep the key and value gradients in the cache's precision.
 * Same operation, rows, arguments and write semantics as recsa_backward, except:
 *   d_k, d_v [n_kv_heads][capacity][head_dim] bf16, both required, WRITTEN for tokens
 *     [0, length): each token row is its full fp32 gradient (the summaries' part plus the
 *     rows' own token entries, summed in fp32) rounded once to bf16, nearest even;
 *   d_q, d_w: fp32, as recsa_backward computes them.
 * Each row's own token entries are first summed per (level-1 parent, item of up to 16
 * rows) into an fp32 staging buffer in ws; the pass over the level-1 nodes then adds a
 * node's staged sums to its tree part as it writes each token once.  Half the token
 * gradient bytes of recsa_backward's fp32 output; it pays where the rows keep few
 * distinct level-1 nodes (decode batches), since the staging grows with the kept pairs.
 * Supported with bf16 storage, fanout_b <= 32, path other than RECSA_PATH_ROWWISE and at
 * most one pass of rows (n_q * n_q_heads <= 262144 rounded down to a multiple of
 * n_q_heads); RECSA_ERR_UNSUPPORTED otherwise.  Always runs
 * the parent-major path (any row count).  ws: recsa_backward_bf16_workspace_bytes(p,
 * n_q * n_q_heads) bytes, 256-byte aligned. */
RECSA_API recsa_status recsa_backward_bf16(const recsa_params *p, const recsa_tree_desc *desc, const void *q,
                                 int64_t n_q, int32_t causal, const float *d_out, float *d_q, void *d_k,
                                 void *d_v, float *d_w, const recsa_debug *dbg, void *ws, void *stream);

/* Workspace bytes recsa_dense_decode needs for `batch` queries (device
 * memory, 16-byte aligned): per-span partial softmax states and, for bf16
 * storage, a table of 64 x head_dim/2 RoPE rotation increments the call fills.
 * 0 on invalid arguments. */
RECSA_API size_t recsa_dense_workspace_bytes(const recsa_params *p, int32_t batch);

/* Dense causal attention of decode queries (the pooler distillation's teacher;
 * abstract, sentence on the pooler): out[i][h] = softmax over tokens t <
 * desc->length of softmax_scale * <rope(q, length), rope(K_t, t)>, applied to V
 * (no tree).  q as recsa_decode's; out [batch][n_q_heads][head_dim] out_dtype.
 * ws: recsa_dense_workspace_bytes(p, batch) bytes, 16-byte aligned. */
RECSA_API recsa_status recsa_dense_decode(const recsa_params *p, const recsa_tree_desc *desc,
                                const void *q, int32_t batch, void *out, void *ws, void *stream);

/* Workspace bytes recsa_distill_step needs for `batch` queries (device memory,
 * 256-byte aligned).  0 on invalid arguments. */
RECSA_API size_t recsa_distill_workspace_bytes(const recsa_params *p, int32_t batch);

/* One step of the pooler's distillation from dense attention (abstract,
 * sentence on the pooler; the objective is this library's reading): with the
 * decode queries q[batch][n_q_heads][head_dim] (store_dtype, at position
 * desc->length) and their dense outputs `teacher` (fp32, e.g. from
 * recsa_dense_decode with out_dtype fp32),
 *   loss = (1 / (batch * n_q_heads)) * sum ||recsa_decode(q) - teacher||^2,
 * written to *loss (device fp32), then dloss/dw with the selection held fixed
 * (as recsa_backward), then SGD with momentum on the pooler vectors,
 *   velocity <- momentum * velocity + dloss/dw,  pool_w <- pool_w - lr * velocity,
 * then every summary key is pooled again from the new pool_w (the summary
 * values, subtree means, do not depend on it and stay as built: the tree must
 * have been built over the current cache).  pool_w must be
 * desc->pool_w ([n_kv_heads][head_dim] fp32, updated in place); velocity has
 * its shape (fp32, the caller zeroes it before the first step).  ws:
 * recsa_distill_workspace_bytes(p, batch) bytes, 256-byte aligned.  The loss is
 * the one before the update. */
RECSA_API recsa_status recsa_distill_step(const recsa_params *p, recsa_tree_desc *desc, float *pool_w,
                                const void *q, int32_t batch, const float *teacher, float lr,
                                float momentum, float *velocity, float *loss, void *ws,
                                void *stream);

/* Static name of a status code. */
RECSA_API const char *recsa_status_string(recsa_status s);

/* Message describing the last failure on the calling thread ("" if none). */
RECSA_API const char *recsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RECSA_H */
