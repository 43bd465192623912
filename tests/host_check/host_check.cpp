// Host-side checks of librecsa's validation, tree layout and workspace sizing, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the kernels
// are not built: nothing here launches one).  Exercises the sizing and layout
// arithmetic at the long-context shapes (1M + 8192 and 2M tokens, fanout 64) and the
// argument checks of every entry point, with pointers that are never dereferenced.
// Prints one line per failed check and exits non-zero if any failed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "recsa.h"

static int g_failed = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++g_failed;                                                           \
        }                                                                         \
    } while (0)

static recsa_params params(int32_t hkv, int32_t hq, int32_t d, int32_t b, int32_t k, int64_t cap,
                           int32_t store = RECSA_BF16, int32_t path = RECSA_PATH_AUTO) {
    recsa_params p;
    memset(&p, 0, sizeof p);
    p.n_kv_heads = hkv;
    p.n_q_heads = hq;
    p.head_dim = d;
    p.fanout_b = b;
    p.budget_k = k;
    p.store_dtype = store;
    p.out_dtype = RECSA_FP32;
    p.path = path;
    p.rope_base = 1e6;
    p.softmax_scale = 0.088f;
    p.pool_scale = 0.088f;
    p.capacity = cap;
    return p;
}

// Tree layout: node capacities floor(cap / b^l), arrays 256-byte aligned, in order,
// not overlapping, inside recsa_tree_bytes.
static void check_layout(const recsa_params &p) {
    const int32_t H = recsa_num_levels(&p);
    CHECK(H >= 0);
    const size_t total = recsa_tree_bytes(&p);
    CHECK(total > 0 && total % 256 == 0);
    const size_t es = p.store_dtype == RECSA_BF16 ? 2 : 4;
    int64_t pw = 1;
    size_t prev_end = 0;
    for (int32_t l = 1; l <= H; ++l) {
        pw *= p.fanout_b;
        size_t ko = 0, vo = 0;
        int64_t nc = 0;
        CHECK(recsa_tree_layout(&p, l, &ko, &vo, &nc) == RECSA_OK);
        CHECK(nc == p.capacity / pw);
        const size_t arr = (size_t)p.n_kv_heads * (size_t)nc * (size_t)p.head_dim * es;
        CHECK(ko % 256 == 0 && vo % 256 == 0);
        CHECK(ko >= prev_end);
        CHECK(vo >= ko + arr);
        prev_end = vo + arr;
        CHECK(prev_end <= total);
    }
    CHECK(p.capacity / (pw * p.fanout_b) == 0);      // no level above H
    CHECK(recsa_tree_layout(&p, H + 1, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_tree_layout(&p, 0, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    const int64_t kb = (int64_t)p.budget_k * p.fanout_b + p.fanout_b - 1;
    CHECK(recsa_max_candidates(&p) == std::min<int64_t>(kb, p.capacity));
    // the RoPE table (positions 0..max(max_cand, 64, b), d/2 (cos, sin) pairs) follows
    const int64_t rows = std::max<int64_t>(std::max<int64_t>(recsa_max_candidates(&p), 64), p.fanout_b) + 1;
    CHECK(total >= prev_end + (size_t)rows * (size_t)(p.head_dim / 2) * 8);
}

// Prefill workspace: zero for the row-wise layout; for the parent-major one at least
// the per-pair partial sums of every level plus the per-row logits of one pass
// (passes hold at most 131072 rows), growing with the rows up to one pass.
static void check_workspace(const recsa_params &p, int64_t chunk) {
    const int64_t rows = chunk * p.n_q_heads;
    const size_t ws = recsa_workspace_bytes(&p, rows);
    const int64_t pass = std::min<int64_t>(rows, (131072 / p.n_q_heads) * p.n_q_heads);
    const int64_t maxc = recsa_max_candidates(&p);
    const int32_t lv = recsa_num_levels(&p) + 1;
    const size_t partials = (size_t)lv * (size_t)pass * (size_t)(p.budget_k + 1) * (size_t)p.head_dim * 4;
    const size_t logits = (size_t)pass * (size_t)((maxc + 3) / 4 * 4) * 4;
    CHECK(ws % 256 == 0);
    CHECK(ws >= partials + logits);
    CHECK(ws <= 2 * (partials + logits) + ((size_t)1 << 30));
    CHECK(recsa_workspace_bytes(&p, rows / 2) <= ws);
    recsa_params rw = p;
    rw.path = RECSA_PATH_ROWWISE;
    CHECK(recsa_workspace_bytes(&rw, rows) == 0);
    // backward: fp32 gradients of every level's summary keys and values, then (>= 256
    // rows) the parent-major buffers
    size_t summaries = 0;
    for (int32_t l = 1; l <= recsa_num_levels(&p); ++l) {
        size_t ko, vo;
        int64_t nc;
        recsa_tree_layout(&p, l, &ko, &vo, &nc);
        summaries += 2 * (((size_t)p.n_kv_heads * (size_t)nc * (size_t)p.head_dim * 4 + 255) / 256 * 256);
    }
    CHECK(recsa_backward_workspace_bytes(&rw, rows) == summaries);
    CHECK(recsa_backward_workspace_bytes(&p, rows) >= summaries + partials);
    CHECK(recsa_dense_workspace_bytes(&p, 32) > 0);
    CHECK(recsa_distill_workspace_bytes(&p, 32) >= recsa_backward_workspace_bytes(&p, 32 * p.n_q_heads));
    // bf16 token gradients (fanout <= 32, not row-wise): the parent-major backward's
    // workspace plus two staging buffers of ceil(pairs / 16) + min(pairs, buckets) items
    // of b x d floats, pairs = rows (k + 1) and buckets = Hkv (capacity / b + 1)
    const size_t ws16 = recsa_backward_bf16_workspace_bytes(&p, rows);
    if (p.fanout_b <= 32 && p.path != RECSA_PATH_ROWWISE) {
        const int64_t pairs = rows * (p.budget_k + 1);
        const int64_t nb = (int64_t)p.n_kv_heads * (p.capacity / p.fanout_b + 1);
        const size_t items = (size_t)((pairs + 15) / 16 + std::min(pairs, nb));
        const size_t stage = items * (size_t)p.fanout_b * (size_t)p.head_dim * 4;
        const size_t base = recsa_backward_workspace_bytes(&p, rows);
        CHECK(ws16 % 256 == 0);
        CHECK(ws16 >= base + 2 * stage);
        CHECK(ws16 <= base + 2 * stage + 2 * 256);
        CHECK(recsa_backward_bf16_workspace_bytes(&p, rows / 2) <= ws16);
        CHECK(recsa_backward_bf16_workspace_bytes(&p, 1) > 0);   // any row count runs parent-major
    } else {
        CHECK(ws16 == 0);
    }
    CHECK(recsa_backward_bf16_workspace_bytes(&rw, rows) == 0);
}

// Argument checks of every entry point: each call below fails on the host, before any
// HIP call, with the status given; the descriptor is left as it was.
static void check_validation(const recsa_params &p) {
    char *fake = reinterpret_cast<char *>((uintptr_t)1 << 20);
    recsa_tree_desc d{fake, fake, fake, reinterpret_cast<const float *>(fake), 10};
    recsa_tree_desc empty = d;
    empty.length = 0;
    CHECK(recsa_build_tree(&p, &d, p.capacity + 1, nullptr) == RECSA_ERR_CAPACITY);
    CHECK(recsa_build_tree(&p, &d, -1, nullptr) == RECSA_ERR_CAPACITY);
    recsa_tree_desc mis = d;
    mis.tree = fake + 16;
    CHECK(recsa_build_tree(&p, &mis, 0, nullptr) == RECSA_ERR_INVALID_ARG);
    recsa_tree_desc full = d;
    full.length = p.capacity;
    CHECK(recsa_append(&p, &full, fake, fake, 1, nullptr) == RECSA_ERR_CAPACITY);
    CHECK(full.length == p.capacity);
    CHECK(recsa_append(&p, &d, nullptr, fake, 1, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_append(&p, &d, fake, fake, -5, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_append(&p, &d, fake, fake, INT64_MAX, nullptr) == RECSA_ERR_CAPACITY);
    CHECK(recsa_decode(&p, &empty, fake, 1, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_decode(&p, &d, fake, 0, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_decode(&p, &d, fake + 2, 1, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_decode(&p, nullptr, fake, 1, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_decode_grouped(&p, &d, nullptr, 1, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_prefill(&p, &d, fake, 11, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_prefill(&p, &d, fake, 0, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    recsa_tree_desc big = d;
    big.length = p.capacity;
    // a parent-major prefill (bf16 storage, from 4096 rows) needs its workspace
    if (p.store_dtype == RECSA_BF16 && p.capacity >= 4096)
        CHECK(recsa_prefill(&p, &big, fake, 4096, fake, nullptr, nullptr, nullptr) ==
              RECSA_ERR_INVALID_ARG);
    std::vector<recsa_tree_desc> seqs(40, d);
    CHECK(recsa_decode_multi(&p, seqs.data(), 40, fake, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    seqs[7].length = 0;
    CHECK(recsa_decode_multi(&p, seqs.data(), 8, fake, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_decode_multi(&p, seqs.data(), 0, fake, fake, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    float *f = reinterpret_cast<float *>(fake);
    CHECK(recsa_backward(&p, &d, fake, 0, 0, f, f, f, f, f, nullptr, fake, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_backward(&p, &d, fake, 11, 1, f, f, f, f, f, nullptr, fake, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_backward(&p, &d, fake, 1, 0, f, f, f, nullptr, f, nullptr, fake, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_backward(&p, &d, fake, 1, 0, f, f, f, f, f, nullptr, nullptr, nullptr) == RECSA_ERR_INVALID_ARG);
    // bf16 token gradients: unsupported storage, fanout or path first; then both token
    // buffers required, at most one pass of rows, and the workspace
    const bool bf16_ok = p.store_dtype == RECSA_BF16 && p.fanout_b <= 32 && p.path != RECSA_PATH_ROWWISE;
    const recsa_status arg = bf16_ok ? RECSA_ERR_INVALID_ARG : RECSA_ERR_UNSUPPORTED;
    CHECK(recsa_backward_bf16(&p, &d, fake, 1, 0, f, f, nullptr, nullptr, f, nullptr, fake, nullptr) == arg);
    CHECK(recsa_backward_bf16(&p, &d, fake, 1, 0, f, f, fake, fake, f, nullptr, nullptr, nullptr) == arg);
    CHECK(recsa_backward_bf16(&p, &d, fake, 300000, 0, f, f, fake, fake, f, nullptr, fake, nullptr) ==
          RECSA_ERR_UNSUPPORTED);
    recsa_params rwp = p;
    rwp.path = RECSA_PATH_ROWWISE;
    CHECK(recsa_backward_bf16(&rwp, &d, fake, 1, 0, f, f, fake, fake, f, nullptr, fake, nullptr) ==
          RECSA_ERR_UNSUPPORTED);
    CHECK(recsa_dense_decode(&p, &empty, fake, 1, fake, fake, nullptr) == RECSA_ERR_INVALID_ARG);
    CHECK(recsa_distill_step(&p, &d, f + 1024, fake, 1, f, 0.1f, 0.9f, f, f, fake, nullptr) ==
          RECSA_ERR_INVALID_ARG);
    CHECK(strlen(recsa_last_error()) > 0);
    for (int s = 0; s <= 4; ++s) CHECK(strncmp(recsa_status_string((recsa_status)s), "RECSA_", 6) == 0);
}

int main() {
    const int64_t K1 = 1024, M1 = 1 << 20;
    // the workloads of the path: 131K; 524K + 4096; 1M + 8192 (b = 64); 2M (b = 64, k = 16)
    const recsa_params shapes[] = {
        params(8, 32, 128, 32, 8, 128 * K1),
        params(8, 32, 128, 32, 8, 512 * K1 + 4096),
        params(8, 32, 128, 64, 8, M1 + 8192),
        params(8, 32, 128, 64, 16, 2 * M1),
        params(8, 32, 128, 64, 16, 2 * M1, RECSA_BF16, RECSA_PATH_PARENT_MAJOR),
        params(1, 1, 64, 16, 4, 4096, RECSA_FP32),
        params(1, 2, 64, 2, 3, M1),          // twenty levels
        params(1, 2, 64, 3, 4, 78200),
        params(8, 64, 128, 128, 4, 8 * M1),   // the widest fanout of the parent-major layout
    };
    for (const recsa_params &p : shapes) {
        check_layout(p);
        check_validation(p);
        if (p.store_dtype == RECSA_BF16) {
            check_workspace(p, 4096);
            check_workspace(p, 8192);
        }
    }
    // parameters the library refuses
    recsa_params bad = shapes[0];
    bad.path = 3;
    CHECK(recsa_tree_bytes(&bad) == 0 && recsa_num_levels(&bad) == -1);
    bad = shapes[0];
    bad.capacity = (int64_t)1 << 31;
    CHECK(recsa_tree_bytes(&bad) == 0);
    bad = shapes[0];
    bad.head_dim = 96;
    CHECK(recsa_tree_bytes(&bad) == 0);
    bad = shapes[0];
    bad.n_q_heads = 12;
    CHECK(recsa_workspace_bytes(&bad, 4096) == 0);
    CHECK(recsa_multi_workspace_bytes(32) == 0 && recsa_multi_workspace_bytes(33) >= 33 * 32);
    // one KV head's cache past 4 GiB (32-bit offsets in the descent) is refused
    recsa_params huge = params(1, 1, 128, 64, 8, ((int64_t)1 << 31) - 1);
    recsa_tree_desc hd{reinterpret_cast<void *>(1 << 20), reinterpret_cast<void *>(1 << 20),
                       reinterpret_cast<void *>(1 << 20), reinterpret_cast<const float *>(1 << 20), 0};
    CHECK(recsa_build_tree(&huge, &hd, 0, nullptr) == RECSA_ERR_UNSUPPORTED);
    if (g_failed) {
        fprintf(stderr, "%d checks failed\n", g_failed);
        return 1;
    }
    printf("host checks passed\n");
    return 0;
}
