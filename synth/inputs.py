"""Seeded synthetic inputs for the RecSA hot path.

This module is the only code shared by the CPU oracle side (tests, the
oracle's timing leg) and the GPU side (tests, bench).  It holds no part of
the method's arithmetic: it draws numbers, rounds them to the storage format
and plants designed structure (needle keys, slow drift) into them.

Every tensor is drawn in 65,536-token slabs from
``Generator(PCG64(SeedSequence([config, tensor, kv_head, slab])))`` so a
slab's bits do not depend on how many slabs are drawn or in what order, and
slabs can be drawn on several threads.

Workloads follow the shapes the RecSA pages evaluate on (a Qwen3-4B-shaped
attention layer: 32 query heads, 8 KV heads, head_dim 128, contexts from
131K to 2M tokens; "Recursive Sparse Attention: Million-Token Length
Extrapolation at Logarithmic Cost", abstract, the evaluation sentence).  The
RULER suite the pages score on is not reproduced: planted needle keys stand
in for its retrieval structure.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SLAB = 65536

# tensor ids in the seed sequence
T_K, T_V, T_Q, T_W, T_NEEDLE, T_DRIFT, T_QPREFILL, T_SERVE = 0, 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    L: int                 # cached tokens before any append
    n_kv: int
    n_q: int
    d: int
    b: int                 # tree fanout
    k: int                 # per-level budget
    dtype: str             # "f32" or "bf16": storage of K, V, Q and summaries
    decode_batches: tuple = ()
    prefill_n: int = 0     # queries in the causal chunk appended after L
    needles: int = 0
    needle_recipe: str = ""   # "", "plain" (6 sigma in q.k) or "pooler" (pooler-dominant)
    drift_sigma: float = 0.0  # per-1024-token block mean offset std
    rope_base: float = 1e6

    @property
    def pool_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def capacity(self) -> int:
        return self.L + self.prefill_n

    @property
    def max_batch(self) -> int:
        return max(self.decode_batches) if self.decode_batches else 0


WORKLOADS = {
    "tiny_f32_4k": Workload("tiny_f32_4k", 0, L=4096, n_kv=1, n_q=1, d=64, b=16, k=4,
                            dtype="f32", decode_batches=(8,)),
    "qwen3_4b_131k": Workload("qwen3_4b_131k", 1, L=131072, n_kv=8, n_q=32, d=128, b=32, k=8,
                              dtype="bf16", decode_batches=(1, 8), needles=16,
                              needle_recipe="plain"),
    "qwen3_4b_524k": Workload("qwen3_4b_524k", 2, L=524288, n_kv=8, n_q=32, d=128, b=32, k=8,
                              dtype="bf16", decode_batches=(16,), prefill_n=4096, needles=16,
                              needle_recipe="plain"),
    "qwen3_4b_1m_drift": Workload("qwen3_4b_1m_drift", 3, L=1048576, n_kv=8, n_q=32, d=128,
                                  b=64, k=8, dtype="bf16", decode_batches=(4,),
                                  prefill_n=8192, drift_sigma=0.3),
    "qwen3_4b_2m": Workload("qwen3_4b_2m", 4, L=2097152, n_kv=8, n_q=32, d=128, b=64, k=16,
                            dtype="bf16", decode_batches=(1, 32), needles=64,
                            needle_recipe="pooler"),
}


# Serving batches: independent sequences, each with its own cache and tree at its
# own (ragged) length, one decode query per sequence; layer shape and tree
# parameters of the named workload, plain N(0,1) keys and values.
SERVE_BATCHES = {
    "qwen3_4b_serve16": dict(base="qwen3_4b_131k", n_seq=16, lmin=8192, lmax=40960),
}


def serve_batch(name: str):
    """(per-sequence workloads, queries [n_seq][n_q][d]) of a serving batch."""
    spec = SERVE_BATCHES[name]
    base = WORKLOADS[spec["base"]]
    r = _gen(base.cfg_id, T_SERVE, 0, 0)
    lengths = r.integers(spec["lmin"], spec["lmax"] + 1, size=spec["n_seq"])
    seqs = [dataclasses.replace(base, name=f"{name}_{i}", cfg_id=1000 + 16 * base.cfg_id + i,
                                L=int(L), prefill_n=0, decode_batches=(1,), needles=0,
                                needle_recipe="")
            for i, L in enumerate(lengths)]
    q = r.standard_normal((spec["n_seq"], base.n_q, base.d), dtype=np.float32)
    return seqs, to_storage(q, base.dtype)


def scaled(w: Workload, L: int, prefill_n: int | None = None, **kw) -> Workload:
    """Same recipe at a smaller context (for tests the oracle finishes in seconds)."""
    pn = w.prefill_n if prefill_n is None else prefill_n
    return dataclasses.replace(w, L=L, prefill_n=pn, **kw)


# ----------------------------------------------------------------------------
# storage format helpers (bf16 = upper 16 bits of fp32, round-to-nearest-even)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values exactly representable in the storage dtype."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def storage_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Bit pattern to hand to the device (float32 array, or uint16 bf16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x)


def _gen(cfg_id: int, tensor: int, head: int, slab: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, tensor, head, slab])))


def _normal_rows(cfg_id: int, tensor: int, head: int, t0: int, t1: int, d: int,
                 out: np.ndarray, threads: int = 8) -> None:
    """Fill out[0:t1-t0] with N(0,1) rows for tokens [t0, t1) of one head."""
    s0, s1 = t0 // SLAB, (t1 - 1) // SLAB

    def one(s):
        a, e = s * SLAB, (s + 1) * SLAB
        blk = _gen(cfg_id, tensor, head, s).standard_normal((SLAB, d), dtype=np.float32)
        lo, hi = max(a, t0), min(e, t1)
        out[lo - t0:hi - t0] = blk[lo - a:hi - a]

    if t1 <= t0:
        return
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(s0, s1 + 1)))


def gen_kv(w: Workload, t0: int = 0, t1: int | None = None, heads=None):
    """K, V for tokens [t0, t1) as fp32 arrays [len(heads)][t1-t0][d], rounded to storage.

    Tokens past ``w.L`` (the prefill chunk) are drawn from the same slabs, so a
    chunk is the continuation of the context.  Needles and drift are planted here.
    """
    t1 = w.capacity if t1 is None else t1
    heads = range(w.n_kv) if heads is None else heads
    heads = list(heads)
    n = t1 - t0
    K = np.empty((len(heads), n, w.d), np.float32)
    V = np.empty((len(heads), n, w.d), np.float32)
    for hi, g in enumerate(heads):
        _normal_rows(w.cfg_id, T_K, g, t0, t1, w.d, K[hi])
        _normal_rows(w.cfg_id, T_V, g, t0, t1, w.d, V[hi])
        if w.drift_sigma > 0:
            _add_drift(w, g, t0, t1, K[hi], V[hi])
    if w.needles:
        for (g, pos, key) in needle_keys(w):
            if g in heads and t0 <= pos < t1:
                K[heads.index(g), pos - t0] = key
    for hi in range(len(heads)):
        K[hi] = to_storage(K[hi], w.dtype)
        V[hi] = to_storage(V[hi], w.dtype)
    return K, V


def _add_drift(w: Workload, g: int, t0: int, t1: int, K: np.ndarray, V: np.ndarray) -> None:
    blk = 1024
    nb = (w.capacity + blk - 1) // blk
    for which, arr in ((0, K), (1, V)):
        m = _gen(w.cfg_id, T_DRIFT, g, which).standard_normal((nb, w.d), dtype=np.float32)
        m *= np.float32(w.drift_sigma)
        b0, b1 = t0 // blk, (t1 - 1) // blk
        for bi in range(b0, b1 + 1):
            lo, hi = max(bi * blk, t0), min((bi + 1) * blk, t1)
            arr[lo - t0:hi - t0] += m[bi]


def pool_w(w: Workload) -> np.ndarray:
    """Pooler vector per KV head, N(0, 1/d), fp32 [n_kv][d]."""
    out = np.empty((w.n_kv, w.d), np.float32)
    for g in range(w.n_kv):
        out[g] = _gen(w.cfg_id, T_W, g, 0).standard_normal(w.d, dtype=np.float32)
    return out * np.float32(1.0 / np.sqrt(w.d))


def decode_queries(w: Workload, B: int) -> np.ndarray:
    """Decode queries [B][n_q][d]; batch B is the first B of the largest batch."""
    Bm = max(B, w.max_batch)
    q = _gen(w.cfg_id, T_Q, 0, 0).standard_normal((Bm, w.n_q, w.d), dtype=np.float32)
    if w.needle_recipe == "pooler":
        q = _pooler_needle_queries(w, q)
    return to_storage(q[:B], w.dtype)


def prefill_queries(w: Workload, n: int | None = None) -> np.ndarray:
    n = w.prefill_n if n is None else n
    q = np.empty((n, w.n_q, w.d), np.float32)
    _normal_rows(w.cfg_id, T_QPREFILL, 0, 0, n * w.n_q, w.d, q.reshape(n * w.n_q, w.d))
    return to_storage(q, w.dtype)


def _low_freq_dims(d: int, npairs: int = 8) -> np.ndarray:
    """Dims of the npairs lowest-frequency rotate-half RoPE pairs (j, j + d/2)."""
    h = d // 2
    j = np.arange(h - npairs, h)
    return np.concatenate([j, j + h])


def needle_positions(w: Workload) -> np.ndarray:
    g = _gen(w.cfg_id, T_NEEDLE, 0, 0)
    return np.sort(g.choice(w.L, size=w.needles, replace=False))


def needle_pairs(w: Workload):
    """[(needle j, token position, kv head, query index, query head)]."""
    pos = needle_positions(w)
    out = []
    if w.needle_recipe == "plain":
        nq = max(w.max_batch, 1)
        for j in range(w.needles):
            g = j % w.n_kv
            out.append((j, int(pos[j]), g, j % nq, g * (w.n_q // w.n_kv)))
    elif w.needle_recipe == "pooler":
        per = w.needles // w.n_kv
        for j in range(w.needles):
            g, i = j // per, j % per
            out.append((j, int(pos[j]), g, j % max(w.max_batch, 1), g * (w.n_q // w.n_kv)))
    return out


def _pooler_frame(w: Workload, g: int):
    """Unit pooler direction in the low-frequency subspace and 8 orthonormal
    directions orthogonal to it (both supported on the low-frequency dims)."""
    S = _low_freq_dims(w.d)
    wg = pool_w(w)[g].astype(np.float64)
    ws = np.zeros(w.d)
    ws[S] = wg[S]
    ws /= np.linalg.norm(ws)
    rs = _gen(w.cfg_id, T_NEEDLE, g, 1).standard_normal((len(S), 8))
    A = np.concatenate([ws[S][:, None], rs], axis=1)
    Qm, _ = np.linalg.qr(A)
    U = np.zeros((8, w.d))
    U[:, S] = Qm[:, 1:9].T
    return ws, U


def _pooler_needle_queries(w: Workload, q: np.ndarray) -> np.ndarray:
    """Queries for the pooler-dominant needles: every query head is projected
    orthogonal to its group's pooler direction; the head matching needle i gets
    its low-frequency part along u_i."""
    q = q.astype(np.float64).copy()
    G = w.n_q // w.n_kv
    S = _low_freq_dims(w.d)
    per = w.needles // w.n_kv
    for g in range(w.n_kv):
        ws, U = _pooler_frame(w, g)
        for h in range(g * G, (g + 1) * G):
            q[:, h] -= np.outer(q[:, h] @ ws, ws)
        for (j, pos, gg, qi, qh) in needle_pairs(w):
            if gg != g or qi >= q.shape[0]:
                continue
            i = j % per
            v = q[qi, qh].copy()
            v[S] = 0.0
            v += np.linalg.norm(q[qi, qh][S]) * U[i]
            q[qi, qh] = v
    return q.astype(np.float32)


def needle_keys(w: Workload):
    """[(kv head, position, key fp32[d])] for the planted needles."""
    out = []
    if not w.needles:
        return out
    S = _low_freq_dims(w.d)
    if w.needle_recipe == "plain":
        q = decode_queries(w, max(w.max_batch, 1)).astype(np.float64)
        for (j, pos, g, qi, qh) in needle_pairs(w):
            qv = q[qi, qh]
            qs = np.zeros(w.d)
            qs[S] = qv[S]
            ns = np.linalg.norm(qs)
            key = (6.0 * np.linalg.norm(qv) / ns) * (qs / ns)
            out.append((g, pos, key.astype(np.float32)))
    elif w.needle_recipe == "pooler":
        q = decode_queries(w, max(w.max_batch, 1)).astype(np.float64)
        wv = pool_w(w).astype(np.float64)
        per = w.needles // w.n_kv
        for (j, pos, g, qi, qh) in needle_pairs(w):
            ws, U = _pooler_frame(w, g)
            i = j % per
            # pooler logit pool_scale * w.key >= ln b + 4 on the needle
            alpha = (np.log(w.b) + 4.0) / (w.pool_scale * float(wv[g] @ ws))
            qv = q[qi, qh]
            gamma = 6.0 * np.linalg.norm(qv) / float(qv @ U[i])
            key = alpha * ws + gamma * U[i]
            out.append((g, pos, key.astype(np.float32)))
    return out
