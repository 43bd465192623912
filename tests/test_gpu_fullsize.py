"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: 524K tokens (decode batch 16, per head and with one selection
per KV group, append + prefill of 4096),
1M tokens with block drift (decode batch 4, append + prefill of 8192) and 2M
tokens (decode batch 1 and 32, pooler needles that the descent must reach).
Rows are sampled; the oracle builds the trees of the sampled KV heads only."""
import numpy as np
import pytest
import torch

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _layer_at(w, K, V, W, L, Lt):
    layer = P.make_layer(w, capacity=Lt)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    return layer


def _check(w, layer_out, dbg, Q, rows, n_ctx_of, trees):
    G = w.n_q // w.n_kv
    reps = []
    for g, tree in trees.items():
        rg = [(i, h) for (i, h) in rows if h // G == g]
        reps.append(P.check_rows(tree, Q.astype(np.float64), rg, n_ctx_of, w.k, w.rope_base,
                                 w.softmax_scale, layer_out, dbg, G, w.dtype,
                                 head_of=lambda h: 0))
    return reps


@pytest.mark.parametrize("name", ["qwen3_4b_524k", "qwen3_4b_1m_drift"])
def test_full_decode_and_prefill(name):
    w = synth.WORKLOADS[name]
    B = w.max_batch
    Lt = w.L + w.prefill_n
    _say(f"case {name}: L={w.L} + {w.prefill_n}, B={B}")
    K, V = synth.gen_kv(w, 0, Lt)
    W = synth.pool_w(w)
    Qd = synth.decode_queries(w, B)
    Qp = synth.prefill_queries(w)
    layer = _layer_at(w, K, V, W, w.L, Lt)
    out_d, dbg_d = layer.decode(P.to_device(Qd, w.dtype), debug=True)
    out_g, dbg_g = layer.decode_grouped(P.to_device(Qd, w.dtype), debug=True)
    layer.append(P.to_device(np.ascontiguousarray(K[:, w.L:].transpose(1, 0, 2)), w.dtype),
                 P.to_device(np.ascontiguousarray(V[:, w.L:].transpose(1, 0, 2)), w.dtype))
    out_p, dbg_p = layer.prefill(P.to_device(Qp, w.dtype), debug=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    heads = [0, 5]
    G = w.n_q // w.n_kv
    trees = {g: P.head_tree(K, V, W, g, w, Lt) for g in heads}
    rows_d = [(i, h) for i in range(B) for h in range(w.n_q) if h // G in heads]
    rep = _check(w, out_d, dbg_d, Qd, rows_d, lambda i: w.L, trees)
    _say("decode", rep)
    rep = P.check_groups(trees, Qd.astype(np.float64), [(i, g) for i in range(B) for g in heads],
                         lambda i: w.L, w.k, w.rope_base, w.softmax_scale, out_g, dbg_g, w.n_kv,
                         w.dtype)
    _say("grouped decode", rep)
    qs = sorted(set(rng.choice(w.prefill_n, 12, replace=False).tolist()) | {0, w.prefill_n - 1})
    rows_p = [(j, h) for j in qs for h in range(w.n_q) if h // G in heads]
    rep = _check(w, out_p, dbg_p, Qp, rows_p, lambda j: w.L + j + 1, trees)
    _say("prefill", rep)


def test_full_2m_needles():
    """2M tokens, b=64, k=16: decode B=32 and B=1; every pooler needle's matching
    query reaches its needle token on the GPU, as on the oracle; grouped decode at B=32
    against the oracle's group selection on sampled rows."""
    w = synth.WORKLOADS["qwen3_4b_2m"]
    _say(f"case {w.name}: L={w.L}")
    K, V = synth.gen_kv(w, 0, w.L)
    W = synth.pool_w(w)
    Q = synth.decode_queries(w, 32)
    layer = _layer_at(w, K, V, W, w.L, w.L)
    out32, dbg = layer.decode(P.to_device(Q, w.dtype), debug=True)
    out1, dbg1 = layer.decode(P.to_device(Q[:1], w.dtype), debug=True)
    torch.cuda.synchronize()
    P.assert_same_query(out1[0], dbg1, out32[0], dbg, slice(0, w.n_q), slice(0, w.n_q))
    pairs = synth.needle_pairs(w)
    sel = dbg["selected"].cpu().numpy()
    reached = 0
    for (j, pos, g, qi, qh) in pairs:
        r = qi * w.n_q + qh
        if pos // w.b in sel[r, 0, :w.k].tolist():
            reached += 1
    assert reached == len(pairs), f"GPU descent reached {reached} of {len(pairs)} needles"
    heads = [0, 3]
    G = w.n_q // w.n_kv
    trees = {g: P.head_tree(K, V, W, g, w, w.L) for g in heads}
    rows = sorted({(qi, qh) for (_, _, g, qi, qh) in pairs if g in heads} |
                  {(i, h) for i in (0, 31) for h in range(w.n_q) if h // G in heads})
    rep = _check(w, out32, dbg, Q, rows, lambda i: w.L, trees)
    _say("decode", rep, "needles reached", reached)
    # one selection per (query, KV group) at the widest levels (k = 16, b = 64)
    out_g, dbg_g = layer.decode_grouped(P.to_device(Q, w.dtype), debug=True)
    torch.cuda.synchronize()
    rep = P.check_groups(trees, Q.astype(np.float64), [(i, g) for i in (0, 7, 31) for g in heads],
                         lambda i: w.L, w.k, w.rope_base, w.softmax_scale, out_g, dbg_g, w.n_kv,
                         w.dtype)
    _say("grouped decode", rep)
