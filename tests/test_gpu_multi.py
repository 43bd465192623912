"""GPU parity of multi-sequence decode: a serving batch in which every sequence
has its own cache and tree at its own (ragged) length, one query each.  Each
sequence is checked against the oracle on its own tree, and against a
single-sequence decode of the same layer (the same arithmetic, so bit-exact)."""
import numpy as np
import pytest
import torch

import synth
from long_context_recsa_amd.layer import decode_multi
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _sequences(base, lengths, **kw):
    """One workload per sequence (own seed), its cache loaded and tree built."""
    seqs = []
    for i, L in enumerate(lengths):
        w = synth.scaled(base, L, prefill_n=0, cfg_id=100 + 17 * i + base.cfg_id, **kw)
        K, V = synth.gen_kv(w, 0, L)
        W = synth.pool_w(w)
        layer = P.make_layer(w, capacity=max(lengths))
        P.load_cache(layer, K, V, W, L, w.dtype)
        layer.build(L)
        seqs.append((w, K, V, W, layer))
    return seqs


@pytest.mark.parametrize("name,lengths,kw", [
    # tops at levels 1, 2 and 3 in one batch, ragged tails and orphans at every level
    ("qwen3_4b_131k", [1000, 5003, 17000, 33001, 40961], {}),
    ("tiny_f32_4k", [37, 300, 4096, 2049], {}),
    ("tiny_f32_4k", [200, 3000, 4000], {"dtype": "bf16"}),
])
def test_decode_multi_ragged(name, lengths, kw):
    base = synth.WORKLOADS[name]
    _say(f"case multi {name} lengths={lengths} {kw}")
    seqs = _sequences(base, lengths, **kw)
    w0 = seqs[0][0]
    rng = np.random.default_rng(3)
    Q = (rng.standard_normal((len(lengths), w0.n_q, w0.d))).astype(np.float32)
    Q = synth.to_storage(Q, w0.dtype)
    layers = [s[4] for s in seqs]
    out, dbg = decode_multi(layers, P.to_device(Q, w0.dtype), debug=True)
    torch.cuda.synchronize()
    G = w0.n_q // w0.n_kv
    gout = P.to_host(out)
    for i, (w, K, V, W, layer) in enumerate(seqs):
        single, sdbg = layer.decode(P.to_device(Q[i:i + 1], w.dtype), debug=True)
        torch.cuda.synchronize()
        P.assert_same_query(single[0], sdbg, out[i], dbg, slice(0, w.n_q), slice(i * w.n_q, (i + 1) * w.n_q))
        heads = range(w.n_kv) if w.n_kv <= 2 else [0, w.n_kv - 1]
        for g in heads:
            tree = P.head_tree(K, V, W, g, w, w.L)
            rows = [(0, h) for h in range(w.n_q) if h // G == g]
            sub = {k: v[i * w.n_q:(i + 1) * w.n_q] for k, v in dbg.items()}
            rep = P.check_rows(tree, Q[i:i + 1].astype(np.float64), rows, lambda j: w.L, w.k,
                               w.rope_base, w.softmax_scale, out[i:i + 1], sub, G, w.dtype,
                               head_of=lambda h: 0)
            _say(f"seq {i} L={w.L} head {g}", rep)


def test_serve16_sampled():
    """The serving batch the benchmark times (16 sequences, ragged 8K..40K), in the same
    call; three sequences and two KV heads of each checked against the oracle."""
    seqs_w, Q = synth.serve_batch("qwen3_4b_serve16")
    cap = max(w.L for w in seqs_w)
    _say(f"case serve16 lengths={[w.L for w in seqs_w]}")
    layers, data = [], []
    for w in seqs_w:
        K, V = synth.gen_kv(w, 0, w.L)
        W = synth.pool_w(w)
        layer = P.make_layer(w, capacity=cap)
        P.load_cache(layer, K, V, W, w.L, w.dtype)
        layer.build(w.L)
        layers.append(layer)
        data.append((K, V, W))
    w0 = seqs_w[0]
    out, dbg = decode_multi(layers, P.to_device(Q, w0.dtype), debug=True)
    torch.cuda.synchronize()
    G = w0.n_q // w0.n_kv
    for i in (0, 7, len(seqs_w) - 1):
        w = seqs_w[i]
        K, V, W = data[i]
        for g in (0, 5):
            tree = P.head_tree(K, V, W, g, w, w.L)
            rows = [(0, h) for h in range(w.n_q) if h // G == g]
            sub = {k: v[i * w.n_q:(i + 1) * w.n_q] for k, v in dbg.items()}
            rep = P.check_rows(tree, Q[i:i + 1].astype(np.float64), rows, lambda j: w.L, w.k,
                               w.rope_base, w.softmax_scale, out[i:i + 1], sub, G, w.dtype,
                               head_of=lambda h: 0)
            _say(f"seq {i} L={w.L} head {g}", rep)


def test_decode_multi_device_table():
    """More sequences than travel with the launch (34 > 32): the table goes through
    the workspace; every sequence equals its single-sequence decode, three against
    the oracle."""
    base = synth.WORKLOADS["tiny_f32_4k"]
    rng = np.random.default_rng(8)
    lengths = [int(x) for x in rng.integers(20, 4097, size=34)]
    _say(f"case multi device table lengths={lengths}")
    seqs = _sequences(base, lengths)
    Q = synth.to_storage(rng.standard_normal((34, base.n_q, base.d)).astype(np.float32), "f32")
    layers = [s[4] for s in seqs]
    out, dbg = decode_multi(layers, P.to_device(Q, "f32"), debug=True)
    torch.cuda.synchronize()
    for i, (w, K, V, W, layer) in enumerate(seqs):
        single, sdbg = layer.decode(P.to_device(Q[i:i + 1], "f32"), debug=True)
        torch.cuda.synchronize()
        P.assert_same_query(single[0], sdbg, out[i], dbg, slice(0, w.n_q), slice(i * w.n_q, (i + 1) * w.n_q))
    for i in (0, 17, 33):
        w, K, V, W, _ = seqs[i]
        tree = P.head_tree(K, V, W, 0, w, w.L)
        sub = {k: v[i:i + 1] for k, v in dbg.items()}
        rep = P.check_rows(tree, Q[i:i + 1].astype(np.float64), [(0, 0)], lambda j: w.L, w.k,
                           w.rope_base, w.softmax_scale, out[i:i + 1], sub, 1, "f32",
                           head_of=lambda h: 0)
        _say(f"seq {i} L={w.L}", rep)
