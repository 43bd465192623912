"""GPU parity of decode with one selection per (query, KV group): the G query
heads of a KV group share each level's top-k (by the sum of their logits) and
keep their own softmax.  Compared with the oracle's group descent on the same
seeded inputs: selections exactly (near-ties of the group score replayed),
outputs within 1e-5 (fp32) or 2e-2 x RMS (bf16)."""
import numpy as np
import pytest
import torch

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


CASES = [
    # (workload, L, n_kv, n_q, overrides)
    ("tiny_f32_4k", 4096, 1, 4, {}),                      # G = 4, fp32, d = 64, three levels
    ("tiny_f32_4k", 4229, 2, 4, {}),                      # G = 2, two KV heads, ragged tail
    ("tiny_f32_4k", 3001, 1, 8, {"b": 5, "k": 3}),        # G = 8, odd fanout, orphans everywhere
    ("tiny_f32_4k", 5000, 1, 8, {"d": 128}),              # G = 8 at d = 128
    ("tiny_f32_4k", 7000, 1, 4, {"b": 100, "k": 2}),      # 70 top candidates: scored in a pass
    ("tiny_f32_4k", 10, 1, 4, {}),                        # L < b: the tokens are the top level
    ("tiny_f32_4k", 1, 1, 2, {}),                         # one token
    ("tiny_f32_4k", 300, 1, 2, {"dtype": "bf16"}),        # bf16 storage, d = 64
    ("qwen3_4b_131k", 40961, 8, 32, {}),                  # the Qwen3-4B layer shape, G = 4
]


def _setup(name, L, n_kv, n_q, kw, B):
    w = synth.scaled(synth.WORKLOADS[name], L, prefill_n=0, n_kv=n_kv, n_q=n_q, **kw)
    K, V = synth.gen_kv(w, 0, L)
    W = synth.pool_w(w)
    layer = P.make_layer(w, capacity=L)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    rng = np.random.default_rng(L + 7 * n_q)
    Q = synth.to_storage(rng.standard_normal((B, n_q, w.d)).astype(np.float32) * 1.5, w.dtype)
    return w, K, V, W, layer, Q


@pytest.mark.parametrize("name,L,n_kv,n_q,kw", CASES)
def test_grouped_decode(name, L, n_kv, n_q, kw):
    B = 3
    _say(f"case grouped {name} L={L} n_kv={n_kv} n_q={n_q} {kw}")
    w, K, V, W, layer, Q = _setup(name, L, n_kv, n_q, kw, B)
    out, dbg = layer.decode_grouped(P.to_device(Q, w.dtype), debug=True)
    torch.cuda.synchronize()
    heads = list(range(n_kv)) if n_kv <= 2 else [0, n_kv - 1]
    trees = {g: P.head_tree(K, V, W, g, w, L) for g in heads}
    rows = [(i, g) for i in range(B) for g in heads]
    rep = P.check_groups(trees, Q.astype(np.float64), rows, lambda i: L, w.k, w.rope_base,
                         w.softmax_scale, out, dbg, n_kv, w.dtype)
    _say("grouped", rep)


def test_grouped_with_one_head_per_group_is_decode():
    w, K, V, W, layer, Q = _setup("tiny_f32_4k", 4229, 2, 2, {}, 4)
    q = P.to_device(Q, w.dtype)
    a = layer.decode(q)
    b = layer.decode_grouped(q)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_grouped_batch_rows_are_independent():
    """A query's result does not depend on the other queries of the call."""
    w, K, V, W, layer, Q = _setup("qwen3_4b_131k", 20000, 8, 32, {}, 5)
    q = P.to_device(Q, w.dtype)
    full = layer.decode_grouped(q)
    one = layer.decode_grouped(q[3:4].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(full[3], one[0])
