"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs (selections bit-exact up to near ties, outputs within
1e-5 for fp32 storage and 2e-2 * RMS for bf16 storage)."""
import math

import numpy as np
import pytest
import torch

import long_context_recsa_amd as R
import synth
from oracle import recsa as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bf16_close(a, b, what):
    """bf16 summaries: the two sides round an fp32 and an f64 value, so an element may
    land one bf16 ulp away, and a parent pooled from a child that rounded the other
    way moves by at most that child's ulp.  Bound: one ulp of the element plus half an
    ulp of the node's largest element; at most 1% of the elements differ at all."""
    if a.size == 0:
        return
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(b), 1e-30))) - 7)
    row = 2.0 ** -8 * np.abs(b).max(axis=1, keepdims=True)
    assert np.all(np.abs(a - b) <= ulp + row), (what, np.abs(a - b).max())
    assert np.mean(a != b) < 1e-2, (what, np.mean(a != b))


def _tree_levels_match(layer, tree, w, L, exact_rel):
    for l in range(1, len(tree.keys)):
        gk, gv = layer.level(l)
        n = len(tree.keys[l][0])
        for g in range(w.n_kv):
            ok = P.to_host(gk[g, :n])
            ov = P.to_host(gv[g, :n])
            if w.dtype == "f32":
                np.testing.assert_allclose(ok, tree.keys[l][g], rtol=0, atol=exact_rel)
                np.testing.assert_allclose(ov, tree.vals[l][g], rtol=0, atol=exact_rel)
            else:
                _bf16_close(ok, tree.keys[l][g], (l, g, "key"))
                _bf16_close(ov, tree.vals[l][g], (l, g, "value"))


def _decode_case(w, B, k=None, L=None, out="f32", check_tree=True):
    L = w.L if L is None else L
    k = w.k if k is None else k
    _say(f"case {w.name} L={L} B={B} k={k} out={out}")
    K, V = synth.gen_kv(w, 0, L)
    W = synth.pool_w(w)
    Q = synth.decode_queries(w, B)
    layer = P.make_layer(w, capacity=L, k=k, out=out)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    out_t, dbg = layer.decode(P.to_device(Q, w.dtype), debug=True)
    torch.cuda.synchronize()
    tree = O.build_tree(K, V, W, w.b, w.dtype, w.pool_scale, L)
    if check_tree:
        _tree_levels_match(layer, tree, w, L, 2e-6)
    rows = [(i, h) for i in range(B) for h in range(w.n_q)]
    rep = P.check_rows(tree, Q.astype(np.float64), rows, lambda i: L, k, w.rope_base,
                       w.softmax_scale, out_t, dbg, w.n_q // w.n_kv, w.dtype)
    _say(rep)
    return layer, tree, out_t, dbg, Q


def test_tiny_f32_tree_and_decode():
    _decode_case(synth.WORKLOADS["tiny_f32_4k"], 8)


def test_tiny_f32_dense_special_case():
    """k = N_1 = 256 keeps every candidate: the GPU result is dense attention."""
    w = synth.WORKLOADS["tiny_f32_4k"]
    layer, tree, out_t, dbg, Q = _decode_case(w, 8, k=256, check_tree=False)
    out = P.to_host(out_t)
    K, V = synth.gen_kv(w)
    for i in range(8):
        ref = O.dense(Q[i, 0], K[0], V[0], w.L, w.rope_base, w.softmax_scale)
        assert np.abs(out[i, 0] - ref).max() <= 1e-5
    assert np.all(dbg["n_keys"].cpu().numpy() == 1 + 16 + 256 + 4096)


@pytest.mark.parametrize("L,b,k", [(4229, 16, 4), (2000, 3, 2), (3001, 5, 3), (1, 16, 4),
                                   (15, 16, 4), (256, 16, 4), (4095, 16, 1), (700, 7, 9)])
def test_f32_ragged_and_degenerate(L, b, k):
    w = synth.scaled(synth.WORKLOADS["tiny_f32_4k"], L, b=b, k=k)
    _decode_case(w, 8)


def test_bf16_out_dtype():
    w = synth.scaled(synth.WORKLOADS["qwen3_4b_131k"], 8192)
    layer, tree, out32, dbg, Q = _decode_case(w, 2)
    out16 = layer.decode(P.to_device(Q, w.dtype), out=None)
    p16 = P.make_layer(w, capacity=w.L, out="bf16")
    p16.k_cache.copy_(layer.k_cache)
    p16.v_cache.copy_(layer.v_cache)
    p16.pool_w.copy_(layer.pool_w)
    p16.build(w.L)
    o16 = p16.decode(P.to_device(Q, w.dtype))
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, out16.to(torch.bfloat16))


def test_bf16_decode_needles_small():
    """131K recipe at 32K tokens: parity, and needle reach equal on both sides."""
    w = synth.scaled(synth.WORKLOADS["qwen3_4b_131k"], 32768)
    layer, tree, out_t, dbg, Q = _decode_case(w, 8)
    sel = dbg["selected"].cpu().numpy()
    for (j, pos, g, qi, qh) in synth.needle_pairs(w):
        res = O.descend(tree, Q[qi, qh], g, w.L, w.k, w.rope_base, w.softmax_scale)
        r = qi * w.n_q + qh
        assert sel[r, 0, :w.k].tolist() == res.selected_nodes(1).tolist()


@pytest.mark.parametrize("chunks", [[1, 31, 32, 1000, 3], [4096], [0, 5000]])
def test_append_equals_build(chunks):
    """Appending in chunks gives the tree of a whole build, bit for bit, and every node
    the appends created equals the oracle's incremental extension of its tree (within
    the bf16 rounding bound of the build check)."""
    w = synth.scaled(synth.WORKLOADS["qwen3_4b_524k"], 8192, prefill_n=sum(chunks))
    L0, Lt = w.L, w.L + sum(chunks)
    K, V = synth.gen_kv(w, 0, Lt)
    W = synth.pool_w(w)
    full = P.make_layer(w, capacity=Lt)
    P.load_cache(full, K, V, W, Lt, w.dtype)
    full.build(Lt)
    inc = P.make_layer(w, capacity=Lt)
    P.load_cache(inc, K, V, W, L0, w.dtype)
    inc.build(L0)
    tree = O.build_tree(K, V, W, w.b, w.dtype, w.pool_scale, L0)
    at = L0
    for n in chunks:
        kn = P.to_device(np.ascontiguousarray(K[:, at:at + n].transpose(1, 0, 2)), w.dtype)
        vn = P.to_device(np.ascontiguousarray(V[:, at:at + n].transpose(1, 0, 2)), w.dtype)
        inc.append(kn, vn)
        at += n
        tree = O.extend_tree(tree, K, V, at)
    torch.cuda.synchronize()
    assert inc.length == Lt
    assert torch.equal(inc.k_cache, full.k_cache) and torch.equal(inc.v_cache, full.v_cache)
    for l in range(1, full.n_levels + 1):
        n = Lt // w.b ** l
        fk, fv = full.level(l)
        ik, iv = inc.level(l)
        assert torch.equal(fk[:, :n], ik[:, :n]) and torch.equal(fv[:, :n], iv[:, :n]), l
    # the appended nodes (those past the build's) against the oracle's extension
    new_nodes = 0
    for l in range(1, len(tree.keys)):
        n0 = L0 // w.b ** l
        n1 = Lt // w.b ** l
        ik, iv = inc.level(l)
        for g in range(w.n_kv):
            _bf16_close(P.to_host(ik[g, n0:n1]), tree.keys[l][g][n0:n1], (l, g, "key"))
            _bf16_close(P.to_host(iv[g, n0:n1]), tree.vals[l][g][n0:n1], (l, g, "value"))
        new_nodes += n1 - n0
    _say(f"appended nodes checked against the oracle: {new_nodes} per KV head")
    assert new_nodes > 0


PREFILL_CASES = [
    ("qwen3_4b_524k", 16384, 512, {}),
    ("qwen3_4b_1m_drift", 8192, 300, {}),
    # contexts 901..1200 cross b^2 = 1024: rows of one chunk have different top levels
    ("qwen3_4b_524k", 900, 300, {}),
    # head_dim 64 in bf16, b = 16, k = 4, one head: 300 rows
    ("tiny_f32_4k", 4000, 300, {"dtype": "bf16"}),
    ("tiny_f32_4k", 4000, 96, {}),
    # fanout 3 over 78K tokens: 26,067 token-level parents, past the LDS histogram's
    # 24,576, so the parent-major path counts pairs per range of parents instead
    ("tiny_f32_4k", 78000, 200, {"dtype": "bf16", "b": 3, "k": 4}),
]


@pytest.mark.parametrize("path", ["parent_major", "rowwise"])
@pytest.mark.parametrize("name,L,n,kw", PREFILL_CASES)
def test_prefill_small(name, L, n, kw, path):
    """Causal prefill against the oracle, parent-major (bf16 MFMA, the default for
    large bf16 chunks) and one workgroup per row (fp32 storage always runs this way:
    asking it for the parent-major layout is refused)."""
    w = synth.scaled(synth.WORKLOADS[name], L, prefill_n=n, **kw)
    if path == "parent_major" and w.dtype == "f32":
        layer = P.make_layer(w, capacity=L + n)
        layer.set_path(path)
        layer.build(1)
        with pytest.raises(R.RecsaError) as e:
            layer.prefill(P.to_device(synth.prefill_queries(w, 1), w.dtype))
        assert e.value.status == R.RECSA_ERR_UNSUPPORTED
        return
    _say(f"case prefill {name} L={L} n={n} {kw} path={path}")
    Lt = L + n
    K, V = synth.gen_kv(w, 0, Lt)
    W = synth.pool_w(w)
    Q = synth.prefill_queries(w, n)
    layer = P.make_layer(w, capacity=Lt)
    layer.set_path(path)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    layer.append(P.to_device(np.ascontiguousarray(K[:, L:].transpose(1, 0, 2)), w.dtype),
                 P.to_device(np.ascontiguousarray(V[:, L:].transpose(1, 0, 2)), w.dtype))
    out_t, dbg = layer.prefill(P.to_device(Q, w.dtype), debug=True)
    torch.cuda.synchronize()
    tree = O.build_tree(K, V, W, w.b, w.dtype, w.pool_scale, Lt)
    rng = np.random.default_rng(5)
    qs = sorted(set(rng.choice(n, size=min(n, 24), replace=False).tolist()) | {0, n - 1})
    rows = [(j, h) for j in qs for h in range(w.n_q)]
    rep = P.check_rows(tree, Q.astype(np.float64), rows, lambda j: L + j + 1, w.k, w.rope_base,
                       w.softmax_scale, out_t, dbg, w.n_q // w.n_kv, w.dtype)
    _say(rep)


def test_full_131k_decode():
    """The 131K-token Qwen3-4B-shaped workload at full size: build, decode B=1 and B=8."""
    w = synth.WORKLOADS["qwen3_4b_131k"]
    layer, tree, out_t, dbg, Q = _decode_case(w, 8, check_tree=True)
    out1, dbg1 = layer.decode(P.to_device(Q[:1], w.dtype), debug=True)
    torch.cuda.synchronize()
    P.assert_same_query(out1[0], dbg1, out_t[0], dbg, slice(0, w.n_q), slice(0, w.n_q))
