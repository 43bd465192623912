"""Pins of the oracle's backward pass (selection held fixed) against what the
mathematics fixes: central finite differences of the pinned forward oracle,
torch autograd of dense attention in the case where RecSA is dense attention,
and the conservation of the value gradient."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import recsa as O


def _inputs(seed, L, d, n_kv, nq, nrow):
    r = np.random.default_rng(seed)
    K = r.standard_normal((n_kv, L, d))
    V = r.standard_normal((n_kv, L, d))
    w = r.standard_normal((n_kv, d)) * 2.0 / math.sqrt(d)
    Q = r.standard_normal((nrow, nq, d)) * 1.5
    dO = r.standard_normal((nrow, nq, d))
    return K, V, w, Q, dO


def _loss(K, V, w, Q, dO, b, k, causal, force, ps=0.7, base=1e4, s=0.6):
    tree = O.build_tree(K, V, w, b, "f64", ps, K.shape[1])
    n, nq, _ = Q.shape
    G = nq // K.shape[0]
    tot = 0.0
    for i in range(n):
        for h in range(nq):
            n_ctx = K.shape[1] - n + i + 1 if causal else K.shape[1]
            r = O.descend(tree, Q[i, h], h // G, n_ctx, k, base, s, force=force[(i, h)])
            tot += float(dO[i, h] @ r.out)
    return tot


def _selections(K, V, w, Q, b, k, causal, ps=0.7, base=1e4, s=0.6):
    tree = O.build_tree(K, V, w, b, "f64", ps, K.shape[1])
    n, nq, _ = Q.shape
    G = nq // K.shape[0]
    force = {}
    for i in range(n):
        for h in range(nq):
            n_ctx = K.shape[1] - n + i + 1 if causal else K.shape[1]
            r = O.descend(tree, Q[i, h], h // G, n_ctx, k, base, s)
            assert all(not np.isfinite(t.gap) or t.gap > 1e-6 for t in r.levels), "near-tie input"
            force[(i, h)] = {t.level: t.cand[t.sel_pos] for t in r.levels if t.level > 0}
    return tree, force


@pytest.mark.parametrize("L,b,k,causal", [(47, 3, 2, False), (40, 3, 1, True), (70, 4, 2, False)])
def test_backward_matches_finite_differences(L, b, k, causal):
    d, n_kv, nq, nrow = 4, 1, 2, 2
    K, V, w, Q, dO = _inputs(L + 3 * b, L, d, n_kv, nq, nrow)
    tree, force = _selections(K, V, w, Q, b, k, causal)
    g = O.backward(tree, Q, dO, k, 1e4, 0.6, causal=causal, force=force)
    h = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        up = _loss(K, V, w, Q, dO, b, k, causal, force)
        arr[idx] = old - h
        dn = _loss(K, V, w, Q, dO, b, k, causal, force)
        arr[idx] = old
        return (up - dn) / (2 * h)

    rng = np.random.default_rng(1)
    for name, arr, grad in (("dq", Q, g["dq"]), ("dw", w, g["dw"])):
        for idx in np.ndindex(arr.shape):
            assert abs(fd(arr, idx) - grad[idx]) <= 1e-6 * (1 + abs(grad[idx])), (name, idx)
    # every token's value and key, a sample of the coordinates
    for name, arr, grad in (("dv", V, g["dv"]), ("dk", K, g["dk"])):
        for t in range(L):
            c = int(rng.integers(d))
            idx = (0, t, c)
            assert abs(fd(arr, idx) - grad[idx]) <= 1e-6 * (1 + abs(grad[idx])), (name, idx)


def _rot(x, pos, base, d):
    h = d // 2
    theta = base ** (-2.0 * torch.arange(h, dtype=torch.float64) / d)
    a = pos[:, None].double() * theta[None, :]
    c, sn = torch.cos(a), torch.sin(a)
    return torch.cat([x[:, :h] * c - x[:, h:] * sn, x[:, h:] * c + x[:, :h] * sn], -1)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_dense_case_is_sdpa_autograd(causal):
    """k >= every candidate count: nothing is summarized, the tree carries no
    gradient (dw = 0) and the gradients are those of dense attention (torch
    autograd through scaled_dot_product_attention, float64)."""
    L, d, b, base, s = 200, 8, 16, 1e4, 0.35
    K, V, w, Q, dO = _inputs(5, L, d, 1, 1, 3)
    tree = O.build_tree(K, V, w, b, "f32", 0.5, L)
    g = O.backward(tree, Q, dO, L, base, s, causal=causal)
    assert np.all(g["dw"] == 0)
    Kt = torch.tensor(K[0], requires_grad=True)
    Vt = torch.tensor(V[0], requires_grad=True)
    Qt = torch.tensor(Q[:, 0], requires_grad=True)
    tot = 0
    for i in range(3):
        n = L - 3 + i + 1 if causal else L
        kr = _rot(Kt[:n], torch.arange(n), base, d)
        qr = _rot(Qt[i:i + 1], torch.tensor([n]), base, d)
        out = torch.nn.functional.scaled_dot_product_attention(qr[None, None], kr[None, None],
                                                               Vt[:n][None, None], scale=s)
        tot = tot + (out[0, 0, 0] * torch.tensor(dO[i, 0])).sum()
    tot.backward()
    np.testing.assert_allclose(g["dq"][:, 0], Qt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(g["dk"][0], Kt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(g["dv"][0], Vt.grad.numpy(), atol=1e-10)


def test_backward_value_gradient_is_conserved():
    """Every row's softmax weights sum to 1 and a summary's value is the plain
    mean of its tokens, so the token value gradients of a KV head sum to the sum
    of dO over the rows that read it."""
    w = synth.WORKLOADS["tiny_f32_4k"]
    K, V = synth.gen_kv(w)
    W = synth.pool_w(w)
    tree = O.build_tree(K, V, W, w.b, "f32", w.pool_scale, w.L)
    Q = synth.decode_queries(w, 3)
    dO = np.random.default_rng(2).standard_normal(Q.shape)
    g = O.backward(tree, Q, dO, w.k, w.rope_base, w.softmax_scale)
    np.testing.assert_allclose(g["dv"][0].sum(axis=0), dO[:, 0].sum(axis=0), atol=1e-12)
    assert np.any(g["dw"] != 0)
