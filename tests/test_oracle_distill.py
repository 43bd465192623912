"""Pins of the oracle's pooler distillation (fit w so that RecSA's output
matches dense attention's): the loss gradient in w against central finite
differences through the tree rebuild, a zero loss where RecSA is dense
attention, and descent of the loss under small steps."""
import math

import numpy as np
import pytest

import synth
from oracle import recsa as O


def _setup(seed, L, d, n_kv, nq, B, wscale=2.0):
    r = np.random.default_rng(seed)
    K = r.standard_normal((n_kv, L, d))
    V = r.standard_normal((n_kv, L, d))
    w = r.standard_normal((n_kv, d)) * wscale / math.sqrt(d)
    Q = r.standard_normal((B, nq, d)) * 1.5
    return K, V, w, Q


def _teacher(K, V, Q, L, base, s):
    B, nq, d = Q.shape
    G = nq // K.shape[0]
    return np.stack([np.stack([O.dense(Q[i, h], K[h // G], V[h // G], L, base, s) for h in range(nq)])
                     for i in range(B)])


@pytest.mark.parametrize("L,b,k", [(47, 3, 2), (70, 4, 2)])
def test_distill_gradient_matches_finite_differences(L, b, k):
    d, base, s, ps = 4, 1e4, 0.6, 0.7
    K, V, w, Q = _setup(L, L, d, 1, 2, 2)
    T = _teacher(K, V, Q, L, base, s)
    tree = O.build_tree(K, V, w, b, "f64", ps, L)
    force = {}
    for i in range(2):
        for h in range(2):
            r = O.descend(tree, Q[i, h], 0, L, k, base, s)
            assert all(not np.isfinite(t.gap) or t.gap > 1e-6 for t in r.levels)
            force[(i, h)] = {t.level: t.cand[t.sel_pos] for t in r.levels if t.level > 0}
    loss, g = O.distill_loss(tree, Q, T, k, base, s, force=force)
    assert loss > 0
    h = 1e-6
    for idx in np.ndindex(w.shape):
        wp, wm = w.copy(), w.copy()
        wp[idx] += h
        wm[idx] -= h
        lp, _ = O.distill_loss(O.build_tree(K, V, wp, b, "f64", ps, L), Q, T, k, base, s, force=force)
        lm, _ = O.distill_loss(O.build_tree(K, V, wm, b, "f64", ps, L), Q, T, k, base, s, force=force)
        fd = (lp - lm) / (2 * h)
        assert abs(fd - g["dw"][idx]) <= 1e-6 * (1 + abs(fd)), (idx, fd, g["dw"][idx])


def test_distill_loss_is_zero_where_recsa_is_dense():
    L, d, b = 200, 8, 16
    K, V, w, Q = _setup(3, L, d, 1, 2, 2)
    T = _teacher(K, V, Q, L, 1e4, 0.35)
    loss, g = O.distill_loss(O.build_tree(K, V, w, b, "f32", 0.5, L), Q, T, L, 1e4, 0.35)
    assert loss < 1e-20 and np.all(np.abs(g["dw"]) < 1e-15)


def test_distill_small_steps_descend():
    """Gradient steps with a small rate lower the loss (tiny workload shape)."""
    w0 = synth.scaled(synth.WORKLOADS["tiny_f32_4k"], 1024, n_q=2)
    K, V = synth.gen_kv(w0)
    W = synth.pool_w(w0) * 8.0
    Q = synth.decode_queries(w0, 4)
    T = _teacher(K, V, Q, w0.L, w0.rope_base, w0.softmax_scale)
    vel = np.zeros_like(W)
    losses = []
    for _ in range(4):
        loss, W, vel = O.distill_step(K, V, W, w0.b, "f64", w0.pool_scale, w0.L, Q, T, w0.k,
                                      w0.rope_base, w0.softmax_scale, lr=0.5, mu=0.0, vel=vel)
        losses.append(loss)
    assert all(b_ < a_ for a_, b_ in zip(losses, losses[1:])), losses


def test_golden_momentum_update():
    """The update rule against a hand-worked two-step example (tests/golden/
    momentum_two_steps.json): heavy-ball momentum, velocity first, no dampening."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "momentum_two_steps.json")))
    w, v = np.array(g["w0"]), np.array(g["v0"])
    for grad, ev, ew in zip(g["grads"], g["expected_v"], g["expected_w"]):
        w, v = O.sgd_momentum(w, v, np.array(grad), g["lr"], g["mu"])
        np.testing.assert_allclose(v, ev, rtol=0, atol=1e-15)
        np.testing.assert_allclose(w, ew, rtol=0, atol=1e-15)


def test_distill_two_momentum_steps_follow_finite_differences():
    """Two steps with momentum 0.9: the velocity after step 1 is the loss gradient at
    w0 and after step 2 is 0.9 of it plus the gradient at w1, each gradient taken by
    central differences of the loss through the tree rebuild (selection held at the
    row's own selection, checked to be away from ties); w moves by -lr times the new
    velocity."""
    L, b, k, d, base, s, ps = 70, 4, 2, 4, 1e4, 0.6, 0.7
    K, V, w0, Q = _setup(11, L, d, 1, 2, 2)
    T = _teacher(K, V, Q, L, base, s)
    lr, mu = 0.05, 0.9

    def held(w):
        tree = O.build_tree(K, V, w, b, "f64", ps, L)
        force = {}
        for i in range(2):
            for h in range(2):
                r = O.descend(tree, Q[i, h], 0, L, k, base, s)
                assert all(not np.isfinite(t.gap) or t.gap > 1e-6 for t in r.levels)
                force[(i, h)] = {t.level: t.cand[t.sel_pos] for t in r.levels if t.level > 0}
        return force

    def fd_grad(w, force, h=1e-6):
        gr = np.zeros_like(w)
        for idx in np.ndindex(w.shape):
            wp, wm = w.copy(), w.copy()
            wp[idx] += h
            wm[idx] -= h
            lp, _ = O.distill_loss(O.build_tree(K, V, wp, b, "f64", ps, L), Q, T, k, base, s, force=force)
            lm, _ = O.distill_loss(O.build_tree(K, V, wm, b, "f64", ps, L), Q, T, k, base, s, force=force)
            gr[idx] = (lp - lm) / (2 * h)
        return gr

    vel = np.zeros_like(w0)
    f0 = held(w0)
    _, w1, v1 = O.distill_step(K, V, w0, b, "f64", ps, L, Q, T, k, base, s, lr, mu, vel, force=f0)
    g0 = fd_grad(w0, f0)
    np.testing.assert_allclose(v1, g0, rtol=0, atol=1e-6 * (1 + np.abs(g0).max()))
    np.testing.assert_allclose(w1, w0 - lr * v1, rtol=0, atol=1e-14)
    f1 = held(w1)
    _, w2, v2 = O.distill_step(K, V, w1, b, "f64", ps, L, Q, T, k, base, s, lr, mu, v1, force=f1)
    g1 = fd_grad(w1, f1)
    np.testing.assert_allclose(v2, mu * g0 + g1, rtol=0, atol=2e-6 * (1 + np.abs(g1).max()))
    np.testing.assert_allclose(w2, w1 - lr * v2, rtol=0, atol=1e-14)
    assert np.abs(mu * v1).max() > 1e-3     # the momentum term is not negligible
