"""GPU parity of the pooler distillation pieces against the oracle on the same
seeded inputs: the dense-attention teacher (recsa_dense_decode, vs the oracle's
dense attention, pinned to torch SDPA), and distillation steps (loss, updated
pooler vectors and velocity) against the oracle's step on the GPU's selections.
Tolerances as for outputs: 1e-5 max-abs (fp32 storage), 2e-2 x RMS (bf16)."""
import numpy as np
import pytest
import torch

import synth
from oracle import recsa as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _layer(name, L, n_kv, n_q, kw=None, wscale=1.0):
    w = synth.scaled(synth.WORKLOADS[name], L, prefill_n=0, n_kv=n_kv, n_q=n_q, **(kw or {}))
    K, V = synth.gen_kv(w, 0, L)
    W = synth.pool_w(w) * wscale
    layer = P.make_layer(w, capacity=L)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    return w, K, V, W, layer


@pytest.mark.parametrize("name,L,n_kv,n_q,kw", [
    ("tiny_f32_4k", 4096, 1, 2, {}),
    ("tiny_f32_4k", 3001, 2, 4, {"b": 5}),
    ("tiny_f32_4k", 37, 1, 1, {}),
    ("qwen3_4b_131k", 40961, 8, 32, {}),
    ("tiny_f32_4k", 3001, 2, 4, {"dtype": "bf16"}),            # bf16 MFMA path at d = 64
    ("qwen3_4b_131k", 5000, 1, 32, {}),                        # 96 rows per KV head: two row tiles
])
def test_dense_decode(name, L, n_kv, n_q, kw):
    _say(f"case dense {name} L={L} n_kv={n_kv} n_q={n_q}")
    w, K, V, W, layer = _layer(name, L, n_kv, n_q, kw)
    rng = np.random.default_rng(L)
    Q = synth.to_storage(rng.standard_normal((3, n_q, w.d)).astype(np.float32), w.dtype)
    out = P.to_host(layer.dense_decode(P.to_device(Q, w.dtype)))
    torch.cuda.synchronize()
    G = n_q // n_kv
    heads = range(n_q) if n_q <= 4 else [0, 5, 31]
    want = np.stack([np.stack([O.dense(Q[i, h].astype(np.float64), K[h // G], V[h // G], L, w.rope_base,
                                       w.softmax_scale) for h in heads]) for i in range(3)])
    got = out[:, list(heads)]
    err = float(np.abs(got - want).max())
    tol = 1e-5 if w.dtype == "f32" else 2e-2 * float(np.sqrt(np.mean(want ** 2)))
    _say("dense", err, tol)
    assert err <= tol


def test_distill_steps_follow_the_oracle():
    """Three steps at a small fanout: the GPU's loss, pooler vectors and velocity
    after each step against the oracle's steps from the same start."""
    w, K, V, W, layer = _layer("tiny_f32_4k", 2048, 1, 2, {"b": 8, "k": 2}, wscale=6.0)
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((4, 2, w.d)).astype(np.float32)
    q = P.to_device(Q, "f32")
    teacher = layer.dense_decode(q)
    torch.cuda.synchronize()
    T = teacher.cpu().numpy().astype(np.float64)
    vel = torch.zeros_like(layer.pool_w)
    loss = torch.zeros(1, dtype=torch.float32, device=layer.device)
    lr, mu = 0.5, 0.9
    Wo, velo = W.astype(np.float64), np.zeros_like(W, dtype=np.float64)
    for step in range(3):
        _, dbg = layer.decode(q, debug=True)
        torch.cuda.synchronize()
        sel = dbg["selected"].cpu().numpy()
        tree = O.build_tree(K, V, Wo, w.b, "f32", w.pool_scale, w.L)
        force = {}
        for i in range(4):
            for h in range(2):
                P.check_row(tree, Q[i, h].astype(np.float64), 0, w.L, w.k, w.rope_base, w.softmax_scale,
                            sel[i * 2 + h])
                N = O.level_sizes(w.L, w.b)
                force[(i, h)] = {l: sel[i * 2 + h, l - 1][sel[i * 2 + h, l - 1] >= 0] for l in range(1, len(N))}
        want_loss, Wo, velo = O.distill_step(K, V, Wo, w.b, "f32", w.pool_scale, w.L,
                                             Q.astype(np.float64), T, w.k, w.rope_base,
                                             w.softmax_scale, lr, mu, velo, force=force)
        layer.distill_step(q, teacher, lr, mu, vel, loss)
        torch.cuda.synchronize()
        got_loss = float(loss.item())
        _say(f"step {step}: loss gpu {got_loss:.7g} oracle {want_loss:.7g}")
        assert abs(got_loss - want_loss) <= 1e-5 * max(1.0, want_loss)
        np.testing.assert_allclose(vel.cpu().numpy(), velo, rtol=0, atol=1e-5 * max(1.0, np.abs(velo).max()))
        np.testing.assert_allclose(layer.pool_w.cpu().numpy(), Wo, rtol=0, atol=1e-5)
        # the tree was rebuilt from the new vectors
        keys, _ = layer.level(1)
        np.testing.assert_allclose(keys[0, :3].cpu().numpy(),
                                   O.build_tree(K, V, Wo, w.b, "f32", w.pool_scale, w.L).keys[1][0][:3],
                                   rtol=0, atol=1e-5)


def test_distill_bf16_step():
    """One step on the Qwen3-4B layer shape (bf16 storage): loss and the pooler
    gradient (velocity after one step from zero) against the oracle."""
    w, K, V, W, layer = _layer("qwen3_4b_131k", 8192, 8, 32)
    rng = np.random.default_rng(8)
    Q = synth.to_storage(rng.standard_normal((2, 32, w.d)).astype(np.float32), "bf16")
    q = P.to_device(Q, "bf16")
    teacher = layer.dense_decode(q)         # fp32 output (the test layers' out dtype)
    _, dbg = layer.decode(q, debug=True)
    torch.cuda.synchronize()
    T = teacher.cpu().numpy().astype(np.float64)
    sel = dbg["selected"].cpu().numpy()
    tree = O.build_tree(K, V, W, w.b, "bf16", w.pool_scale, w.L)
    force = {}
    head_trees = {g: P.head_tree(K, V, W, g, w, w.L) for g in range(8)}
    for i in range(2):
        for h in range(32):
            tg = head_trees[h // 4]
            P.check_row(tg, Q[i, h].astype(np.float64), 0, w.L, w.k, w.rope_base, w.softmax_scale, sel[i * 32 + h])
            N = O.level_sizes(w.L, w.b)
            force[(i, h)] = {l: sel[i * 32 + h, l - 1][sel[i * 32 + h, l - 1] >= 0] for l in range(1, len(N))}
    want_loss, g = O.distill_loss(tree, Q.astype(np.float64), T, w.k, w.rope_base, w.softmax_scale, force=force)
    vel = torch.zeros_like(layer.pool_w)
    loss = torch.zeros(1, dtype=torch.float32, device=layer.device)
    layer.distill_step(q, teacher, 0.1, 0.9, vel, loss)
    torch.cuda.synchronize()
    _say("bf16 step loss", float(loss.item()), want_loss)
    assert abs(float(loss.item()) - want_loss) <= 2e-2 * want_loss
    dw = vel.cpu().numpy()
    assert np.abs(dw - g["dw"]).max() <= 2e-2 * float(np.sqrt(np.mean(g["dw"] ** 2)))
