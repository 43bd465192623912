"""GPU parity over a seeded sweep of small random configurations: fanout, budget,
context length, head dim, storage, KV heads and group size drawn at random (fixed
seed), each call of the path checked against the oracle on the same inputs:
decode, grouped decode, causal prefill (row-wise, and parent-major for bf16
storage), and the backward (the same two layouts, and with bf16 token gradients for bf16
storage and fanouts up to 32).  The shapes reach what the fixed cases do
not: fanouts from 2 (deep trees) to 47, budgets from 1 to 9 (levels where every
candidate is kept), contexts shorter than one node, odd head groupings."""
import numpy as np
import pytest
import torch

import synth
from oracle import recsa as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _configs(n=30, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        base = "tiny_f32_4k" if i % 2 == 0 else "qwen3_4b_131k"
        out.append(dict(
            idx=i, base=base,
            dtype="f32" if rng.random() < 0.4 else "bf16",
            b=int(rng.integers(2, 48)),
            k=int(rng.integers(1, 10)),
            n_kv=int(rng.integers(1, 3)),
            G=int(rng.choice([1, 2, 4])),
            L=int(rng.integers(1, 2500)),
            B=int(rng.integers(1, 4)),
            nP=int(rng.integers(1, 13)),
        ))
    return out


# and three edges the draws miss: fanout 2 (nine levels), a context shorter than one
# node, a budget that keeps every candidate (dense) with groups of eight heads
CONFIGS = _configs() + [
    dict(idx=30, base="tiny_f32_4k", dtype="bf16", b=2, k=3, n_kv=1, G=2, L=700, B=2, nP=6),
    dict(idx=31, base="qwen3_4b_131k", dtype="bf16", b=13, k=4, n_kv=2, G=2, L=5, B=2, nP=5),
    dict(idx=32, base="tiny_f32_4k", dtype="f32", b=4, k=12, n_kv=1, G=8, L=200, B=2, nP=9),
]


def _tol(ref, dtype):
    if dtype == "f32":
        return 1e-5 * max(1.0, float(np.abs(ref).max()))
    return 2e-2 * float(np.sqrt(np.mean(ref ** 2))) + 1e-12


@pytest.mark.parametrize("c", CONFIGS, ids=[f"cfg{c['idx']}" for c in CONFIGS])
def test_sweep(c):
    L = c["L"]
    nP = min(c["nP"], L)
    w = synth.scaled(synth.WORKLOADS[c["base"]], L, prefill_n=0, n_kv=c["n_kv"],
                     n_q=c["n_kv"] * c["G"], b=c["b"], k=c["k"], dtype=c["dtype"], needles=0)
    _say(f"case sweep {c}")
    K, V = synth.gen_kv(w, 0, L)
    W = synth.pool_w(w)
    layer = P.make_layer(w, capacity=L)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    tree = O.build_tree(K, V, W, w.b, w.dtype, w.pool_scale, L)
    trees = {g: P.head_tree(K, V, W, g, w, L) for g in range(w.n_kv)}
    rng = np.random.default_rng(1000 + c["idx"])
    G = w.n_q // w.n_kv

    # decode
    Qd = synth.to_storage(rng.standard_normal((c["B"], w.n_q, w.d)).astype(np.float32), w.dtype)
    out, dbg = layer.decode(P.to_device(Qd, w.dtype), debug=True)
    torch.cuda.synchronize()
    rows = [(i, h) for i in range(c["B"]) for h in range(w.n_q)]
    rep = P.check_rows(tree, Qd.astype(np.float64), rows, lambda i: L, w.k, w.rope_base,
                       w.softmax_scale, out, dbg, G, w.dtype)
    _say("decode", rep)

    # grouped decode (one selection per query and KV group)
    out_g, dbg_g = layer.decode_grouped(P.to_device(Qd, w.dtype), debug=True)
    torch.cuda.synchronize()
    rep = P.check_groups(trees, Qd.astype(np.float64), [(i, g) for i in range(c["B"]) for g in range(w.n_kv)],
                         lambda i: L, w.k, w.rope_base, w.softmax_scale, out_g, dbg_g, w.n_kv, w.dtype)
    _say("grouped", rep)

    # causal prefill of the last nP tokens' queries, both paths
    Qp = synth.to_storage(rng.standard_normal((nP, w.n_q, w.d)).astype(np.float32), w.dtype)
    rows = [(j, h) for j in range(nP) for h in range(w.n_q)]
    paths = ("rowwise", "parent_major") if w.dtype == "bf16" else ("rowwise",)
    for path in paths:
        layer.set_path(path)
        out_p, dbg_p = layer.prefill(P.to_device(Qp, w.dtype), debug=True)
        torch.cuda.synchronize()
        rep = P.check_rows(tree, Qp.astype(np.float64), rows, lambda j: L - nP + j + 1, w.k, w.rope_base,
                           w.softmax_scale, out_p, dbg_p, G, w.dtype)
        _say("prefill", path, rep)

    # backward, decode-shaped and causal, both paths, on the GPU's selections
    for causal, n in ((False, c["B"]), (True, nP)):
        Q = Qd if not causal else Qp
        dO = rng.standard_normal((n, w.n_q, w.d)).astype(np.float32)
        for path in paths:
            layer.set_path(path)
            grads, bdbg = layer.backward(P.to_device(Q, w.dtype), torch.from_numpy(dO).cuda(), causal=causal,
                                         debug=True)
            torch.cuda.synchronize()
            sel = bdbg["selected"].cpu().numpy()
            force = {}
            for i in range(n):
                n_ctx = L - n + i + 1 if causal else L
                N = O.level_sizes(n_ctx, w.b)
                for h in range(w.n_q):
                    P.check_row(trees[h // G], Q[i, h].astype(np.float64), 0, n_ctx, w.k, w.rope_base,
                                w.softmax_scale, sel[i * w.n_q + h])
                    force[(i, h)] = {l: sel[i * w.n_q + h, l - 1][sel[i * w.n_q + h, l - 1] >= 0]
                                     for l in range(1, len(N))}
            ref = O.backward(tree, Q.astype(np.float64), dO.astype(np.float64), w.k, w.rope_base,
                             w.softmax_scale, causal=causal, force=force)
            got = {k_: v.cpu().numpy().astype(np.float64) for k_, v in grads.items()}
            for key in ("dq", "dk", "dv", "dw"):
                g_ = got[key] if key in ("dq", "dw") else got[key][:, :L]
                err = float(np.abs(g_ - ref[key]).max())
                tol = _tol(ref[key], w.dtype)
                assert err <= tol, f"backward {path} causal={causal} {key}: {err:.3g} > {tol:.3g}"
            _say("backward", path, "causal" if causal else "decode", "ok")
            if path == "parent_major" and w.b <= 32:
                # bf16 token gradients: the same forward (same selections), each token's
                # gradient rounded once, so within 2^-8 of it beyond the fp32 bar
                g16, d16 = layer.backward(P.to_device(Q, w.dtype), torch.from_numpy(dO).cuda(), causal=causal,
                                          debug=True, grad_dtype="bf16")
                torch.cuda.synchronize()
                assert np.array_equal(d16["selected"].cpu().numpy(), sel), "bf16-gradient run selected differently"
                for key in ("dq", "dk", "dv", "dw"):
                    g_ = g16[key].float().cpu().numpy().astype(np.float64)
                    g_ = g_ if key in ("dq", "dw") else g_[:, :L]
                    slack = 2.0 ** -8 * np.abs(ref[key]) if key in ("dk", "dv") else 0.0
                    over = float((np.abs(g_ - ref[key]) - slack).max())
                    tol = _tol(ref[key], w.dtype)
                    assert over <= tol, f"backward bf16 causal={causal} {key}: {over:.3g} > {tol:.3g}"
                _say("backward bf16 grads", "causal" if causal else "decode", "ok")
