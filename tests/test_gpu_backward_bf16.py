"""GPU parity of recsa_backward_bf16 (token gradients in bf16) against recsa_backward's
fp32 gradients on the same seeded inputs and the same (parent-major) path, and against
the oracle's backward on the GPU's selections.

Bars, per element of dk and dv over tokens [0, L):
  against the fp32 path: |bf16 - fp32| <= 2^-8 |fp32| + 1e-5 max(1, max |fp32|)
    (round to nearest bf16 moves a value by at most half its unit in the last place,
    2^-8 of it; the second term is the fp32 summation-order difference between the two
    calls, whose atomics and pair orders differ);
  against the oracle: 2^-8 |oracle| plus the fp32 path's own bar (2e-2 x RMS for bf16
  storage).
dq and dw are fp32 in both calls and must agree to 1e-5 of their largest magnitude."""
import numpy as np
import pytest
import torch

import synth
from oracle import recsa as O
from tests import parity as P

pytestmark = pytest.mark.gpu

BF16_REL = 2.0 ** -8


def _say(*a):
    print(*a, flush=True)


CASES = [
    # (workload, L, n_kv, n_q, n rows, causal, overrides)
    ("tiny_f32_4k", 300, 1, 2, 2, False, {"dtype": "bf16"}),
    ("tiny_f32_4k", 10, 1, 2, 4, True, {"dtype": "bf16"}),                  # L < b: tokens only
    ("tiny_f32_4k", 3001, 1, 2, 24, True, {"b": 5, "k": 3, "dtype": "bf16"}),  # odd fanout, orphans
    ("tiny_f32_4k", 4229, 2, 4, 40, True, {"dtype": "bf16"}),               # GQA, ragged tail
    ("tiny_f32_4k", 2000, 1, 2, 64, False, {"dtype": "bf16", "b": 32}),      # buckets over several items
    ("qwen3_4b_131k", 20000, 8, 32, 2, False, {}),
    ("qwen3_4b_131k", 9000, 8, 32, 3, True, {}),
]


def _setup(w, L, cap=None):
    K, V = synth.gen_kv(w, 0, L)
    W = synth.pool_w(w)
    layer = P.make_layer(w, capacity=cap or L)
    layer.set_path("parent_major")
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    return layer, K, V, W


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_vs_f32(g16, g32, L):
    rep = {}
    for key in ("dk", "dv"):
        x, y = _host(g16[key])[:, :L], _host(g32[key])[:, :L]
        bound = BF16_REL * np.abs(y) + 1e-5 * max(1.0, float(np.abs(y).max()))
        over = np.abs(x - y) - bound
        worst = float(over.max()) if over.size else -1.0
        assert worst <= 0, f"{key}: bf16 vs fp32 exceeds 2^-8 |x| + 1e-5 max by {worst:.3g}"
        rep[key] = float(np.abs(x - y).max())
    for key in ("dq", "dw"):
        x, y = _host(g16[key]), _host(g32[key])
        tol = 1e-5 * max(1.0, float(np.abs(y).max()))
        err = float(np.abs(x - y).max())
        assert err <= tol, f"{key}: {err:.3g} > {tol:.3g}"
        rep[key] = err
    return rep


@pytest.mark.parametrize("name,L,n_kv,n_q,n,causal,kw", CASES)
def test_backward_bf16(name, L, n_kv, n_q, n, causal, kw):
    _say(f"case backward bf16 {name} L={L} n_kv={n_kv} n_q={n_q} n={n} causal={causal} {kw}")
    w = synth.scaled(synth.WORKLOADS[name], L, prefill_n=0, n_kv=n_kv, n_q=n_q, **kw)
    cap = L + 50
    layer, K, V, W = _setup(w, L, cap)
    rng = np.random.default_rng(L + 7 * n)
    Q = synth.to_storage(rng.standard_normal((n, n_q, w.d)).astype(np.float32), w.dtype)
    dO = rng.standard_normal((n, n_q, w.d)).astype(np.float32)
    q, dOd = P.to_device(Q, w.dtype), torch.from_numpy(dO).cuda()
    g32 = layer.backward(q, dOd, causal=causal)
    # bf16 buffers that held other values: rows [0, L) are written, the rest kept
    junk = {"dk": torch.full((n_kv, cap, w.d), 7.5, dtype=torch.bfloat16, device="cuda"),
            "dv": torch.full((n_kv, cap, w.d), -7.5, dtype=torch.bfloat16, device="cuda"),
            "dw": torch.full((n_kv, w.d), 3.0, dtype=torch.float32, device="cuda")}
    g16, dbg = layer.backward(q, dOd, causal=causal, debug=True, grads=junk, grad_dtype="bf16")
    torch.cuda.synchronize()
    assert g16["dk"].dtype == torch.bfloat16 and g16["dv"].dtype == torch.bfloat16
    assert torch.all(g16["dk"][:, L:] == 7.5) and torch.all(g16["dv"][:, L:] == -7.5)
    rep = _check_vs_f32(g16, g32, L)
    # against the oracle on the GPU's selections (each checked against the oracle's own)
    sel = dbg["selected"].cpu().numpy()
    G = n_q // n_kv
    trees = [P.head_tree(K, V, W, g, w, L) for g in range(n_kv)]
    force = {}
    for i in range(n):
        n_ctx = L - n + i + 1 if causal else L
        for h in range(n_q):
            r = i * n_q + h
            P.check_row(trees[h // G], Q[i, h].astype(np.float64), 0, n_ctx, w.k, w.rope_base,
                        w.softmax_scale, sel[r])
            N = O.level_sizes(n_ctx, w.b)
            force[(i, h)] = {l: sel[r, l - 1][sel[r, l - 1] >= 0] for l in range(1, len(N))}
    tree = O.build_tree(K[:, :L], V[:, :L], W, w.b, w.dtype, w.pool_scale, L)
    ref = O.backward(tree, Q.astype(np.float64), dO.astype(np.float64), w.k, w.rope_base, w.softmax_scale,
                     causal=causal, force=force)
    for key in ("dk", "dv"):
        x, y = _host(g16[key])[:, :L], ref[key]
        bar = 2e-2 * float(np.sqrt(np.mean(y ** 2))) + 1e-12
        over = np.abs(x - y) - (BF16_REL * np.abs(y) + bar)
        assert float(over.max()) <= 0, f"{key}: bf16 vs oracle exceeds its bar by {float(over.max()):.3g}"
    _say("bf16 vs fp32", {k: f"{v:.2e}" for k, v in rep.items()})


def test_backward_bf16_decode_batch_524k():
    """The Qwen3-4B layer at 524288 tokens, the 16-query decode batch (512 rows): bf16
    token gradients against the fp32 ones of the same path."""
    w = synth.WORKLOADS["qwen3_4b_524k"]
    L, n = w.L, 16
    _say(f"case backward bf16 decode batch qwen3_4b_524k L={L} n={n}")
    layer, _, _, _ = _setup(w, L)
    q = P.to_device(synth.decode_queries(w, n), w.dtype)
    rng = np.random.default_rng(5)
    dO = torch.from_numpy(rng.standard_normal((n, w.n_q, w.d)).astype(np.float32)).cuda()
    g32 = layer.backward(q, dO)
    g16 = layer.backward(q, dO, grad_dtype="bf16")
    torch.cuda.synchronize()
    rep = _check_vs_f32(g16, g32, L)
    _say("bf16 vs fp32", {k: f"{v:.2e}" for k, v in rep.items()})


@pytest.mark.parametrize("what", ["f32_storage", "fanout_40", "rowwise_path"])
def test_backward_bf16_unsupported(what):
    """Where the bf16 token gradients do not run, the call fails with an error and
    writes nothing."""
    kw = {"f32_storage": {}, "fanout_40": {"dtype": "bf16", "b": 40}, "rowwise_path": {"dtype": "bf16"}}[what]
    L = 500
    w = synth.scaled(synth.WORKLOADS["tiny_f32_4k"], L, prefill_n=0, n_q=2, **kw)
    layer, _, _, _ = _setup(w, L)
    layer.set_path("rowwise" if what == "rowwise_path" else "auto")
    rng = np.random.default_rng(3)
    q = P.to_device(synth.to_storage(rng.standard_normal((2, 2, w.d)).astype(np.float32), w.dtype), w.dtype)
    dO = torch.from_numpy(rng.standard_normal((2, 2, w.d)).astype(np.float32)).cuda()
    junk = {"dk": torch.full((1, L, w.d), 1.5, dtype=torch.bfloat16, device="cuda"),
            "dv": torch.full((1, L, w.d), 1.5, dtype=torch.bfloat16, device="cuda"),
            "dw": torch.full((1, w.d), 1.5, dtype=torch.float32, device="cuda")}
    with pytest.raises(RuntimeError, match="bf16 token gradients"):
        layer.backward(q, dO, grads=junk, grad_dtype="bf16")
    torch.cuda.synchronize()
    assert all(torch.all(junk[k] == 1.5) for k in ("dk", "dv", "dw"))
