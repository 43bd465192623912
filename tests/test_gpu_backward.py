"""GPU parity of the backward pass (selection held fixed) against the oracle's
backward on the same seeded inputs: the GPU's selections are checked against
the oracle's (near-ties replayed), then dq, token dk and dv, and dw are compared
with the oracle run on the GPU's selections.  Tolerance: 1e-5 of the largest
magnitude of each gradient for fp32 storage (fp32 sums over up to a few thousand
entries and, for dk/dv/dw, over the rows that share a node, in atomic order),
2e-2 x RMS for bf16 storage, as for outputs."""
import numpy as np
import pytest
import torch

import synth
from oracle import recsa as O
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


CASES = [
    # (workload, L, n_kv, n_q, n rows, causal, overrides)
    ("tiny_f32_4k", 4096, 1, 1, 3, False, {}),
    ("tiny_f32_4k", 4229, 2, 4, 2, False, {}),                 # GQA, ragged tail and orphans
    ("tiny_f32_4k", 3001, 1, 2, 24, True, {"b": 5, "k": 3}),   # causal chunk, odd fanout
    ("tiny_f32_4k", 10, 1, 2, 4, True, {}),                    # L < b: tokens only, dw = 0
    ("tiny_f32_4k", 300, 1, 2, 2, False, {"dtype": "bf16"}),
    ("qwen3_4b_131k", 20000, 8, 32, 2, False, {}),             # the Qwen3-4B layer shape, bf16
    ("qwen3_4b_131k", 9000, 8, 32, 3, True, {}),
]

# The parent-major backward (bf16 storage; the library takes it for large row counts),
# forced on small cases: buckets of one parent spanning several items, odd fanouts,
# fanouts of one to four 32-child chunks, L < b.
TILED_CASES = [
    ("tiny_f32_4k", 300, 1, 2, 2, False, {"dtype": "bf16"}),
    ("tiny_f32_4k", 10, 1, 2, 4, True, {"dtype": "bf16"}),
    ("tiny_f32_4k", 3001, 1, 2, 24, True, {"b": 5, "k": 3, "dtype": "bf16"}),
    ("tiny_f32_4k", 4229, 2, 4, 40, True, {"dtype": "bf16"}),
    ("tiny_f32_4k", 3000, 1, 2, 8, True, {"b": 100, "k": 3, "dtype": "bf16"}),
    ("tiny_f32_4k", 5000, 1, 3, 6, False, {"b": 40, "k": 5, "dtype": "bf16"}),
    ("qwen3_4b_131k", 20000, 8, 32, 2, False, {}),
    ("qwen3_4b_131k", 9000, 8, 32, 3, True, {}),
]


def _tol(ref, dtype):
    if dtype == "f32":
        return 1e-5 * max(1.0, float(np.abs(ref).max()))
    return 2e-2 * float(np.sqrt(np.mean(ref ** 2))) + 1e-12


@pytest.mark.parametrize("name,L,n_kv,n_q,n,causal,kw", CASES)
def test_backward(name, L, n_kv, n_q, n, causal, kw):
    _say(f"case backward {name} L={L} n_kv={n_kv} n_q={n_q} n={n} causal={causal} {kw}")
    _run(name, L, n_kv, n_q, n, causal, kw, "rowwise")


@pytest.mark.parametrize("name,L,n_kv,n_q,n,causal,kw", TILED_CASES)
def test_backward_tiled(name, L, n_kv, n_q, n, causal, kw):
    _say(f"case backward tiled {name} L={L} n_kv={n_kv} n_q={n_q} n={n} causal={causal} {kw}")
    _run(name, L, n_kv, n_q, n, causal, kw, "parent_major")


def test_backward_default_path():
    """256 rows of a causal chunk: the library's own choice (the parent-major path)."""
    _say("case backward default path qwen3_4b_131k L=9000 n=8 causal")
    _run("qwen3_4b_131k", 9000, 8, 32, 8, True, {}, "auto")


def _run(name, L, n_kv, n_q, n, causal, kw, path):
    w = synth.scaled(synth.WORKLOADS[name], L, prefill_n=0, n_kv=n_kv, n_q=n_q, **kw)
    K, V = synth.gen_kv(w, 0, L)
    W = synth.pool_w(w)
    layer = P.make_layer(w, capacity=L)
    layer.set_path(path)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    rng = np.random.default_rng(L + n)
    Q = synth.to_storage(rng.standard_normal((n, n_q, w.d)).astype(np.float32), w.dtype)
    dO = rng.standard_normal((n, n_q, w.d)).astype(np.float32)
    grads, dbg = layer.backward(P.to_device(Q, w.dtype), torch.from_numpy(dO).cuda(), causal=causal,
                                debug=True)
    torch.cuda.synchronize()
    sel = dbg["selected"].cpu().numpy()
    G = n_q // n_kv
    # selections: GPU vs oracle (near-ties excused), then the oracle on the GPU's selections
    force = {}
    trees = [P.head_tree(K, V, W, g, w, L) for g in range(n_kv)]
    for i in range(n):
        n_ctx = L - n + i + 1 if causal else L
        for h in range(n_q):
            g = h // G
            tree_g = trees[g]
            P.check_row(tree_g, Q[i, h].astype(np.float64), 0, n_ctx, w.k, w.rope_base, w.softmax_scale,
                        sel[i * n_q + h])
            N = O.level_sizes(n_ctx, w.b)
            force[(i, h)] = {l: sel[i * n_q + h, l - 1][sel[i * n_q + h, l - 1] >= 0]
                             for l in range(1, len(N))}
    tree = O.build_tree(K[:, :L], V[:, :L], W, w.b, w.dtype, w.pool_scale, L)
    ref = O.backward(tree, Q.astype(np.float64), dO.astype(np.float64), w.k, w.rope_base, w.softmax_scale,
                     causal=causal, force=force)
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    rep = {}
    for key in ("dq", "dk", "dv", "dw"):
        g_ = got[key] if key in ("dq", "dw") else got[key][:, :L]
        err = float(np.abs(g_ - ref[key]).max())
        tol = _tol(ref[key], w.dtype)
        rep[key] = (err, tol)
        assert err <= tol, f"{key}: max abs error {err:.3g} > {tol:.3g}"
    # tokens past the length keep their gradients untouched
    assert np.all(got["dk"][:, L:] == 0) and np.all(got["dv"][:, L:] == 0)
    _say("backward", {k: f"{e:.2e}/{t:.2e}" for k, (e, t) in rep.items()})


@pytest.mark.parametrize("path,dtype,nq,L,b", [("rowwise", "f32", 2, 2000, 16), ("parent_major", "bf16", 64, 2000, 16),
                                              ("rowwise", "bf16", 2, 10, 16), ("parent_major", "bf16", 8, 10, 16),
                                              ("rowwise", "f32", 2, 3000, 40), ("parent_major", "bf16", 64, 3000, 40)])
def test_backward_overwrites_given_gradients(path, dtype, nq, L, b):
    """dk, dv (tokens [0, length)) and dw are written whatever the buffers held; rows
    from the length on are left alone.  Row-wise (two phases around the tree pass) and
    parent-major in one pass of rows (the tree pass between the levels), each also with
    fewer tokens than one node (no tree pass at all) and with a fanout above 32 (the
    general tree kernel writes the children, two 32-child chunks per parent)."""
    cap = L + 100
    w = synth.scaled(synth.WORKLOADS["tiny_f32_4k"], L, prefill_n=0, n_q=2, dtype=dtype, b=b)
    K, V = synth.gen_kv(w, 0, L)
    W = synth.pool_w(w)
    layer = P.make_layer(w, capacity=cap)
    layer.set_path(path)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    _say(f"case overwrite {path} {dtype} nq={nq} L={L} b={b}")
    rng = np.random.default_rng(9)
    q = P.to_device(synth.to_storage(rng.standard_normal((nq, 2, w.d)).astype(np.float32), w.dtype), w.dtype)
    dO = torch.from_numpy(rng.standard_normal((nq, 2, w.d)).astype(np.float32)).cuda()
    once = layer.backward(q, dO)
    junk = {k: torch.full_like(once[k], 7.5) for k in ("dk", "dv", "dw")}
    twice = layer.backward(q, dO, grads=junk)
    torch.cuda.synchronize()
    for k in ("dk", "dv"):
        torch.testing.assert_close(twice[k][:, :L], once[k][:, :L], rtol=1e-5, atol=1e-6)
        assert torch.all(twice[k][:, L:] == 7.5)
    torch.testing.assert_close(twice["dw"], once["dw"], rtol=1e-5, atol=1e-6)
    torch.testing.assert_close(twice["dq"], once["dq"], rtol=1e-5, atol=1e-6)


def test_backward_tiled_full_131k():
    """The Qwen3-4B layer at its full 131072-token context, a causal chunk of 8320
    queries (266240 rows: the parent-major path's two passes of at most 262144 rows):
    the parent-major backward against the row-wise one (itself pinned to the oracle
    above).  Rows whose selections differ between the two (a near-tie under the
    parent-major forward's split-bf16 logits) are each checked against the oracle
    (both selections valid under the near-tie rule), then get dO = 0, which removes
    them from every gradient on both paths; all four gradients must then agree to the bf16 bar
    (the parent-major run writes over buffers that held other values).  Sampled rows' dq, in both passes, is also checked against the oracle on the GPU's
    selections."""
    w = synth.WORKLOADS["qwen3_4b_131k"]
    L, n = w.L, 8320
    _say(f"case backward tiled vs rowwise qwen3_4b_131k L={L} n={n} causal")
    K, V = synth.gen_kv(w, 0, L)
    W = synth.pool_w(w)
    layer = P.make_layer(w, capacity=L)
    P.load_cache(layer, K, V, W, L, w.dtype)
    layer.build(L)
    rng = np.random.default_rng(11)
    Q = synth.to_storage(rng.standard_normal((n, w.n_q, w.d)).astype(np.float32), w.dtype)
    q = P.to_device(Q, w.dtype)
    dO = torch.from_numpy(rng.standard_normal((n, w.n_q, w.d)).astype(np.float32)).cuda()

    def run(path, d, grads=None):
        layer.set_path(path)
        g, dbg = layer.backward(q, d, causal=True, debug=True, grads=grads)
        torch.cuda.synchronize()
        return g, dbg

    gt, dt = run("parent_major", dO)
    gr, dr = run("rowwise", dO)
    bad = (dt["selected"] != dr["selected"]).flatten(1).any(1)
    _say(f"rows with another selection: {int(bad.sum())} of {bad.numel()}")
    assert int(bad.sum()) <= 32, "too many rows select differently for near-ties alone"
    # each such row: both paths' selections against the oracle (a near tie of the
    # oracle's logits, every disputed candidate inside the tie band)
    G = w.n_q // w.n_kv
    sel_t, sel_r = dt["selected"].cpu().numpy(), dr["selected"].cpu().numpy()
    trees = {}
    for r in torch.nonzero(bad).flatten().tolist():
        i, h = divmod(r, w.n_q)
        g = h // G
        if g not in trees:
            trees[g] = P.head_tree(K, V, W, g, w, L)
        for sel_ in (sel_t, sel_r):
            _, ex = P.check_row(trees[g], Q[i, h].astype(np.float64), 0, L - n + i + 1, w.k, w.rope_base,
                                w.softmax_scale, sel_[r])
        _say(f"row {r}: both selections valid under the near-tie rule")
    dO2 = dO.clone().view(-1, w.d)
    dO2[bad] = 0
    dO2 = dO2.view_as(dO)
    # two passes of rows clear the token gradients first: start the parent-major run
    # from buffers that hold something else
    junk = {k: torch.full_like(gt[k], -3.25) for k in ("dk", "dv", "dw")}
    gt, dt = run("parent_major", dO2, junk)
    gr, _ = run("rowwise", dO2)
    rep = {}
    for key in ("dq", "dk", "dv", "dw"):
        x, y = gt[key].cpu().numpy().astype(np.float64), gr[key].cpu().numpy().astype(np.float64)
        err = float(np.abs(x - y).max())
        tol = _tol(y, "bf16")
        rep[key] = f"{err:.2e}/{tol:.2e}"
        assert err <= tol, f"{key}: parent-major vs row-wise {err:.3g} > {tol:.3g}"
    _say("tiled vs rowwise", rep)
    # sampled rows' dq against the oracle on the parent-major path's selections
    sel = dt["selected"].cpu().numpy()
    dq_gpu = gt["dq"].cpu().numpy().astype(np.float64).reshape(n * w.n_q, w.d)
    dOn = dO2.cpu().numpy().astype(np.float64).reshape(n * w.n_q, w.d)
    refs, gots = [], []
    for r in (0, 5 * w.n_q + 7, (n // 2) * w.n_q + 20, 262144 + 5, n * w.n_q - 1):
        if bool(bad[r]):
            continue
        i, h = divmod(r, w.n_q)
        g = h // G
        if g not in trees:
            trees[g] = P.head_tree(K, V, W, g, w, L)
        tree = trees[g]
        n_ctx = L - n + i + 1
        P.check_row(tree, Q[i, h].astype(np.float64), 0, n_ctx, w.k, w.rope_base, w.softmax_scale, sel[r])
        N = O.level_sizes(n_ctx, w.b)
        force = {l: sel[r, l - 1][sel[r, l - 1] >= 0] for l in range(1, len(N))}
        gk = [np.zeros(np.shape(tree.keys[l])) for l in range(len(tree.keys))]
        gv = [np.zeros(np.shape(tree.vals[l])) for l in range(len(tree.vals))]
        refs.append(O.backward_row(tree, Q[i, h].astype(np.float64), 0, n_ctx, w.k, w.rope_base,
                                   w.softmax_scale, dOn[r], gk, gv, force=force))
        gots.append(dq_gpu[r])
    ref, got = np.array(refs), np.array(gots)
    err = float(np.abs(got - ref).max())
    tol = _tol(ref, "bf16")
    assert err <= tol, f"sampled dq vs oracle {err:.3g} > {tol:.3g}"
    _say(f"sampled dq vs oracle {err:.2e}/{tol:.2e} over {len(refs)} rows")
