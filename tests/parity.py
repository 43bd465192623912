"""Helpers for GPU-vs-oracle parity: move seeded inputs to the device, and
compare the GPU's per-level selections and outputs with the oracle's.

Selections must match exactly, except where the oracle's k-th and (k+1)-th
logits of that level differ by less than 1e-3 relative
(gap < 1e-3 * max(|z_k|, |z_k+1|, 1e-6)) and every candidate the two sides
disagree on scores inside that band around the boundary; such a row is then
compared with the oracle replaying the GPU's selection from that level down
(its keys-read count included).

Outputs: fp32 storage within 1e-5 max-abs; bf16 storage within 2e-2 x the RMS
of the oracle's output over the checked rows (the bar the hot path's
specification sets), and also within a regression bound REG_REL x that RMS,
which sits near the errors the GPU path reaches (fp32 arithmetic against the
oracle's f64 on the same bf16 inputs) and far below what one wrong summary
entry would cause.
"""
from __future__ import annotations

import numpy as np
import torch

import long_context_recsa_amd as R
import synth
from oracle import recsa as O

TIE_REL = 1e-3
# Regression bound for bf16 storage, relative to the oracle's output RMS.  One
# summary entry with a wrong value row moves a row's output by about its softmax
# weight times the row's difference, ~1e-3 x RMS at the workloads' shapes.  The
# GPU path reaches at most 2.1e-4 x RMS (a fanout-3 tree of ten levels, where
# summaries that round one bf16 ulp away from the oracle's are most frequent) and
# below 1e-4 x RMS on every workload shape.
REG_REL = 5e-4


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    bits = synth.storage_bits(x, dtype)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def make_layer(w: synth.Workload, capacity: int | None = None, k: int | None = None,
               out: str = "f32") -> R.RecsaLayer:
    p = R.make_params(w.n_kv, w.n_q, w.d, w.b, w.k if k is None else k,
                      w.capacity if capacity is None else capacity, store=w.dtype, out=out,
                      rope_base=w.rope_base, softmax_scale=w.softmax_scale,
                      pool_scale=w.pool_scale)
    return R.RecsaLayer(p)


def load_cache(layer: R.RecsaLayer, K: np.ndarray, V: np.ndarray, W: np.ndarray, n: int,
               dtype: str) -> None:
    for g in range(K.shape[0]):
        layer.k_cache[g, :n].copy_(to_device(K[g, :n], dtype))
        layer.v_cache[g, :n].copy_(to_device(V[g, :n], dtype))
    layer.pool_w.copy_(torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda())


def sorted_topk_gap(z: np.ndarray, m: int):
    zs = np.sort(z)[::-1]
    return float(zs[m - 1]), float(zs[m])


def _near_tie(lt, got, what):
    """Excuse a differing selection at one level: the k-th and (k+1)-th oracle logits
    lie within the relative tie band, and so does every candidate the two sides
    disagree on."""
    m = len(lt.sel_pos)
    zk, zk1 = sorted_topk_gap(lt.z, m)
    band = TIE_REL * max(abs(zk), abs(zk1), 1e-6)
    want = lt.cand[lt.sel_pos]
    if not (zk - zk1 < band):
        raise AssertionError(
            f"{what} differs at level {lt.level}: oracle {want.tolist()} gpu {got.tolist()}; "
            f"k-th/k+1-th logits {zk:.7g} {zk1:.7g}")
    pos = {int(c): i for i, c in enumerate(lt.cand)}
    for node in set(want.tolist()) ^ set(got.tolist()):
        assert node in pos, f"level {lt.level}: gpu kept node {node}, not a candidate"
        z = lt.z[pos[node]]
        assert zk1 - band <= z <= zk + band, (
            f"{what} at level {lt.level}: node {node} (logit {z:.7g}) is kept by one side only "
            f"but lies outside the tie band [{zk1 - band:.7g}, {zk + band:.7g}]")


def check_row(tree, q, g, n_ctx, k, base, scale, gpu_sel_row, max_excuses=3):
    """Compare one row's per-level selections with the oracle; returns
    (oracle RowResult to compare the output with, number of excused levels)."""
    force: dict = {}
    for _ in range(64):
        res = O.descend(tree, q, g, n_ctx, k, base, scale, force=force or None)
        bad = None
        for lt in res.levels[:-1]:
            want = lt.cand[lt.sel_pos]
            got = gpu_sel_row[lt.level - 1]
            assert np.all(got[len(want):] == -1), (lt.level, got)
            if lt.level in force:
                continue
            if not np.array_equal(want, got[:len(want)]):
                bad = (lt, got[:len(want)])
                break
        if bad is None:
            return res, len(force)
        lt, got = bad
        _near_tie(lt, got, f"selection (n_ctx {n_ctx}, head {g})")
        assert len(force) < max_excuses, "too many near-tie levels in one row"
        force[lt.level] = got.copy()
    raise AssertionError("replay did not converge")


def _check_out(err_rows, want, dtype):
    """Spec bar and regression bound on the stacked outputs of the checked rows."""
    err = float(np.abs(err_rows).max()) if err_rows.size else 0.0
    if dtype == "f32":
        tol = 1e-5
        assert err <= tol, f"max abs error {err:.3g} > {tol:.3g}"
        return err, tol, None
    rms = float(np.sqrt(np.mean(want ** 2)))
    tol = 2e-2 * rms
    assert err <= tol, f"max abs error {err:.3g} > {tol:.3g} (2e-2 x oracle RMS {rms:.3g})"
    assert err <= REG_REL * rms, (f"max abs error {err:.3g} > regression bound {REG_REL} x oracle RMS "
                                  f"{rms:.3g} = {REG_REL * rms:.3g}")
    return err, tol, err / rms if rms > 0 else 0.0


def check_rows(tree, Q, rows, n_ctx_of, k, base, scale, gpu_out, dbg, G, dtype, head_of=None):
    """rows: list of (query index, head); Q [n][Hq][d] host fp32; gpu_out [n][Hq][d];
    dbg: the debug dict (device tensors).  Asserts selection parity, the keys-read
    count of every row (of the replay where a near tie was excused) and the output
    bars (1e-5 max-abs for fp32 storage; for bf16, 2e-2 and REG_REL x the RMS of the
    oracle's output over these rows)."""
    Hq = Q.shape[1]
    sel = dbg["selected"].cpu().numpy()
    nkeys = dbg["n_keys"].cpu().numpy()
    gout = to_host(gpu_out)
    want = np.zeros((len(rows), Q.shape[2]))
    got = np.zeros_like(want)
    excused = 0
    for idx, (qi, h) in enumerate(rows):
        r = qi * Hq + h
        g = h // G if head_of is None else head_of(h)
        res, ex = check_row(tree, Q[qi, h], g, n_ctx_of(qi), k, base, scale, sel[r])
        excused += ex > 0
        assert nkeys[r] == res.keys_read, (qi, h, nkeys[r], res.keys_read)
        want[idx] = res.out
        got[idx] = gout[qi, h]
    err, tol, rel = _check_out(got - want, want, dtype)
    return {"max_abs_err": err, "tol": tol, "err_over_rms": rel, "excused_rows": excused,
            "rows": len(rows)}


def head_tree(K, V, W, g, w, length):
    """Oracle tree of KV head g alone (K, V [n_kv][>=length][d])."""
    return O.build_tree(K[g:g + 1], V[g:g + 1], W[g:g + 1], w.b, w.dtype, w.pool_scale, length)


def check_group(tree, Qg, n_ctx, k, base, scale, gpu_sel_row, max_excuses=3):
    """Selections of one (query, KV group) row with a shared selection, compared
    level by level with the oracle's (group score = the sum of the heads' logits);
    a near-tie of the group score is replayed as in check_row.  Returns (oracle
    GroupResult, number of excused levels)."""
    force: dict = {}
    for _ in range(64):
        res = O.descend_group(tree, Qg, 0, n_ctx, k, base, scale, force=force or None)
        bad = None
        for lt in res.levels[:-1]:
            want = lt.cand[lt.sel_pos]
            got = gpu_sel_row[lt.level - 1]
            assert np.all(got[len(want):] == -1), (lt.level, got)
            if lt.level in force:
                continue
            if not np.array_equal(want, got[:len(want)]):
                bad = (lt, got[:len(want)])
                break
        if bad is None:
            return res, len(force)
        lt, got = bad
        _near_tie(lt, got, f"group selection (n_ctx {n_ctx})")
        assert len(force) < max_excuses, "too many near-tie levels in one row"
        force[lt.level] = got.copy()
    raise AssertionError("replay did not converge")


def check_groups(trees, Q, rows, n_ctx_of, k, base, scale, gpu_out, dbg, n_kv, dtype):
    """rows: list of (query index, KV head g); trees: {g: oracle tree of head g};
    Q [n][Hq][d] host fp32; gpu_out [n][Hq][d]; dbg rows are i * n_kv + g.  Asserts
    selection parity per group, the keys-read count and the output bars on every
    head of the group."""
    Hq = Q.shape[1]
    G = Hq // n_kv
    sel = dbg["selected"].cpu().numpy()
    nkeys = dbg["n_keys"].cpu().numpy()
    gout = to_host(gpu_out)
    want, got = [], []
    excused = 0
    for (qi, g) in rows:
        r = qi * n_kv + g
        res, ex = check_group(trees[g], Q[qi, g * G:(g + 1) * G], n_ctx_of(qi), k, base, scale,
                              sel[r])
        excused += ex > 0
        assert nkeys[r] == sum(len(t.cand) for t in res.levels), (qi, g, nkeys[r])
        want.append(res.out)
        got.append(gout[qi, g * G:(g + 1) * G])
    want, got = np.concatenate(want), np.concatenate(got)
    err, tol, rel = _check_out(got - want, want, dtype)
    return {"max_abs_err": err, "tol": tol, "err_over_rms": rel, "excused_rows": excused,
            "rows": len(rows)}


def assert_same_query(out_a, dbg_a, out_b, dbg_b, rows_a, rows_b):
    """One query decoded in two calls of different batch sizes: the same selections
    at every level, bit for bit, and the same output up to fp32 summation order (a
    decode of at most one row per compute unit runs eight waves per row, a larger one
    four, and the two fold the softmax in different groupings)."""
    import torch
    sa, sb = dbg_a["selected"][rows_a], dbg_b["selected"][rows_b]
    assert torch.equal(sa, sb), "the same query selected differently in two batch sizes"
    torch.testing.assert_close(out_a, out_b, rtol=1e-5, atol=1e-6)
