"""Helpers for GPU-vs-oracle parity: move seeded inputs to the device, and
compare the GPU's per-level selections and outputs with the oracle's.

Selections must match exactly, except where the oracle's k-th and (k+1)-th
logits of that level differ by less than 1e-3 relative
(gap < 1e-3 * max(|z_k|, |z_k+1|, 1e-6)); such a row is then compared with the
oracle replaying the GPU's selection from that level down.
"""
from __future__ import annotations

import numpy as np
import torch

import long_context_recsa_amd as R
import synth
from oracle import recsa as O

TIE_REL = 1e-3


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
        zk, zk1 = sorted_topk_gap(lt.z, len(lt.sel_pos))
        if not (zk - zk1 < TIE_REL * max(abs(zk), abs(zk1), 1e-6)):
            raise AssertionError(
                f"selection differs at level {lt.level} (n_ctx {n_ctx}, head {g}): oracle "
                f"{lt.cand[lt.sel_pos].tolist()} gpu {got.tolist()}; k-th/k+1-th logits {zk:.7g} {zk1:.7g}")
        assert len(force) < max_excuses, "too many near-tie levels in one row"
        force[lt.level] = got.copy()
    raise AssertionError("replay did not converge")


def check_rows(tree, Q, rows, n_ctx_of, k, base, scale, gpu_out, dbg, G, dtype,
               all_out_rms=None, head_of=None):
    """rows: list of (query index, head); Q [n][Hq][d] host fp32; gpu_out [n][Hq][d];
    dbg: the debug dict (device tensors).  Asserts selection parity and the output
    tolerance (1e-5 max-abs for fp32 storage, 2e-2 * RMS of the oracle output for bf16)."""
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
        if ex == 0:
            assert nkeys[r] == res.keys_read, (qi, h, nkeys[r], res.keys_read)
        want[idx] = res.out
        got[idx] = gout[qi, h]
    err = np.abs(got - want).max()
    if dtype == "f32":
        tol = 1e-5
    else:
        rms = all_out_rms if all_out_rms is not None else float(np.sqrt(np.mean(want ** 2)))
        tol = 2e-2 * rms
    assert err <= tol, f"max abs error {err:.3g} > {tol:.3g}"
    return {"max_abs_err": float(err), "tol": tol, "excused_rows": excused, "rows": len(rows)}


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
        zk, zk1 = sorted_topk_gap(lt.z, len(lt.sel_pos))
        if not (zk - zk1 < TIE_REL * max(abs(zk), abs(zk1), 1e-6)):
            raise AssertionError(
                f"group selection differs at level {lt.level} (n_ctx {n_ctx}): oracle "
                f"{lt.cand[lt.sel_pos].tolist()} gpu {got.tolist()}; k-th/k+1-th scores {zk:.7g} {zk1:.7g}")
        assert len(force) < max_excuses, "too many near-tie levels in one row"
        force[lt.level] = got.copy()
    raise AssertionError("replay did not converge")


def check_groups(trees, Q, rows, n_ctx_of, k, base, scale, gpu_out, dbg, n_kv, dtype,
                 all_out_rms=None):
    """rows: list of (query index, KV head g); trees: {g: oracle tree of head g};
    Q [n][Hq][d] host fp32; gpu_out [n][Hq][d]; dbg rows are i * n_kv + g.  Asserts
    selection parity per group and the output tolerance on every head of the group."""
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
        if ex == 0:
            assert nkeys[r] == sum(len(t.cand) for t in res.levels), (qi, g, nkeys[r])
        want.append(res.out)
        got.append(gout[qi, g * G:(g + 1) * G])
    want, got = np.concatenate(want), np.concatenate(got)
    err = np.abs(got - want).max()
    if dtype == "f32":
        tol = 1e-5
    else:
        rms = all_out_rms if all_out_rms is not None else float(np.sqrt(np.mean(want ** 2)))
        tol = 2e-2 * rms
    assert err <= tol, f"max abs error {err:.3g} > {tol:.3g}"
    return {"max_abs_err": float(err), "tol": tol, "excused_rows": excused, "rows": len(rows)}
