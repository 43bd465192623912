"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test pins the oracle to something other than itself: hand-worked
examples (tests/golden), closed forms, invariants the RecSA abstract states,
an independent brute-force implementation, and a library attention routine
in the special case where RecSA reduces to dense attention.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import recsa as O
from tests import brute_force as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_inputs(seed, L, d, n_kv=1, scale_w=1.0):
    r = np.random.default_rng(seed)
    K = r.standard_normal((n_kv, L, d)).astype(np.float32)
    V = r.standard_normal((n_kv, L, d)).astype(np.float32)
    w = (r.standard_normal((n_kv, d)) * scale_w / math.sqrt(d)).astype(np.float32)
    return r, K, V, w


# ---------------------------------------------------------------- golden --
def test_golden_hand_q0():
    g = _load("hand_q0.json")
    K = np.array([g["K"]], np.float32)
    V = np.array([g["V"]], np.float32)
    w = np.array([g["w"]], np.float32)
    tree = O.build_tree(K, V, w, g["b"], "f32", 1 / math.sqrt(g["d"]), g["length"])
    r = O.descend(tree, np.array(g["q"]), 0, g["length"], g["k"], g["rope_base"], 1.0)
    np.testing.assert_allclose(r.out, g["expected_out"], rtol=0, atol=1e-12)
    for lev, nodes in g["expected_selected"].items():
        assert list(r.selected_nodes(int(lev))) == nodes
    assert [[int(a), int(b)] for a, b in zip(r.entry_level, r.entry_node)] == g["expected_entries"]
    assert r.keys_read == g["expected_keys_read"]
    assert r.max_position == g["expected_max_position"]


def test_golden_hand_pool():
    g = _load("hand_pool.json")
    d = g["d"]
    K = np.array([g["K"]], np.float32)
    w = np.array([g["w_over_sqrt2_ln3"]], np.float64) * math.sqrt(2) * math.log(3)
    tree = O.build_tree(K, K, w, g["b"], "f32", 1 / math.sqrt(d), len(g["K"]))
    np.testing.assert_allclose(tree.keys[1][0], g["expected_level1"], atol=1e-7)
    a1 = 3 ** 1.8 / (3 ** 0.75 + 3 ** 1.8)
    want = (1 - a1) * np.array([0.75, 0.25]) + a1 * np.array([1.8, 0.2])
    np.testing.assert_allclose(tree.keys[2][0][0], want, atol=1e-6)


def test_golden_bf16_rounding():
    for c in _load("bf16_rounding.json")["cases"]:
        got = O.round_store(np.array([c["x"]]), "bf16")[0]
        assert got == c["bf16"], c


# ----------------------------------------------------------- brute force --
CASES = [
    # (L, b, k, d): non-aligned lengths so orphans and tails occur
    (37, 2, 1, 2), (53, 3, 2, 4), (70, 4, 2, 4), (101, 3, 3, 2), (129, 2, 3, 4),
    (200, 4, 3, 8), (255, 4, 1, 4), (300, 3, 2, 2), (17, 4, 3, 4), (9, 3, 1, 2),
]


@pytest.mark.parametrize("L,b,k,d", CASES)
def test_brute_force_tiny(L, b, k, d):
    r, K, V, w = _rand_inputs(1000 + L, L, d, scale_w=3.0)
    base, ps, s = 10000.0, 1 / math.sqrt(d), 1 / math.sqrt(d)
    tree = O.build_tree(K, V, w, b, "f32", ps, L)
    bk, bv = BF.build(K[0].tolist(), V[0].tolist(), w[0].tolist(), b, ps, L)
    for l in range(1, len(bk)):
        np.testing.assert_allclose(tree.keys[l][0], bk[l], rtol=0, atol=1e-6)
        np.testing.assert_allclose(tree.vals[l][0], bv[l], rtol=0, atol=1e-6)
    for t in range(4):
        q = r.standard_normal(d) * 2.0
        n_ctx = int(r.integers(1, L + 1)) if t else L
        res = O.descend(tree, q, 0, n_ctx, k, base, s)
        out, sels, entries = BF.row(bk, bv, q.tolist(), n_ctx, b, k, base, s)
        near_tie = any(np.isfinite(lt.gap) and lt.gap < 1e-9 for lt in res.levels)
        if not near_tie:
            for lev, nodes in sels.items():
                assert list(res.selected_nodes(lev)) == nodes
            assert sorted(zip(res.entry_level.tolist(), res.entry_node.tolist())) == sorted(entries)
        np.testing.assert_allclose(res.out, out, rtol=0, atol=1e-6)


# ------------------------------------------------- dense special case pin --
def _sdpa_dense(q, K, V, n, base, s):
    """torch scaled_dot_product_attention (CPU, float64) on RoPE'd inputs,
    the query at position n and key i at position i."""
    d = K.shape[-1]
    h = d // 2
    theta = base ** (-2.0 * torch.arange(h, dtype=torch.float64) / d)

    def rot(x, pos):
        a = pos[:, None].double() * theta[None, :]
        c, sn = torch.cos(a), torch.sin(a)
        return torch.cat([x[:, :h] * c - x[:, h:] * sn, x[:, h:] * c + x[:, :h] * sn], -1)

    kr = rot(torch.tensor(K[:n], dtype=torch.float64), torch.arange(n))
    qr = rot(torch.tensor(q, dtype=torch.float64)[None], torch.tensor([n]))
    out = torch.nn.functional.scaled_dot_product_attention(
        qr[None, None], kr[None, None], torch.tensor(V[:n], dtype=torch.float64)[None, None],
        scale=s)
    return out[0, 0, 0].numpy()


def test_dense_pin_library():
    r, K, V, w = _rand_inputs(7, 300, 16)
    q = r.standard_normal(16)
    for n in (1, 2, 77, 300):
        np.testing.assert_allclose(O.dense(q, K[0], V[0], n, 1e6, 0.25),
                                   _sdpa_dense(q, K[0], V[0], n, 1e6, 0.25), atol=1e-12)


def test_dense_equality_k_covers_everything():
    """k >= every candidate count: nothing is summarized, so RecSA is dense
    attention with the query at position n (tiny fp32 workload, k = N_1)."""
    w = synth.WORKLOADS["tiny_f32_4k"]
    K, V = synth.gen_kv(w)
    W = synth.pool_w(w)
    Q = synth.decode_queries(w, 8)
    tree = O.build_tree(K, V, W, w.b, "f32", w.pool_scale, w.L)
    kbig = w.L // w.b
    for i in range(8):
        r = O.descend(tree, Q[i, 0], 0, w.L, kbig, w.rope_base, w.softmax_scale)
        assert len(r.entry_z) == w.L and np.all(r.entry_level == 0)
        ref = _sdpa_dense(Q[i, 0], K[0], V[0], w.L, w.rope_base, w.softmax_scale)
        np.testing.assert_allclose(r.out, ref, atol=1e-10)


@pytest.mark.parametrize("L,b", [(15, 4), (200, 16), (1023, 32)])
def test_dense_equality_short_context(L, b):
    """L < b^2 and k >= b: at most one level, all of it selected."""
    r, K, V, w = _rand_inputs(L, L, 8)
    tree = O.build_tree(K, V, w, b, "f32", 0.3, L)
    for _ in range(3):
        q = r.standard_normal(8)
        res = O.descend(tree, q, 0, L, b, 1e4, 0.35)
        np.testing.assert_allclose(res.out, _sdpa_dense(q, K[0], V[0], L, 1e4, 0.35), atol=1e-10)


# ------------------------------------------------------------ invariants --
@pytest.mark.parametrize("store", ["f32", "bf16"])
def test_node_values_are_subtree_means(store):
    """Each node's value is its subtree's mean: checked against the mean of
    the children's means (a different summation) at every level."""
    r, K, V, w = _rand_inputs(3, 5000, 8)
    tree = O.build_tree(K, V, w, 4, store, 0.3, 5000)
    V64 = V[0].astype(np.float64)
    prev = V64
    for l in range(1, len(tree.keys)):
        n = len(tree.vals[l][0])
        means = prev[:n * 4].reshape(n, 4, -1).mean(axis=1)
        if store == "f32":
            np.testing.assert_allclose(tree.vals[l][0], means, rtol=1e-6, atol=1e-7)
        else:
            ulp = 2.0 ** (np.floor(np.log2(np.abs(means) + 1e-30)) - 7)
            assert np.all(np.abs(tree.vals[l][0] - means) <= ulp)
        prev = means


def test_pooler_zero_w_gives_mean():
    r, K, V, _ = _rand_inputs(4, 700, 8)
    tree = O.build_tree(K, V, np.zeros((1, 8)), 3, "f32", 0.3, 700)
    prev = K[0].astype(np.float64)
    for l in range(1, len(tree.keys)):
        n = len(tree.keys[l][0])
        want = tree.keys[l - 1][0][:n * 3].reshape(n, 3, -1).mean(axis=1)
        np.testing.assert_allclose(tree.keys[l][0], want, rtol=1e-6, atol=1e-7)


def test_pooler_convex_and_shared_across_levels():
    r, K, V, w = _rand_inputs(5, 2000, 8, scale_w=8.0)
    tree = O.build_tree(K, V, w, 5, "f32", 1 / math.sqrt(8), 2000)
    for l in range(1, len(tree.keys)):
        ch = tree.keys[l - 1][0][:len(tree.keys[l][0]) * 5].reshape(-1, 5, 8)
        assert np.all(tree.keys[l][0] <= ch.max(axis=1) + 1e-6)
        assert np.all(tree.keys[l][0] >= ch.min(axis=1) - 1e-6)
    # level-2 keys from the stored level-1 keys with the one level-1 vector w
    ch = tree.keys[1][0][:len(tree.keys[2][0]) * 5].reshape(-1, 5, 8)
    lg = (ch @ w[0].astype(np.float64)) / math.sqrt(8)
    a = np.exp(lg - lg.max(1, keepdims=True))
    a /= a.sum(1, keepdims=True)
    np.testing.assert_allclose(tree.keys[2][0], np.einsum("nc,ncd->nd", a, ch), atol=1e-6)


def _token_cover(res, b, n_ctx):
    cover = np.zeros(n_ctx, np.int64)
    for lev, node in zip(res.entry_level, res.entry_node):
        cover[node * b ** lev:(node + 1) * b ** lev] += 1
    return cover


@pytest.mark.parametrize("L,b,k", [(4096, 16, 4), (4229, 16, 4), (5000, 3, 2), (999, 7, 1),
                                   (65536, 32, 8), (70000, 64, 16)])
def test_entries_partition_and_cost(L, b, k):
    """Entries cover every token exactly once; keys read stay within
    N_H + H*k*b + orphans (O(log L)); RoPE positions within k*b + b - 1."""
    r, K, V, w = _rand_inputs(L, L, 4)
    tree = O.build_tree(K, V, w, b, "f32", 0.5, L)
    for t in range(3):
        n_ctx = L - t * 7
        res = O.descend(tree, r.standard_normal(4), 0, n_ctx, k, 1e4, 0.5)
        assert np.all(_token_cover(res, b, n_ctx) == 1)
        N = O.level_sizes(n_ctx, b)
        H = len(N) - 1
        orphans = sum(N[l] - b * N[l + 1] for l in range(H))
        assert res.keys_read <= N[H] + H * k * b + orphans
        assert res.keys_read <= (H + 1) * k * b + orphans
        assert res.max_position <= k * b + b - 1
        for lt in res.levels[:-1]:
            assert len(lt.sel_pos) == min(k, len(lt.cand))


@pytest.mark.parametrize("b,k", [(4, 2), (16, 4), (32, 8)])
def test_positions_bounded_at_any_length(b, k):
    """Largest RoPE position is the same at L = b^2, b^3, b^4 (not growing with L)."""
    seen = []
    for p in (2, 3, 4):
        L = b ** p
        if L > 1 << 20:
            continue
        r, K, V, w = _rand_inputs(p, L, 4)
        tree = O.build_tree(K, V, w, b, "f32", 0.5, L)
        res = O.descend(tree, r.standard_normal(4), 0, L, k, 1e4, 0.5)
        assert res.max_position <= k * b + b - 1
        seen.append(res.max_position)
    assert len(set(seen[1:])) <= 1


def test_rope_is_rotation_by_position():
    """Pair j of rope(x, p), read as the complex number x_j + i x_{j+d/2}, is that
    number times exp(i p base^(-2j/d)); so norms are kept and scores depend only
    on the position difference (what makes candidate indices relative positions)."""
    r = np.random.default_rng(11)
    d, base = 16, 1e4
    x = r.standard_normal(d)
    y = r.standard_normal(d)
    for p in (0, 1, 7, 1000, 123457):
        got = O.rope(x, p, base)
        z = (x[:d // 2] + 1j * x[d // 2:]) * np.exp(1j * p * base ** (-np.arange(0, d, 2) / d))
        np.testing.assert_allclose(got[:d // 2], z.real, atol=1e-12)
        np.testing.assert_allclose(got[d // 2:], z.imag, atol=1e-12)
        assert abs(np.linalg.norm(got) - np.linalg.norm(x)) < 1e-12
    for n, i, t in ((5, 2, 3), (300, 0, 1000), (64, 63, 77777)):
        a = O.rope(x, n, base) @ O.rope(y, i, base)
        b_ = O.rope(x, n + t, base) @ O.rope(y, i + t, base)
        assert abs(a - b_) < 1e-9


def test_q_zero_closed_form():
    """q = 0: every logit is 0, each level keeps its first min(k, n)
    candidates, and the output is the plain mean of the entry values."""
    L, b, k = 1234, 5, 2
    r, K, V, w = _rand_inputs(11, L, 4)
    tree = O.build_tree(K, V, w, b, "f32", 0.5, L)
    res = O.descend(tree, np.zeros(4), 0, L, k, 1e4, 0.5)
    # independent walk: keep the first k candidates at each level
    N = O.level_sizes(L, b)
    cand = list(range(N[-1]))
    vals = []
    for l in range(len(N) - 1, 0, -1):
        keep = cand[:k]
        vals += [tree.vals[l][0][c] for c in cand[k:]]
        cand = [c * b + j for c in keep for j in range(b)] + list(range(b * N[l], N[l - 1]))
    vals += [V[0][c].astype(np.float64) for c in cand]
    np.testing.assert_allclose(res.out, np.mean(vals, axis=0), atol=1e-12)


def test_value_affine_equivariance():
    L, b, k = 3000, 8, 3
    r, K, V, w = _rand_inputs(12, L, 8)
    q = r.standard_normal(8)
    base = O.descend(O.build_tree(K, V, w, b, "f32", 0.4, L), q, 0, L, k, 1e4, 0.4).out
    c = np.float32(2.5)
    shifted = O.descend(O.build_tree(K, V + c, w, b, "f32", 0.4, L), q, 0, L, k, 1e4, 0.4).out
    np.testing.assert_allclose(shifted, base + 2.5, atol=2e-6)
    scaled = O.descend(O.build_tree(K, V * np.float32(4), w, b, "f32", 0.4, L), q, 0, L, k, 1e4, 0.4).out
    np.testing.assert_allclose(scaled, base * 4, atol=1e-12)


# ---------------------------------------------------------------- prefill --
@pytest.mark.parametrize("L0,n,b,k", [(200, 60, 3, 2), (230, 30, 3, 1), (1000, 40, 4, 3), (5, 20, 2, 2)])
def test_prefill_prefix_tree_equals_sequential(L0, n, b, k):
    """Prefill over the prefix tree equals appending one token and querying
    it, repeated -- bit for bit (complete nodes never change)."""
    r, K, V, w = _rand_inputs(L0 + n, L0 + n, 4, n_kv=2)
    Q = r.standard_normal((n, 4, 4))
    tree = O.build_tree(K, V, w, b, "f32", 0.5, L0 + n)
    a, _ = O.prefill(tree, Q, k, 1e4, 0.5)
    s = O.prefill_sequential(K, V, w, b, "f32", 0.5, L0, Q, k, 1e4, 0.5)
    assert np.array_equal(a, s)


def test_append_equals_rebuild():
    r, K, V, w = _rand_inputs(9, 3000, 8, n_kv=2)
    full = O.build_tree(K, V, w, 4, "bf16", 0.3, 3000)
    inc = O.build_tree(K, V, w, 4, "bf16", 0.3, 100)
    for n in (101, 500, 511, 2047, 2048, 3000):
        O.extend_tree(inc, K, V, n)
    for l in range(len(full.keys)):
        for g in range(2):
            assert np.array_equal(full.keys[l][g], inc.keys[l][g])
            assert np.array_equal(full.vals[l][g], inc.vals[l][g])


# ---------------------------------------------------------------- needles --
def test_pooler_needles_are_reached():
    """Pooler-dominant needle recipe (2M workload, at 65,536 tokens): the
    descent of each needle's matching query reaches the needle token."""
    w = synth.scaled(synth.WORKLOADS["qwen3_4b_2m"], 1 << 16)
    Q = synth.decode_queries(w, w.max_batch)
    W = synth.pool_w(w)
    pairs = synth.needle_pairs(w)
    heads = sorted({g for (_, _, g, _, _) in pairs})[:2]
    K, V = synth.gen_kv(w, heads=heads)
    Kf = np.zeros((w.n_kv,) + K.shape[1:], np.float32)
    Vf = np.zeros_like(Kf)
    for i, g in enumerate(heads):
        Kf[g], Vf[g] = K[i], V[i]
    tree = O.build_tree(Kf, Vf, W, w.b, "bf16", w.pool_scale, w.L)
    for (j, pos, g, qi, qh) in pairs:
        if g not in heads:
            continue
        res = O.descend(tree, Q[qi, qh], g, w.L, w.k, w.rope_base, w.softmax_scale)
        assert pos in set(res.levels[-1].cand.tolist()), (j, pos)


def test_generator_slabs_independent():
    w = synth.scaled(synth.WORKLOADS["qwen3_4b_131k"], 70000)
    K, V = synth.gen_kv(w, heads=[3])
    K2, V2 = synth.gen_kv(w, 65000, 70000, heads=[3])
    assert np.array_equal(K[0, 65000:], K2[0]) and np.array_equal(V[0, 65000:], V2[0])
    assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(K)), K)


# -------------------------------------------- group-shared selection variant --
@pytest.mark.parametrize("L,b,k,d", CASES[:6])
def test_group_selection_is_the_summed_query_brute_force(L, b, k, d):
    """The group score is the sum of the heads' logits.  RoPE and the inner
    product are linear in q, so the shared selection must be the one the
    brute-force enumeration makes for the single query q_1 + ... + q_G."""
    r, K, V, w = _rand_inputs(2000 + L, L, d, scale_w=3.0)
    base, ps, s = 10000.0, 1 / math.sqrt(d), 1 / math.sqrt(d)
    tree = O.build_tree(K, V, w, b, "f32", ps, L)
    bk, bv = BF.build(K[0].tolist(), V[0].tolist(), w[0].tolist(), b, ps, L)
    for t in range(3):
        Qg = r.standard_normal((4, d)) * 2.0
        n_ctx = int(r.integers(1, L + 1)) if t else L
        res = O.descend_group(tree, Qg, 0, n_ctx, k, base, s)
        _, sels, _ = BF.row(bk, bv, Qg.sum(axis=0).tolist(), n_ctx, b, k, base, s)
        if any(np.isfinite(lt.gap) and lt.gap < 1e-9 for lt in res.levels):
            continue
        for lev, nodes in sels.items():
            assert list(res.selected_nodes(lev)) == nodes


@pytest.mark.parametrize("L,b,k", [(300, 3, 2), (1000, 4, 3), (4096, 16, 4)])
def test_group_heads_are_per_head_descents_on_the_shared_selection(L, b, k):
    """Each head's output is the per-head mixed softmax with the selection
    replaced by the group's (the per-head oracle replays a given selection)."""
    d = 8
    r, K, V, w = _rand_inputs(L + 5, L, d, n_kv=2)
    tree = O.build_tree(K, V, w, b, "f32", 0.4, L)
    for g in range(2):
        Qg = r.standard_normal((3, d)) * 1.5
        n_ctx = L - 7 * g
        res = O.descend_group(tree, Qg, g, n_ctx, k, 1e4, 0.35)
        force = {t.level: t.cand[t.sel_pos] for t in res.levels if t.level > 0}
        for h in range(3):
            ref = O.descend(tree, Qg[h], g, n_ctx, k, 1e4, 0.35, force=force)
            np.testing.assert_allclose(res.out[h], ref.out, rtol=0, atol=1e-12)
            # the heads' logits are their own, not the group score
            for lt, z in zip(ref.levels, res.head_z):
                np.testing.assert_allclose(z[h], lt.z, rtol=0, atol=1e-12)


def test_group_of_one_and_identical_heads_reduce_to_per_head():
    w = synth.WORKLOADS["tiny_f32_4k"]
    K, V = synth.gen_kv(w)
    tree = O.build_tree(K, V, synth.pool_w(w), w.b, "f32", w.pool_scale, w.L)
    Q = synth.decode_queries(w, 4)
    for i in range(4):
        q = Q[i, 0]
        ref = O.descend(tree, q, 0, w.L, w.k, w.rope_base, w.softmax_scale)
        one = O.descend_group(tree, q[None], 0, w.L, w.k, w.rope_base, w.softmax_scale)
        same = O.descend_group(tree, np.stack([q] * 4), 0, w.L, w.k, w.rope_base,
                               w.softmax_scale)
        for res in (one, same):
            for lev in range(1, len(ref.levels)):
                assert list(res.selected_nodes(lev)) == list(ref.selected_nodes(lev))
            np.testing.assert_allclose(res.out, np.stack([ref.out] * len(res.out)), atol=1e-12)


def test_group_k_covers_everything_is_dense_per_head():
    """With k >= every candidate count nothing is summarized: every head's
    output is its own dense causal attention, whatever the group shares."""
    r, K, V, w = _rand_inputs(11, 1023, 8)
    tree = O.build_tree(K, V, w, 32, "f32", 0.3, 1023)
    Qg = r.standard_normal((4, 8))
    res = O.descend_group(tree, Qg, 0, 1023, 32, 1e4, 0.35)
    for h in range(4):
        np.testing.assert_allclose(res.out[h], _sdpa_dense(Qg[h], K[0], V[0], 1023, 1e4, 0.35),
                                   atol=1e-10)
