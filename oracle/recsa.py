"""CPU oracle for the RecSA hot path (tree build and append, level-wise descent,
mixed softmax) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The GPU library never calls it and
shares no code with it.

Plain and slow on purpose: NumPy in float64, one row at a time, with the
method's steps in the order the pages state them.  Library primitives used
as steps: an inner product, ``np.exp``, ``np.lexsort``.

Source: "Recursive Sparse Attention: Million-Token Length Extrapolation at
Logarithmic Cost" (arXiv 2611.07232), abstract.  Its sentences are cited
below by what they say:

* [tree]      a tree over the KV cache whose nodes each stand for their whole
              subtree through a single key and the average of its values;
* [pooler]    a single pooler per layer, the same at every level, makes the
              keys;
* [selection] no more than k candidates survive at each level above the
              tokens; the dropped ones enter, through their summaries, the
              same softmax as the exact tokens;
* [rope]      an entry's rotary position is its rank in its level's
              candidate list;
* [cost]      selection cost and entries read are O(log L) per query.

Points the pages leave open are fixed as follows (the pages say nothing that
contradicts them):

* tree shape: b-ary over aligned blocks; level l has N_l = floor(n / b^l)
  complete nodes over n tokens; the top level H is the highest with N_H >= 1
  and all of its nodes are the first candidates;
* a partial node has no summary: its complete children ("orphans", the
  tokens past b*N_1 at level 0) join the candidates of the level below,
  after the selected nodes' children;
* candidates are kept in ascending node order, orphans last; "index among
  the candidates" is the position in that list;
* the query's RoPE position at a level is that level's candidate count;
* RoPE is rotate-half: pairs (i, i + d/2), angle p * base^(-2i/d);
* the selection score is the softmax logit s * <rope(q, n), rope(key, i)>;
  equal scores go to the lower candidate index;
* the pooler is attention pooling with a per-KV-head vector w:
  alpha = softmax_c(pool_scale * w . key_c), key = sum_c alpha_c key_c,
  applied to the stored child keys at every level;
* a node's value is the mean of its subtree's token values;
* summaries are stored in the cache's format (fp32 or bf16, rounded to
  nearest even) -- the only rounding points besides the inputs.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# storage format
# ----------------------------------------------------------------------------
def round_store(x: np.ndarray, store: str) -> np.ndarray:
    """Round float64 values to the summary storage format, returned as float64."""
    x = np.ascontiguousarray(x, dtype=F64)
    if store == "f64":          # no rounding (gradient checks by finite differences)
        return x
    if store == "f32":
        return x.astype(np.float32).astype(F64)
    if store != "bf16":
        raise ValueError(store)
    # bf16 keeps 7 of float64's 52 fraction bits: round away 45 bits, ties to even
    a = np.abs(x)
    if np.any((a > 0) & (a < 2.0 ** -126)):
        raise ValueError("value below bf16's normal range")
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    r = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(F64)


# ----------------------------------------------------------------------------
# geometry [tree], [selection]
# ----------------------------------------------------------------------------
def level_sizes(n_ctx: int, b: int) -> list[int]:
    """[N_0, N_1, ..., N_H]: complete nodes per level over n_ctx tokens.

    N_0 = n_ctx tokens; N_l = floor(n_ctx / b^l); H is the highest level with
    at least one complete node ([tree]; reading: aligned b-ary blocks).
    """
    N = [int(n_ctx)]
    while N[-1] // b >= 1:
        N.append(N[-1] // b)
    return N


# ----------------------------------------------------------------------------
# RoPE [rope]
# ----------------------------------------------------------------------------
def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate-half RoPE of x[..., d] at integer position(s) pos (broadcast over
    the leading axis): pair (i, i + d/2) turns by pos * base^(-2i/d)."""
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    h = d // 2
    theta = np.power(F64(base), -2.0 * np.arange(h, dtype=F64) / d)
    ang = np.multiply.outer(np.asarray(pos, dtype=F64), theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------
# tree [tree], [pooler]
# ----------------------------------------------------------------------------
def pool_keys(children: np.ndarray, w: np.ndarray, pool_scale: float) -> np.ndarray:
    """Attention pooling of children[n][b][d] with vector w[d] -> keys[n][d] (unrounded).

    alpha_c = softmax over the b children of pool_scale * (w . child_c);
    key = sum_c alpha_c * child_c.  One w serves every level ([pooler]).
    """
    children = np.asarray(children, dtype=F64)
    logits = pool_scale * (children * np.asarray(w, dtype=F64)).sum(axis=-1)      # [n][b]
    logits = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    alpha = e / e.sum(axis=1, keepdims=True)
    return (alpha[:, :, None] * children).sum(axis=1)


def subtree_means(V: np.ndarray, level: int, b: int, n0: int, n1: int) -> np.ndarray:
    """Mean of V over each node's tokens, for level-`level` nodes [n0, n1) ([tree])."""
    span = b ** level
    blk = np.asarray(V[n0 * span:n1 * span], dtype=F64).reshape(n1 - n0, span, -1)
    return blk.sum(axis=1) / span


@dataclasses.dataclass
class Tree:
    """Summaries of every KV head: keys[l][g] and vals[l][g] are [N_l][d]
    float64 arrays holding storage-format values; level 0 is the token cache."""
    b: int
    store: str
    pool_scale: float
    w: np.ndarray                  # [n_kv][d]
    keys: list                     # keys[l] : list over heads of [N_l][d]
    vals: list
    length: int

    @property
    def n_kv(self) -> int:
        return len(self.keys[0])


def build_tree(K: np.ndarray, V: np.ndarray, w: np.ndarray, b: int, store: str,
               pool_scale: float, length: int) -> Tree:
    """Tree over the first `length` tokens of K, V [n_kv][>=length][d]."""
    tree = Tree(b=b, store=store, pool_scale=pool_scale, w=np.asarray(w, F64),
                keys=[[np.asarray(K[g][:0], F64) for g in range(len(K))]],
                vals=[[np.asarray(V[g][:0], F64) for g in range(len(V))]], length=0)
    return extend_tree(tree, K, V, length)


def extend_tree(tree: Tree, K: np.ndarray, V: np.ndarray, new_length: int) -> Tree:
    """Grow the tree to `new_length` tokens: store the new tokens and summarize
    every node that became complete, lowest level first.  Existing nodes are
    never touched (a complete node's subtree never changes)."""
    b = tree.b
    old, new = level_sizes(tree.length, b), level_sizes(new_length, b)
    for g in range(tree.n_kv):
        tree.keys[0][g] = np.asarray(K[g][:new_length], F64)
        tree.vals[0][g] = np.asarray(V[g][:new_length], F64)
    for l in range(1, len(new)):
        if len(tree.keys) <= l:
            tree.keys.append([np.zeros((0, K.shape[-1])) for _ in range(tree.n_kv)])
            tree.vals.append([np.zeros((0, K.shape[-1])) for _ in range(tree.n_kv)])
        n0 = old[l] if l < len(old) else 0
        n1 = new[l]
        if n1 == n0:
            continue
        for g in range(tree.n_kv):
            child = tree.keys[l - 1][g][n0 * b:n1 * b].reshape(n1 - n0, b, -1)
            k_new = round_store(pool_keys(child, tree.w[g], tree.pool_scale), tree.store)
            v_new = round_store(subtree_means(tree.vals[0][g], l, b, n0, n1), tree.store)
            tree.keys[l][g] = np.concatenate([tree.keys[l][g][:n0], k_new])
            tree.vals[l][g] = np.concatenate([tree.vals[l][g][:n0], v_new])
    tree.length = new_length
    return tree


# ----------------------------------------------------------------------------
# descent and mixed softmax [selection], [rope]
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class LevelTrace:
    level: int
    cand: np.ndarray        # node ids (token ids at level 0), in candidate order
    z: np.ndarray           # logits, one per candidate
    sel_pos: np.ndarray     # selected candidate positions, ascending (empty at level 0)
    gap: float              # z_(m) - z_(m+1) in sorted order; nan if nothing is left out


@dataclasses.dataclass
class RowResult:
    out: np.ndarray
    levels: list            # LevelTrace, top level first, level 0 last
    entry_z: np.ndarray
    entry_level: np.ndarray
    entry_node: np.ndarray

    @property
    def keys_read(self) -> int:
        return int(sum(len(t.cand) for t in self.levels))

    @property
    def max_position(self) -> int:
        return int(max(len(t.cand) for t in self.levels))

    def selected_nodes(self, level: int) -> np.ndarray:
        for t in self.levels:
            if t.level == level:
                return t.cand[t.sel_pos]
        return np.zeros(0, np.int64)


def descend(tree: Tree, q: np.ndarray, g: int, n_ctx: int, k: int, base: float,
            scale: float, force: dict | None = None) -> RowResult:
    """One query row of KV head g against the first n_ctx tokens.

    Per level l = H..1: score every candidate with its candidate-index RoPE
    and the query at the level's candidate count; keep the min(k, n) best;
    every other candidate becomes a softmax entry with its summary value; the
    kept nodes' children, then the level's orphans, form the next candidates.
    Level 0: every candidate token is an entry with its exact value.  One
    softmax runs over all the entries.  `force` maps level -> node ids to select
    instead (replay of another selection).
    """
    b = tree.b
    N = level_sizes(n_ctx, b)
    H = len(N) - 1
    q = np.asarray(q, dtype=F64)
    cand = np.arange(N[H], dtype=np.int64)
    traces, ez, ev, elev, enode = [], [], [], [], []
    for l in range(H, -1, -1):
        n = len(cand)
        qr = rope(q, n, base)
        kr = rope(tree.keys[l][g][cand], np.arange(n), base)
        z = scale * (kr @ qr)
        if l == 0:
            traces.append(LevelTrace(0, cand, z, np.zeros(0, np.int64), float("nan")))
            ez.append(z)
            ev.append(tree.vals[0][g][cand])
            elev.append(np.zeros(n, np.int64))
            enode.append(cand)
            break
        m = min(k, n)
        order = np.lexsort((np.arange(n), -z))            # z descending, index ascending
        gap = float(z[order[m - 1]] - z[order[m]]) if n > m else float("nan")
        if force is not None and l in force:
            sel = np.searchsorted(cand, np.asarray(force[l], np.int64))
            if len(sel) != m or np.any(cand[np.minimum(sel, n - 1)] != np.asarray(force[l])):
                raise ValueError(f"forced selection at level {l} is not a candidate set")
        else:
            sel = np.sort(order[:m])
        traces.append(LevelTrace(l, cand, z, sel, gap))
        keep = np.ones(n, bool)
        keep[sel] = False
        ez.append(z[keep])
        ev.append(tree.vals[l][g][cand[keep]])
        elev.append(np.full(int(keep.sum()), l, np.int64))
        enode.append(cand[keep])
        children = (cand[sel][:, None] * b + np.arange(b)).reshape(-1)
        orphans = np.arange(b * N[l], N[l - 1], dtype=np.int64)
        cand = np.concatenate([children, orphans])
    z_all = np.concatenate(ez)
    v_all = np.concatenate(ev)
    e = np.exp(z_all - z_all.max())
    out = (e @ v_all) / e.sum()
    return RowResult(out, traces, z_all, np.concatenate(elev), np.concatenate(enode))


def decode(tree: Tree, Q: np.ndarray, k: int, base: float, scale: float,
           n_ctx: int | None = None, rows=None, force=None) -> tuple[np.ndarray, dict]:
    """Decode queries Q[B][n_q][d] against the whole tree (all at position
    `n_ctx`, default the tree length).  Query head h reads KV head
    h // (n_q / n_kv).  Returns out[B][n_q][d] (rows not listed stay nan) and
    the per-row results."""
    Q = np.asarray(Q, F64)
    B, nq, d = Q.shape
    G = nq // tree.n_kv
    n_ctx = tree.length if n_ctx is None else n_ctx
    rows = [(i, h) for i in range(B) for h in range(nq)] if rows is None else rows
    out = np.full((B, nq, d), np.nan)
    res = {}
    for (i, h) in rows:
        f = None if force is None else force.get((i, h))
        r = descend(tree, Q[i, h], h // G, n_ctx, k, base, scale, force=f)
        out[i, h] = r.out
        res[(i, h)] = r
    return out, res


# ----------------------------------------------------------------------------
# variant: one selection shared by the query heads of a KV group
# ----------------------------------------------------------------------------
# Prior art, not the RecSA pages' rule: the MiniMax Sparse Attention abstract (on
# the search-results page for "coarse attention block") selects its top-k once
# per GQA group.  The pages do not say how a group's heads combine into one
# score; the reading taken here is the plainest one that keeps each head's
# softmax intact:
#   * the group's score of a candidate is the sum of its G heads' logits (by
#     linearity of RoPE and the inner product, the logit of the summed query);
#   * equal scores go to the lower candidate index, as per head;
#   * every head keeps its own logits for its own softmax over the shared
#     entry set, and its own output.
@dataclasses.dataclass
class GroupResult:
    out: np.ndarray         # [G][d], one output per head of the group
    levels: list            # LevelTrace over the group score, top level first
    head_z: list            # per level (same order): logits [G][n_candidates]

    def selected_nodes(self, level: int) -> np.ndarray:
        for t in self.levels:
            if t.level == level:
                return t.cand[t.sel_pos]
        return np.zeros(0, np.int64)


def descend_group(tree: Tree, Qg: np.ndarray, g: int, n_ctx: int, k: int, base: float,
                  scale: float, force: dict | None = None) -> GroupResult:
    """Query rows Qg[G][d] of the heads that read KV head g, with one shared
    selection per level.  The levels, candidates, entries and RoPE positions
    are those of `descend`; only the selection score differs (the sum of the
    heads' logits), and each head's entries carry its own logits.  `force`
    maps level -> node ids to select instead, as in `descend`."""
    b = tree.b
    N = level_sizes(n_ctx, b)
    H = len(N) - 1
    Qg = np.asarray(Qg, dtype=F64)
    G = Qg.shape[0]
    cand = np.arange(N[H], dtype=np.int64)
    traces, head_z = [], []
    ez = [[] for _ in range(G)]
    ev = []
    for l in range(H, -1, -1):
        n = len(cand)
        kr = rope(tree.keys[l][g][cand], np.arange(n), base)
        z = np.stack([scale * (kr @ rope(Qg[h], n, base)) for h in range(G)])   # [G][n]
        head_z.append(z)
        if l == 0:
            traces.append(LevelTrace(0, cand, z.sum(axis=0), np.zeros(0, np.int64), float("nan")))
            for h in range(G):
                ez[h].append(z[h])
            ev.append(tree.vals[0][g][cand])
            break
        s = z.sum(axis=0)
        m = min(k, n)
        order = np.lexsort((np.arange(n), -s))
        gap = float(s[order[m - 1]] - s[order[m]]) if n > m else float("nan")
        if force is not None and l in force:
            sel = np.searchsorted(cand, np.asarray(force[l], np.int64))
            if len(sel) != m or np.any(cand[np.minimum(sel, n - 1)] != np.asarray(force[l])):
                raise ValueError(f"forced selection at level {l} is not a candidate set")
        else:
            sel = np.sort(order[:m])
        traces.append(LevelTrace(l, cand, s, sel, gap))
        keep = np.ones(n, bool)
        keep[sel] = False
        for h in range(G):
            ez[h].append(z[h][keep])
        ev.append(tree.vals[l][g][cand[keep]])
        children = (cand[sel][:, None] * b + np.arange(b)).reshape(-1)
        orphans = np.arange(b * N[l], N[l - 1], dtype=np.int64)
        cand = np.concatenate([children, orphans])
    v_all = np.concatenate(ev)
    out = np.zeros((G, v_all.shape[1]))
    for h in range(G):
        z_all = np.concatenate(ez[h])
        e = np.exp(z_all - z_all.max())
        out[h] = (e @ v_all) / e.sum()
    return GroupResult(out, traces, head_z)


def decode_group(tree: Tree, Q: np.ndarray, k: int, base: float, scale: float,
                 n_ctx: int | None = None, groups=None) -> tuple[np.ndarray, dict]:
    """Decode queries Q[B][n_q][d] with one selection per (query, KV group):
    query heads g*G .. g*G + G - 1 share it.  Returns out[B][n_q][d] (heads of
    groups not listed stay nan) and the per-(query, group) results."""
    Q = np.asarray(Q, F64)
    B, nq, d = Q.shape
    G = nq // tree.n_kv
    n_ctx = tree.length if n_ctx is None else n_ctx
    groups = [(i, g) for i in range(B) for g in range(tree.n_kv)] if groups is None else groups
    out = np.full((B, nq, d), np.nan)
    res = {}
    for (i, g) in groups:
        r = descend_group(tree, Q[i, g * G:(g + 1) * G], g, n_ctx, k, base, scale)
        out[i, g * G:(g + 1) * G] = r.out
        res[(i, g)] = r
    return out, res


def prefill(tree: Tree, Q: np.ndarray, k: int, base: float, scale: float,
            rows=None, force=None) -> tuple[np.ndarray, dict]:
    """Causal chunk: Q[n][n_q][d] are the queries of the last n tokens of the
    tree; query j attends to tokens [0, L0 + j] (its own included), L0 =
    length - n, through the tree of that prefix (complete nodes only)."""
    Q = np.asarray(Q, F64)
    n, nq, d = Q.shape
    G = nq // tree.n_kv
    L0 = tree.length - n
    rows = [(j, h) for j in range(n) for h in range(nq)] if rows is None else rows
    out = np.full((n, nq, d), np.nan)
    res = {}
    for (j, h) in rows:
        f = None if force is None else force.get((j, h))
        r = descend(tree, Q[j, h], h // G, L0 + j + 1, k, base, scale, force=f)
        out[j, h] = r.out
        res[(j, h)] = r
    return out, res


def prefill_sequential(K, V, w, b, store, pool_scale, L0, Q, k, base, scale):
    """The same chunk computed literally: append one token, then run that
    token's query against the tree as it stands, and repeat."""
    Q = np.asarray(Q, F64)
    n, nq, d = Q.shape
    G = nq // len(K)
    tree = build_tree(K, V, w, b, store, pool_scale, L0)
    out = np.zeros((n, nq, d))
    for j in range(n):
        extend_tree(tree, K, V, L0 + j + 1)
        for h in range(nq):
            out[j, h] = descend(tree, Q[j, h], h // G, L0 + j + 1, k, base, scale).out
    return out


# ----------------------------------------------------------------------------
# backward through the mixed softmax, the selection held fixed
# ----------------------------------------------------------------------------
# The pages train RecSA end to end from a Qwen3-4B initialisation (abstract,
# sentence on evaluation), which needs the gradient of the attention output with
# respect to the query, the token keys and values and the pooler.  The pages give
# no formula; the readings taken here:
#   * the kept sets are held fixed: selection is piecewise constant in its
#     inputs, so only the softmax entries carry gradient;
#   * rounding a summary to the storage format passes the gradient through
#     unchanged;
#   * a summary key depends on its stored children's keys and on w through the
#     pooler, and a summary value is the mean of its subtree's token values, so
#     gradients reaching summaries flow down the tree to the tokens and to w.
# With z = s <rope(q, n), rope(key, i)> = s q . R_(i-n) key (rotations compose):
#   dz/dq = s rope(key, i - n),   dz/dkey = s rope(q, n - i).
def backward_row(tree: Tree, q: np.ndarray, g: int, n_ctx: int, k: int, base: float, scale: float,
                 dout: np.ndarray, gk: list, gv: list, force: dict | None = None) -> np.ndarray:
    """Gradient of <dout, out> for one query row of KV head g.  Adds the
    gradients of its entries' keys and values into gk[l][g], gv[l][g] (level 0:
    tokens) and returns d/dq."""
    q = np.asarray(q, F64)
    dout = np.asarray(dout, F64)
    res = descend(tree, q, g, n_ctx, k, base, scale, force=force)
    p = np.exp(res.entry_z - res.entry_z.max())
    p /= p.sum()
    D = float(dout @ res.out)
    dq = np.zeros_like(q)
    e = 0
    for lt in res.levels:
        n = len(lt.cand)
        keep = np.ones(n, bool)
        keep[lt.sel_pos] = False
        for i in np.nonzero(keep)[0]:
            node = int(lt.cand[i])
            key = tree.keys[lt.level][g][node]
            val = tree.vals[lt.level][g][node]
            dz = p[e] * (float(dout @ val) - D)
            dq += dz * scale * rope(key, i - n, base)
            gk[lt.level][g][node] += dz * scale * rope(q, n - i, base)
            gv[lt.level][g][node] += p[e] * dout
            e += 1
    assert e == len(p)
    return dq


def backward_tree(tree: Tree, gk: list, gv: list) -> np.ndarray:
    """Push the summaries' gradients down the tree, top level first: a node's
    value is the mean of its b children's (its subtree's tokens), and its key is
    the pooler over its b stored children's keys.  Leaves token gradients in
    gk[0], gv[0] and returns d/dw [n_kv][d]."""
    b = tree.b
    dw = np.zeros_like(tree.w)
    for l in range(len(tree.keys) - 1, 0, -1):
        for g in range(tree.n_kv):
            w = tree.w[g]
            for j in range(len(tree.keys[l][g])):
                x = tree.keys[l - 1][g][j * b:(j + 1) * b]          # the stored children
                a = tree.pool_scale * (x @ w)
                alpha = np.exp(a - a.max())
                alpha /= alpha.sum()
                gkey = gk[l][g][j]
                dalpha = x @ gkey
                da = alpha * (dalpha - alpha @ dalpha)
                gk[l - 1][g][j * b:(j + 1) * b] += np.outer(alpha, gkey) + tree.pool_scale * np.outer(da, w)
                dw[g] += tree.pool_scale * (da @ x)
                gv[l - 1][g][j * b:(j + 1) * b] += gv[l][g][j] / b
    return dw


def backward(tree: Tree, Q: np.ndarray, dO: np.ndarray, k: int, base: float, scale: float,
             causal: bool = False, rows=None, force=None) -> dict:
    """Gradients of sum <dO, out> for decode queries Q[n][n_q][d] at the tree's
    length (causal=False) or for the causal chunk of the last n tokens
    (causal=True, query j at n_ctx = length - n + j + 1).  Returns dict with
    dq [n][n_q][d], dk and dv [n_kv][length][d] and dw [n_kv][d]."""
    Q = np.asarray(Q, F64)
    n, nq, d = Q.shape
    G = nq // tree.n_kv
    gk = [[np.zeros_like(a) for a in lev] for lev in tree.keys]
    gv = [[np.zeros_like(a) for a in lev] for lev in tree.vals]
    dq = np.zeros((n, nq, d))
    rows = [(i, h) for i in range(n) for h in range(nq)] if rows is None else rows
    for (i, h) in rows:
        n_ctx = tree.length - n + i + 1 if causal else tree.length
        f = None if force is None else force.get((i, h))
        dq[i, h] = backward_row(tree, Q[i, h], h // G, n_ctx, k, base, scale, dO[i, h], gk, gv, f)
    dw = backward_tree(tree, gk, gv)
    return {"dq": dq, "dk": np.stack(gk[0]), "dv": np.stack(gv[0]), "dw": dw}


# ----------------------------------------------------------------------------
# pooler distillation from dense attention
# ----------------------------------------------------------------------------
# The pages distill the per-layer pooler from dense attention (abstract, sentence
# on the pooler) and give no objective.  Reading: on a set of training queries at
# the cache's length, the pooler vectors w are fitted so that RecSA's output
# matches dense attention's output,
#   loss = (1 / rows) sum_rows || out_recsa(q) - out_dense(q) ||^2,
# its gradient in w taken with the selection held fixed (the backward above) and
# the tree rebuilt from the new w after each step; the optimizer is SGD with
# momentum: vel <- mu vel + dloss/dw, w <- w - lr vel.
def distill_loss(tree: Tree, Q: np.ndarray, teacher: np.ndarray, k: int, base: float,
                 scale: float, force=None) -> tuple[float, dict]:
    """Loss of the decode queries Q[B][n_q][d] against teacher outputs, and the
    gradients (backward's dict, dw included) of that loss."""
    Q = np.asarray(Q, F64)
    out, _ = decode(tree, Q, k, base, scale,
                    force=None if force is None else force)
    rows = Q.shape[0] * Q.shape[1]
    diff = out - np.asarray(teacher, F64)
    loss = float((diff ** 2).sum() / rows)
    grads = backward(tree, Q, 2.0 * diff / rows, k, base, scale, force=force)
    return loss, grads


def sgd_momentum(w, vel, grad, lr, mu):
    """Heavy-ball SGD, the update of the distillation reading: the velocity first
    takes mu times itself plus the gradient, then w moves by -lr times the new
    velocity (no dampening, no look-ahead).  Returns (new w, new velocity)."""
    vel = mu * np.asarray(vel, F64) + np.asarray(grad, F64)
    return np.asarray(w, F64) - lr * vel, vel


def distill_step(K, V, w, b, store, pool_scale, L, Q, teacher, k, base, scale, lr, mu, vel,
                 force=None):
    """One step: build the tree from w, the loss and dloss/dw (selection held at
    `force` where given), then the update.  Returns (loss before the step, new w,
    new velocity)."""
    tree = build_tree(K, V, w, b, store, pool_scale, L)
    loss, grads = distill_loss(tree, Q, teacher, k, base, scale, force=force)
    w_new, vel = sgd_momentum(w, vel, grads["dw"], lr, mu)
    return loss, w_new, vel


# ----------------------------------------------------------------------------
# dense causal attention (the comparison point of the pages' speed claim)
# ----------------------------------------------------------------------------
def dense(q: np.ndarray, K: np.ndarray, V: np.ndarray, n: int, base: float, scale: float):
    """Softmax over tokens i < n of s*<rope(q, n), rope(K_i, i)>, applied to V."""
    qr = rope(np.asarray(q, F64), n, base)
    kr = rope(np.asarray(K[:n], F64), np.arange(n), base)
    z = scale * (kr @ qr)
    e = np.exp(z - z.max())
    return (e @ np.asarray(V[:n], F64)) / e.sum()
