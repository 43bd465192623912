"""Brute-force RecSA for tiny inputs, in pure Python floats (f64).

Written separately from the oracle to pin it: lists and the math module
only, and the per-level selection found by enumerating every subset of the
allowed size rather than by sorting.  A subset is chosen when its summed
logit is largest; among equal sums the lexicographically smallest index
tuple wins, which is the same set as "the k best, equal scores to the lower
candidate index" (RecSA abstract, the sentence on selecting at most k
candidates per level).
"""
import itertools
import math
import struct


def _f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def _rot(vec, pos, base):
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        a = pos * base ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        out[i] = vec[i] * c - vec[i + h] * s
        out[i + h] = vec[i + h] * c + vec[i] * s
    return out


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def sizes(n, b):
    out = [n]
    while out[-1] >= b:
        out.append(out[-1] // b)
    return out


def build(K, V, w, b, pool_scale, n, round_f32=True):
    """keys[l][j], vals[l][j] as lists of float lists for one head."""
    N = sizes(n, b)
    keys = [[list(r) for r in K[:n]]]
    vals = [[list(r) for r in V[:n]]]
    for l in range(1, len(N)):
        kl, vl = [], []
        for j in range(N[l]):
            ch = keys[l - 1][j * b:(j + 1) * b]
            logit = [pool_scale * _dot(w, c) for c in ch]
            mx = max(logit)
            e = [math.exp(x - mx) for x in logit]
            tot = sum(e)
            key = [sum(e[c] / tot * ch[c][t] for c in range(b)) for t in range(len(w))]
            toks = V[j * b ** l:(j + 1) * b ** l]
            val = [sum(r[t] for r in toks) / len(toks) for t in range(len(w))]
            if round_f32:
                key = [_f32(x) for x in key]
                val = [_f32(x) for x in val]
            kl.append(key)
            vl.append(val)
        keys.append(kl)
        vals.append(vl)
    return keys, vals


def row(keys, vals, q, n_ctx, b, k, base, scale):
    """Returns (out, selections {level: [node ids]}, entries [(level, node)])."""
    N = sizes(n_ctx, b)
    H = len(N) - 1
    cand = list(range(N[H]))
    zs, vs, sels, entries = [], [], {}, []
    for l in range(H, -1, -1):
        n = len(cand)
        qr = _rot(q, n, base)
        z = [scale * _dot(qr, _rot(keys[l][c], i, base)) for i, c in enumerate(cand)]
        if l == 0:
            for i, c in enumerate(cand):
                zs.append(z[i])
                vs.append(vals[0][c])
                entries.append((0, c))
            break
        m = min(k, n)
        best, best_key = None, None
        for sub in itertools.combinations(range(n), m):
            key = (sum(z[i] for i in sub), [-i for i in sub])
            if best is None or key > best_key:
                best, best_key = sub, key
        sels[l] = [cand[i] for i in best]
        for i, c in enumerate(cand):
            if i not in best:
                zs.append(z[i])
                vs.append(vals[l][c])
                entries.append((l, c))
        nxt = [cand[i] * b + c for i in best for c in range(b)]
        nxt += list(range(b * N[l], N[l - 1]))
        cand = nxt
    mx = max(zs)
    e = [math.exp(x - mx) for x in zs]
    tot = sum(e)
    d = len(q)
    out = [sum(e[i] * vs[i][t] for i in range(len(e))) / tot for t in range(d)]
    return out, sels, entries
