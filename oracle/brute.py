"""The decode step in pure-Python loops, for tiny inputs — oracle only.

Same definition as ``oracle.decode.decode_ref`` ([es §2.B], [fr §2.B],
[de §2.B]) written with explicit sums, an explicit sort and math.exp, and no
NumPy, so a mistake in the vectorised version (a transposed operand, a wrong
head slice, a dropped text term) shows up as a disagreement.  Inputs are
nested lists (or anything indexable); sizes must stay tiny (N <= ~16).
"""
from __future__ import annotations

import math


def decode_brute(U_k, B_k, U_v, B_v, q, n_kv_heads, head_dim, r_lo, top_k, scale,
                 text_k=(), text_v=(), keys=None, weights=None):
    """keys: optional per-head importance lists to rank by instead of the low-rank
    score; weights: if a list is given, each head's visual attention weights are
    appended to it."""
    N = len(U_k)
    r = len(B_k)
    d = head_dim
    Hq = len(q) // d
    G = Hq // n_kv_heads
    T = len(text_k)
    out = [0.0] * (Hq * d)
    tops = []
    for h in range(Hq):
        g = h // G
        qh = [float(q[h * d + j]) for j in range(d)]

        def khat(n, rank):
            return [sum(float(U_k[n][i]) * float(B_k[i][g * d + j]) for i in range(rank))
                    for j in range(d)]

        def vhat(n, rank):
            return [sum(float(U_v[n][i]) * float(B_v[i][g * d + j]) for i in range(rank))
                    for j in range(d)]

        def dot(a, b):
            return sum(x * y for x, y in zip(a, b))

        s_lo = [scale * dot(khat(n, r_lo), qh) for n in range(N)]
        rank_by = s_lo if keys is None else [float(x) for x in keys[h]]
        ranked = sorted(range(N), key=lambda n: (-rank_by[n], n))
        top = sorted(ranked[:top_k])
        chosen = set(top)
        scores = []
        for n in range(N):
            scores.append(scale * dot(khat(n, r), qh) if n in chosen else s_lo[n])
        for t in range(T):
            kt = [float(text_k[t][g * d + j]) for j in range(d)]
            scores.append(scale * dot(kt, qh))
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        z = sum(w)
        o = [0.0] * d
        for n in range(N):
            v = vhat(n, r if n in chosen else r_lo)
            for j in range(d):
                o[j] += w[n] / z * v[j]
        for t in range(T):
            for j in range(d):
                o[j] += w[N + t] / z * float(text_v[t][g * d + j])
        out[h * d:(h + 1) * d] = o
        tops.append(top)
        if weights is not None:
            weights.append([w[n] / z for n in range(N)])
    return out, tops


def decode_ema_brute(U_k, B_k, U_v, B_v, qs, n_kv_heads, head_dim, r_lo, top_k, scale,
                     alpha, per_head, text_k=(), text_v=()):
    """Several steps of the moving-average selector with explicit loops: the first
    step ranks by the low-rank score and sets the importance to its attention
    weights; later steps rank by the importance, then blend in their own weights."""
    d = head_dim
    Hq = len(qs[0]) // d
    N = len(U_k)
    imp = None
    outs, tops_all, states = [], [], []
    for q in qs:
        if imp is None:
            keys = None
        elif per_head:
            keys = imp
        else:
            keys = [imp for _ in range(Hq)]
        wts = []
        out, tops = decode_brute(U_k, B_k, U_v, B_v, q, n_kv_heads, head_dim, r_lo, top_k,
                                 scale, text_k, text_v, keys=keys, weights=wts)
        if per_head:
            new = wts
        else:
            new = [sum(wts[h][n] for h in range(Hq)) / Hq for n in range(N)]
        if imp is None:
            imp = new
        elif per_head:
            imp = [[alpha * imp[h][n] + (1.0 - alpha) * new[h][n] for n in range(N)] for h in range(Hq)]
        else:
            imp = [alpha * imp[n] + (1.0 - alpha) * new[n] for n in range(N)]
        outs.append(out)
        tops_all.append(tops)
        states.append([list(row) for row in imp] if per_head else list(imp))
    return outs, tops_all, states


def decode_segments_brute(segments, q, n_kv_heads, head_dim, scale, dense_k=(), dense_v=()):
    """Several factored segments plus dense tokens, with explicit loops: per segment and
    head, rank its tokens by the low-rank score (its own r_lo, top_k), score each token
    at its rank, then one softmax over every segment's tokens and the dense ones."""
    d = head_dim
    Hq = len(q) // d
    G = Hq // n_kv_heads
    out = [0.0] * (Hq * d)
    tops = [[] for _ in segments]
    for h in range(Hq):
        g = h // G
        qh = [float(q[h * d + j]) for j in range(d)]

        def dot(a, b):
            return sum(x * y for x, y in zip(a, b))

        scores, values = [], []
        for si, sg in enumerate(segments):
            Uk, Bk, Uv, Bv = sg["U_k"], sg["B_k"], sg["U_v"], sg["B_v"]
            r_lo, k = sg["r_lo"], sg["top_k"]
            N, r = len(Uk), len(Bk)

            def rec(U, B, n, rank):
                return [sum(float(U[n][i]) * float(B[i][g * d + j]) for i in range(rank)) for j in range(d)]

            s_lo = [scale * dot(rec(Uk, Bk, n, r_lo), qh) for n in range(N)]
            ranked = sorted(range(N), key=lambda n: (-s_lo[n], n))
            chosen = set(ranked[:k])
            tops[si].append(sorted(chosen))
            for n in range(N):
                rank = r if n in chosen else r_lo
                scores.append(scale * dot(rec(Uk, Bk, n, rank), qh))
                values.append(rec(Uv, Bv, n, rank))
        for t in range(len(dense_k)):
            scores.append(scale * dot([float(dense_k[t][g * d + j]) for j in range(d)], qh))
            values.append([float(dense_v[t][g * d + j]) for j in range(d)])
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        z = sum(w)
        for j in range(d):
            out[h * d + j] = sum(w[i] / z * values[i][j] for i in range(len(w)))
    return out, tops
