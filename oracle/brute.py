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
                 text_k=(), text_v=()):
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
        ranked = sorted(range(N), key=lambda n: (-s_lo[n], n))
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
    return out, tops
