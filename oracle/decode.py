"""One decode step of attention over a compressed visual cache — oracle only.

What is computed ([es §2.B], [fr §2.B "Stratégie"], [de §2.B "Mechanismus"]):
at each decoding step every visual token is decompressed from its factors;
the important tokens are decompressed at the full rank R and the others at a
reduced rank (the French page gives R/4 as the example); attention then runs
over the decompressed keys and values.  25% of the tokens at full rank is the
setting the Spanish page reports ([es §4 "Análisis de Sensibilidad"]).

Readings taken where the summaries are open:
  * importance of a token for query head h at this step = its low-rank
    attention logit s_lo (the score from the first r_lo components).  The
    summaries instead keep a moving average of accumulated attention scores
    (parameter alpha, never given); ranking by the current low-rank logit is
    the plainest stateless stand-in, and softmax is monotone, so ranking
    logits ranks low-rank attention weights.
  * selection is per query head; ties go to the lower token index;
  * the same selected set is used for K and for V;
  * "first r_lo components" = the r_lo components of largest singular value
    (columns 0..r_lo-1 of U, rows 0..r_lo-1 of B);
  * query head h reads KV head g = h // (Hq / Hkv): columns g*d..(g+1)*d of B;
  * dense text tokens (the summaries compress text separately, [fr §2.A
    "Traitement séparé"]; here they stay uncompressed) join the softmax at
    full precision and are never selected or reduced.

Explicit decompression, in float64:
  K_lo = U_k[:, :r_lo] B_k,g[:r_lo],  K_full = U_k B_k,g          (N x d)
  s_lo = scale * K_lo q_h;   Top_h = top_k largest s_lo
  s[n] = scale * K_full[n] q_h if n in Top_h else s_lo[n];  text s_t = scale * K_t,g q_h
  p    = softmax([s; s_t])
  o_h  = sum_n p[n] Vhat_{r(n)}[n] + sum_t p_t V_t,g[t],   r(n) = r if n in Top_h else r_lo
"""
from __future__ import annotations

import numpy as np


def select_top(s_lo: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores (ties: lower index first), ascending."""
    n = np.arange(s_lo.shape[0])
    order = np.lexsort((n, -s_lo))   # primary key -s_lo, then index
    return np.sort(order[:k])


def decode_ref(U_k, B_k, U_v, B_v, q, n_kv_heads: int, head_dim: int, r_lo: int,
               top_k: int, scale: float, text_k=None, text_v=None, select_keys=None):
    """Decode one query vector q [Hq*d] for one sequence.

    U_k, U_v: N x r;  B_k, B_v: r x (Hkv*d);  text_k, text_v: T x (Hkv*d).
    select_keys: optional [Hq][N] importance to rank tokens by instead of s_lo
    (the moving-average selector, see ``decode_ema_steps``).
    Returns dict(out [Hq*d], top [Hq][top_k] ascending ids, s_lo [Hq][N],
    p [Hq][N] the attention weight of each visual token, text included in the
    normalisation).
    """
    U_k = np.asarray(U_k, np.float64); B_k = np.asarray(B_k, np.float64)
    U_v = np.asarray(U_v, np.float64); B_v = np.asarray(B_v, np.float64)
    q = np.asarray(q, np.float64)
    N, r = U_k.shape
    d = head_dim
    Hq = q.shape[0] // d
    G = Hq // n_kv_heads
    T = 0 if text_k is None else np.asarray(text_k).shape[0]
    if T:
        text_k = np.asarray(text_k, np.float64)
        text_v = np.asarray(text_v, np.float64)
    out = np.zeros(Hq * d)
    tops, s_los, ps = [], [], []
    for h in range(Hq):
        g = h // G
        cols = slice(g * d, (g + 1) * d)
        qh = q[h * d:(h + 1) * d]
        K_lo = U_k[:, :r_lo] @ B_k[:r_lo, cols]
        K_full = U_k @ B_k[:, cols]
        V_lo = U_v[:, :r_lo] @ B_v[:r_lo, cols]
        V_full = U_v @ B_v[:, cols]
        s_lo = scale * (K_lo @ qh)
        top = select_top(s_lo if select_keys is None else np.asarray(select_keys[h], np.float64), top_k)
        s = s_lo.copy()
        s[top] = scale * (K_full[top] @ qh)
        V_sel = V_lo.copy()
        V_sel[top] = V_full[top]
        if T:
            s_all = np.concatenate([s, scale * (text_k[:, cols] @ qh)])
        else:
            s_all = s
        p = np.exp(s_all - s_all.max())
        p /= p.sum()
        o = p[:N] @ V_sel
        if T:
            o = o + p[N:] @ text_v[:, cols]
        out[h * d:(h + 1) * d] = o
        tops.append(top)
        s_los.append(s_lo)
        ps.append(p[:N])
    return dict(out=out, top=np.array(tops, dtype=np.int64).reshape(Hq, top_k),
                s_lo=np.array(s_los), p=np.array(ps))


def decode_ema_steps(U_k, B_k, U_v, B_v, qs, n_kv_heads: int, head_dim: int, r_lo: int,
                     top_k: int, scale: float, alpha: float, per_head: bool,
                     text_k=None, text_v=None, state=None):
    """Several decode steps with the moving-average importance selector.

    [es §2.B], [fr §2.B "Score d'importance"], [de §2.B "Mechanismus"]: each token's
    importance is a moving average, with parameter alpha, of the attention it has
    received; the tokens of highest importance are decompressed at full rank.
    Readings where the pages are open: the average is taken over the attention weights
    p of each step, I <- alpha * I + (1 - alpha) * p; a step selects with the
    importance left by the steps before it; the first step (state None) has no
    history and selects by its own low-rank logit, and then I = p.  per_head: one
    importance per (query head, token), else one per token, fed with the mean of
    the query heads' weights and shared by all of them.

    qs: [steps][Hq*d].  Returns (list of decode_ref results, state after each step:
    [Hq][N] per head, [N] shared).
    """
    results, states = [], []
    I = None if state is None else np.asarray(state, np.float64).copy()
    Hq = np.asarray(qs[0]).shape[0] // head_dim
    for q in qs:
        keys = None
        if I is not None:
            keys = I if per_head else np.broadcast_to(I, (Hq, I.shape[-1]))
        res = decode_ref(U_k, B_k, U_v, B_v, q, n_kv_heads, head_dim, r_lo, top_k, scale,
                         text_k, text_v, select_keys=keys)
        p = res["p"] if per_head else res["p"].mean(axis=0)
        I = p.copy() if I is None else alpha * I + (1.0 - alpha) * p
        results.append(res)
        states.append(I.copy())
    return results, states


def band_mask(s_lo_h: np.ndarray, k: int, rel: float = 1e-3) -> np.ndarray:
    """Tokens whose low-rank score is within rel of the k-th largest (the cutoff).

    |s - tau| <= rel * max(|tau|, rel * max|s|); the absolute floor keeps the
    band meaningful when the cutoff is near zero.
    """
    if k == 0 or k >= s_lo_h.shape[0]:
        return np.zeros(s_lo_h.shape[0], dtype=bool)
    tau = np.sort(s_lo_h)[::-1][k - 1]
    tol = rel * max(abs(tau), rel * float(np.max(np.abs(s_lo_h))))
    return np.abs(s_lo_h - tau) <= tol


def recon_error(A, U, B) -> float:
    """Relative Frobenius error ||A - U B||_F / ||A||_F in float64."""
    A = np.asarray(A, np.float64)
    R = A - np.asarray(U, np.float64) @ np.asarray(B, np.float64)
    return float(np.linalg.norm(R) / np.linalg.norm(A))


def decode_segments(segments, q, n_kv_heads: int, head_dim: int, scale: float,
                    dense_k=None, dense_v=None):
    """One decode step over several separately factored segments plus dense tokens.

    [es §2.A], [fr §2.A "Traitement séparé"], [de §2.A "Optimierung"]: visual and
    text tokens are factored by separate SVDs.  Each segment here is a dict with its
    own factors U_k, B_k, U_v, B_v (its own rank) and its own reduced rank r_lo and
    full-rank count top_k; the attention-aware decompression of [fr §2.B] is applied
    inside each segment (its top_k tokens by its own low-rank score, per query head,
    ties to the lower index).  Dense tokens (dense_k, dense_v, e.g. tokens appended
    during decoding and not yet factored) join at full precision.

    Written as the plain definition: every segment is decompressed explicitly, the
    keys and values of all segments and the dense tokens are concatenated, and one
    dense softmax attention runs over them.  Returns dict(out [Hq*d], top: per segment
    [Hq][top_k] ascending ids, p: per segment [Hq][N_seg] attention weights).
    """
    q = np.asarray(q, np.float64)
    d = head_dim
    Hq = q.shape[0] // d
    G = Hq // n_kv_heads
    segs = [{k: (np.asarray(v, np.float64) if k in ("U_k", "B_k", "U_v", "B_v") else v)
             for k, v in s.items()} for s in segments]
    T = 0 if dense_k is None else np.asarray(dense_k).shape[0]
    dk = np.asarray(dense_k, np.float64) if T else None
    dv = np.asarray(dense_v, np.float64) if T else None
    out = np.zeros(Hq * d)
    tops = [[] for _ in segs]
    ps = [[] for _ in segs]
    for h in range(Hq):
        g = h // G
        cols = slice(g * d, (g + 1) * d)
        qh = q[h * d:(h + 1) * d]
        K_parts, V_parts, sizes = [], [], []
        for i, s in enumerate(segs):
            r_lo, k = s["r_lo"], s["top_k"]
            Uk, Bk, Uv, Bv = s["U_k"], s["B_k"], s["U_v"], s["B_v"]
            K_lo = Uk[:, :r_lo] @ Bk[:r_lo, cols]
            top = select_top(scale * (K_lo @ qh), k)
            rank_of = np.full(Uk.shape[0], r_lo)
            rank_of[top] = Uk.shape[1]
            # explicit decompression of every token at its own rank
            K_hat = np.stack([Uk[n, :rank_of[n]] @ Bk[:rank_of[n], cols] for n in range(Uk.shape[0])])
            V_hat = np.stack([Uv[n, :rank_of[n]] @ Bv[:rank_of[n], cols] for n in range(Uv.shape[0])])
            K_parts.append(K_hat)
            V_parts.append(V_hat)
            sizes.append(Uk.shape[0])
            tops[i].append(top)
        if T:
            K_parts.append(dk[:, cols])
            V_parts.append(dv[:, cols])
        K_all = np.concatenate(K_parts)
        V_all = np.concatenate(V_parts)
        s_all = scale * (K_all @ qh)
        p = np.exp(s_all - s_all.max())
        p /= p.sum()
        out[h * d:(h + 1) * d] = p @ V_all
        off = 0
        for i, n in enumerate(sizes):
            ps[i].append(p[off:off + n])
            off += n
    return dict(out=out,
                top=[np.array(t, dtype=np.int64).reshape(Hq, s["top_k"]) for t, s in zip(tops, segs)],
                p=[np.array(x) for x in ps])
