"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case rewrites one line of an oracle module's source text (a dropped
term, a wrong sign, a wrong index, a transposed operand), loads the mutant
next to the real module, and checks that an independent pin rejects it.
Nothing here touches the GPU.
"""
import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle.decode as dec
import oracle.jacobi as jac
import oracle.factorize as rs
from oracle.brute import decode_brute


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert src.count(old) >= 1, old
    m = types.ModuleType(module.__name__ + "_mutant")
    m.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new, 1), module.__name__ + "_mutant", "exec"), m.__dict__)
    return m


def _brute_pin_ok(decode_fn):
    g = np.random.default_rng(7)
    N, r, r_lo, k, Hkv, Hq, d, T = 7, 4, 2, 3, 2, 4, 3, 2
    W = Hkv * d
    Uk, Bk, Uv, Bv = (g.standard_normal(s) for s in [(N, r), (r, W), (N, r), (r, W)])
    Kt, Vt = g.standard_normal((T, W)), g.standard_normal((T, W))
    q = g.standard_normal(Hq * d)
    try:
        res = decode_fn(Uk, Bk, Uv, Bv, q, Hkv, d, r_lo, k, 0.7, Kt, Vt)
    except Exception:
        return False
    out, tops = decode_brute(Uk.tolist(), Bk.tolist(), Uv.tolist(), Bv.tolist(), q.tolist(),
                             Hkv, d, r_lo, k, 0.7, Kt.tolist(), Vt.tolist())
    ok = (np.max(np.abs(res["out"] - np.array(out))) <= 1e-12
          and [list(t) for t in res["top"]] == tops)
    # a case made of ties: duplicated key rows cut through by the top-k boundary
    Uk2 = Uk.copy()
    Uk2[[2, 4, 6]] = Uk2[0]
    q2 = np.zeros_like(q)                   # every score ties: top-k = lowest indices
    res2 = decode_fn(Uk2, Bk, Uv, Bv, q2, Hkv, d, r, 2, 0.7, Kt, Vt)
    out2, tops2 = decode_brute(Uk2.tolist(), Bk.tolist(), Uv.tolist(), Bv.tolist(), q2.tolist(),
                               Hkv, d, r, 2, 0.7, Kt.tolist(), Vt.tolist())
    return bool(ok and np.max(np.abs(res2["out"] - np.array(out2))) <= 1e-12
                and [list(t) for t in res2["top"]] == tops2)


def test_real_decode_passes_brute_pin():
    assert _brute_pin_ok(dec.decode_ref)


@pytest.mark.parametrize("old,new", [
    ("g = h // G", "g = h % n_kv_heads"),                              # wrong KV head
    ("order = np.lexsort((n, -s_lo))", "order = np.lexsort((n, s_lo))"),  # smallest instead of largest
    ("order = np.lexsort((n, -s_lo))", "order = np.lexsort((-n, -s_lo))"),  # ties to higher index
    ("o = o + p[N:] @ text_v[:, cols]", "o = o"),                    # text values dropped
    ("V_sel[top] = V_full[top]", "pass"),                             # V never upgraded
    ("s[top] = scale * (K_full[top] @ qh)", "s[top] = K_full[top] @ qh"),  # scale dropped
    ("K_lo = U_k[:, :r_lo] @ B_k[:r_lo, cols]", "K_lo = U_k[:, :r_lo] @ B_k[:r_lo, cols] * 1.0001"),
])
def test_decode_mutants_are_caught(old, new):
    m = _mutant(dec, old, new)
    assert not _brute_pin_ok(m.decode_ref)


@pytest.mark.parametrize("old,new", [
    ("new_i = c * xi - s * xj", "new_i = c * xi + s * xj"),
    ("zeta = (beta - alpha) / (2.0 * gamma)", "zeta = (alpha - beta) / (2.0 * gamma)"),
    ("V[:, i] = c * vi - s * vj", "V[:, i] = c * vi + s * vj"),
])
def test_jacobi_mutants_are_caught(old, new):
    m = _mutant(jac, old, new)
    A = np.random.default_rng(3).standard_normal((12, 9))
    try:
        U, s, V = m.jacobi_svd(A, max_sweeps=30)
    except RuntimeError:
        return       # failing to converge is also a rejection
    ok = (np.allclose(s, np.linalg.svd(A, compute_uv=False), rtol=1e-12)
          and np.linalg.norm(A - (U * s) @ V.T) <= 1e-12 * np.linalg.norm(A))
    assert not ok


@pytest.mark.parametrize("old,new", [
    ("U = (Q @ Uc[:, :r]) * s[None, :r]", "U = Q @ Uc[:, :r]"),     # singular values dropped
    ("Qt = orth_mgs2(A.T @ Q)", "Qt = orth_mgs2(A @ Q[:A.shape[1]])"),  # wrong operand
    ("C = Q.T @ A", "C = Q.T @ A[::-1]"),                              # rows scrambled
])
def test_rsvd_mutants_are_caught(old, new):
    m = _mutant(rs, old, new)
    g = np.random.default_rng(4)
    N, W, k = 30, 20, 4
    A = g.standard_normal((N, k)) @ g.standard_normal((k, W))
    try:
        U, B, _ = m.rsvd(A, 4, g.standard_normal((W, 8)))
        ok = np.linalg.norm(A - U @ B) <= 1e-11 * np.linalg.norm(A)
    except (ValueError, RuntimeError, np.linalg.LinAlgError):
        ok = False
    assert not ok


@pytest.mark.parametrize("old,new", [
    ("I = p.copy() if I is None else alpha * I + (1.0 - alpha) * p",
     "I = p.copy() if I is None else (1.0 - alpha) * I + alpha * p"),        # swapped weights
    ("p = res[\"p\"] if per_head else res[\"p\"].mean(axis=0)",
     "p = res[\"p\"] if per_head else res[\"p\"].sum(axis=0)"),              # sum, not mean
    ("            keys = I if per_head else np.broadcast_to(I, (Hq, I.shape[-1]))",
     "            keys = None"),                                               # history ignored
])
def test_mutated_ema_selector_is_caught(old, new):
    from oracle.brute import decode_ema_brute
    m = _mutant(dec, old, new)
    g = np.random.default_rng(70)
    N, r, Hkv, Hq, d, T = 9, 4, 2, 4, 3, 2
    W = Hkv * d
    Uk, Bk, Uv, Bv = (g.standard_normal(s) for s in [(N, r), (r, W), (N, r), (r, W)])
    Kt, Vt = g.standard_normal((T, W)), g.standard_normal((T, W))
    qs = [g.standard_normal(Hq * d) for _ in range(4)]
    res, states = m.decode_ema_steps(Uk, Bk, Uv, Bv, qs, Hkv, d, 2, 3, 0.8, 0.7, False, Kt, Vt)
    outs, tops, bstates = decode_ema_brute(Uk.tolist(), Bk.tolist(), Uv.tolist(), Bv.tolist(),
                                           [q.tolist() for q in qs], Hkv, d, 2, 3, 0.8, 0.7,
                                           False, Kt.tolist(), Vt.tolist())
    agree = all(np.max(np.abs(states[t] - np.array(bstates[t]))) <= 1e-12 and
                [list(x) for x in res[t]["top"]] == tops[t] for t in range(len(qs)))
    assert not agree, "the planted mistake went unnoticed"


# ---------------------------------------------------------------- 4-bit factors
import oracle.quant as qnt


def _quant_pins_ok(mod):
    from test_oracle_pins import _quant_brute, _quant_case
    try:
        for seed in (70, 71):
            U = _quant_case(seed)
            codes, scales = mod.quantize_u4(U)
            bc, bs = _quant_brute(U.astype(np.float64).tolist())
            if codes.tolist() != bc or scales.astype(np.float64).tolist() != bs:
                return False
            dq = mod.dequant_u4(codes, scales)
            s = np.repeat(np.asarray(bs), 32, axis=0)[:U.shape[0]]
            if not np.all(np.abs(U.astype(np.float64) - dq) <= s / 2):
                return False
    except Exception:
        return False
    return True


def test_real_quantizer_passes_pins():
    assert _quant_pins_ok(qnt)


@pytest.mark.parametrize("old,new", [
    ("np.rint(t)", "np.sign(t) * np.floor(np.abs(t) + 0.5)"),           # ties away from zero
    ("m = np.max(np.abs(rows), axis=0)", "m = np.max(np.abs(U32), axis=0)"),  # one scale per column
    ("inv7 = np.float32(1.0) / np.float32(QMAX)", "inv7 = np.float32(1.0) / np.float32(QMAX + 1)"),
    ("s = _bf16_rne(m * inv7)", "s = m * inv7"),                         # scale not rounded to bf16
    ("np.repeat(np.asarray(scales, np.float64), BLOCK, axis=0)[:N]",
     "np.repeat(np.asarray(scales, np.float64), BLOCK, axis=0)[1:N + 1]"),  # dequant off by a token
])
def test_quantizer_mutants_are_caught(old, new):
    assert not _quant_pins_ok(_mutant(qnt, old, new))


# ---------------------------------------------------------------- segments
def _segments_pin_ok(mod):
    from oracle.brute import decode_segments_brute
    from test_oracle_pins import _seg_case
    try:
        for seed, T in ((80, 2), (82, 5)):
            segs, Kd, Vd, q = _seg_case(seed, T=T)
            res = mod.decode_segments(segs, q, 2, 3, 0.6, Kd, Vd)
            lsegs = [{k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in s.items()} for s in segs]
            out, tops = decode_segments_brute(lsegs, q.tolist(), 2, 3, 0.6, Kd.tolist(), Vd.tolist())
            if np.max(np.abs(res["out"] - np.array(out))) > 1e-12:
                return False
            if any([list(t) for t in res["top"][i]] != tops[i] for i in range(len(segs))):
                return False
    except Exception:
        return False
    return True


def test_real_segments_pass_brute_pin():
    assert _segments_pin_ok(dec)


@pytest.mark.parametrize("old,new", [
    ('r_lo, k = s["r_lo"], s["top_k"]', 'r_lo, k = segs[0]["r_lo"], s["top_k"]'),      # one r_lo for all
    ("            K_parts.append(dk[:, cols])\n            V_parts.append(dv[:, cols])",
     "            K_parts.append(dk[:, cols])\n            V_parts.append(0 * dv[:, cols])"),  # dense values dropped
    ("top = select_top(scale * (K_lo @ qh), k)",
     "top = select_top(scale * ((Uk @ Bk[:, cols]) @ qh), k)"),                          # ranked at full rank
    ("rank_of[top] = Uk.shape[1]", "rank_of[top] = Uk.shape[1] - 1"),                  # one rank short
])
def test_segments_mutants_are_caught(old, new):
    assert not _segments_pin_ok(_mutant(dec, old, new))


# ---------------------------------------------------------------- acceptance band
def _band_pins_ok(mod):
    from test_oracle_pins import BAND_CASES
    try:
        return all(np.flatnonzero(mod.band_mask(np.array(s), k)).tolist() == want
                   for s, k, want in BAND_CASES)
    except Exception:
        return False


def test_real_band_passes_pins():
    assert _band_pins_ok(dec)


@pytest.mark.parametrize("old,new", [
    ("tau = np.sort(s_lo_h)[::-1][k - 1]", "tau = np.sort(s_lo_h)[::-1][k]"),        # one token off
    ("tau = np.sort(s_lo_h)[::-1][k - 1]", "tau = np.sort(s_lo_h)[k - 1]"),          # k-th smallest
    ("rel * max(abs(tau), rel * float(np.max(np.abs(s_lo_h))))",
     "rel * max(abs(tau), float(np.max(np.abs(s_lo_h))))"),                           # floor too wide
    ("rel * max(abs(tau), rel * float(np.max(np.abs(s_lo_h))))", "rel * abs(tau)"),  # no floor
    ("rel * max(abs(tau), rel * float(np.max(np.abs(s_lo_h))))",
     "rel * max(tau, rel * float(np.max(np.abs(s_lo_h))))"),                          # signed cutoff
    ("if k == 0 or k >= s_lo_h.shape[0]:", "if k == 0 or k > s_lo_h.shape[0]:"),     # k = N not empty
])
def test_band_mutants_are_caught(old, new):
    assert not _band_pins_ok(_mutant(dec, old, new))
