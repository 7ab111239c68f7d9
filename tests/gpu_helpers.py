"""Shared pieces of the GPU parity tests: build a device cache from seeded
workload inputs and check the library's outputs against the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

from oracle.decode import band_mask, decode_ref
from oracle.quant import quantize_dequant_u4
from rank_compressed_kv_ap_amd import workloads as wl

# 4-bit caches attend over bf16-class operands (codes expanded to bf16, bf16 queries
# and weights in the MFMAs): the bf16 bar
TOL = {"bf16": 2e-2, "f32": 1e-4, "int4": 2e-2}


def torch_storage(w):
    """dtype of K, V, text and B on the device."""
    return torch.float32 if w.storage == "f32" else torch.bfloat16


def torch_u(w):
    """dtype of U handed to set_factors (float32 values for a 4-bit cache)."""
    return torch.float32 if w.storage in ("f32", "int4") else torch.bfloat16


def binding_storage(w):
    return "int4" if w.storage == "int4" else torch_storage(w)


def stored_u(w, U):
    """The U values the cache holds: the oracle's 4-bit round trip for a 4-bit cache."""
    return quantize_dequant_u4(U) if w.storage == "int4" else U


def make_inputs(w, n_distinct=None):
    """Host inputs for min(B, n_distinct) distinct sequences (float32, storage-exact)."""
    S = w.batch if n_distinct is None else min(w.batch, n_distinct)
    return [wl.gen_decode_inputs(w, b) for b in range(S)]


def upload_decode(w, seqs, binding):
    """Device cache + tensors for the whole batch; sequence b uses seqs[b % len(seqs)]."""
    dt = torch_storage(w)
    B = w.batch
    idx = [b % len(seqs) for b in range(B)]

    def stack(key, dtype):
        return torch.from_numpy(np.stack([seqs[i][key] for i in idx])).to(dtype).cuda().contiguous()

    U_k, U_v = (stack(k, torch_u(w)) for k in ("U_k", "U_v"))
    B_k, B_v = (stack(k, dt) for k in ("B_k", "B_v"))
    q = stack("q", torch.float32)
    cache = binding.compress(None, None, batch=B, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                             n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank,
                             storage=binding_storage(w))
    cache.set_factors(U_k, B_k, U_v, B_v)
    text_k = text_v = None
    if w.n_text:
        text_k, text_v = stack("text_k", dt), stack("text_v", dt)
    return cache, q, text_k, text_v


def run_decode(w, seqs, binding, splits=0, with_sel=True):
    cache, q, tk, tv = upload_decode(w, seqs, binding)
    sel = None
    if with_sel:
        sel = torch.full((w.batch, w.n_q_heads, w.top_k), -1, dtype=torch.int32, device="cuda")
    out = binding.decode(cache, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk,
                         text_v=tv, sel_out=sel, splits=splits)
    torch.cuda.synchronize()
    res = out.cpu().numpy(), (sel.cpu().numpy() if sel is not None else None)
    cache.free()
    return res


def oracle_decode(w, s):
    return decode_ref(stored_u(w, s["U_k"]), s["B_k"], stored_u(w, s["U_v"]), s["B_v"], s["q"],
                      w.n_kv_heads, w.head_dim,
                      w.r_lo, w.top_k, w.scale,
                      s["text_k"] if w.n_text else None, s["text_v"] if w.n_text else None)


def check_against_oracle(w, seqs, out, sel, b_list=None):
    """Assert top-k sets (outside the 1e-3 band) and outputs match the oracle.

    Returns (max abs error, number of band tokens that differ) for reporting.
    """
    tol = TOL[w.storage]
    worst, flips = 0.0, 0
    for b in (range(len(seqs)) if b_list is None else b_list):
        ref = oracle_decode(w, seqs[b])
        err = float(np.max(np.abs(out[b].astype(np.float64) - ref["out"])))
        worst = max(worst, err)
        assert err <= tol, f"sequence {b}: max abs error {err:.3e} > {tol}"
        if sel is not None:
            for h in range(w.n_q_heads):
                g = sel[b, h]
                assert np.all(np.diff(g) > 0), f"seq {b} head {h}: ids not strictly ascending"
                assert g.min(initial=0) >= 0 and g.max(initial=0) < w.n_tokens
                diff = set(g.tolist()) ^ set(ref["top"][h].tolist())
                if diff:
                    band = band_mask(ref["s_lo"][h], w.top_k)
                    outside = [n for n in diff if not band[n]]
                    assert not outside, f"seq {b} head {h}: tokens {outside[:8]} differ outside the band"
                    flips += len(diff)
    return worst, flips
