"""GPU parity of the moving-average importance selector (needs an MI355X).

Each step is checked on its own against the CPU oracle:
  * the first step ranks by the low-rank logits: its sets are compared with the
    oracle's inside the usual 1e-3 band;
  * a later step ranks by the importance state the GPU left: the GPU's sets must be
    exactly the top-k of that (downloaded) state, ties to the lower index - the same
    integer decision from the same keys;
  * the oracle, run with the GPU's sets, gives the output (max-abs 2e-2 bf16, 1e-4
    fp32) and the attention weights p; the GPU's new state must equal
    alpha * (state before) + (1 - alpha) * p (or p on the first step), per head or
    averaged over heads, within a bound derived from the arithmetic: with bf16 factors
    the decode kernels round the latent query q~ to bf16 in its columns at or above
    r_lo (relative 2^-9 per element, products and sums in fp32; the columns below r_lo
    carry a hi + lo split), so a logit moves by at most
    2^-8 * scale * sum_i |U_k[n,i] q~_i| (taken over every column, an upper bound) and
    a weight p = exp(s - M) / L by at most twice the largest such move, relatively;
    fp32 factors: 1e-4.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, make_inputs, stored_u, upload_decode
from oracle.decode import band_mask, decode_ref, select_top
from rank_compressed_kv_ap_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = {
    "bf16_text": wl.LLAVA.replace(cfg_id=121, batch=3, n_q_heads=8, n_kv_heads=8, head_dim=64,
                                  n_tokens=200, n_text=70, rank=48, r_lo=20, top_k=50, grid=None,
                                  inner_dim=200),
    "f32_gqa": wl.GQA.replace(cfg_id=122, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=32,
                              n_tokens=70, rank=40, r_lo=20, top_k=17, storage="f32", inner_dim=64),
    "llava7b_layer": wl.LLAVA,
    # rank 64 with r_lo = 16: the single-kernel decode (two and three steps per wavefront)
    "bf16_single": wl.LLAVA.replace(cfg_id=124, batch=3, n_q_heads=6, n_kv_heads=2, head_dim=64,
                                    n_tokens=300, n_text=20, rank=64, r_lo=16, top_k=75, grid=None,
                                    inner_dim=300),
    "bf16_single_3": wl.LLAVA.replace(cfg_id=125, batch=2, n_q_heads=4, n_kv_heads=4, head_dim=32,
                                      n_tokens=2100, n_text=0, rank=64, r_lo=16, top_k=500,
                                      grid=None, inner_dim=256),
    # grouped-query heads with no text on the split path: the combine that reads each
    # B_v row chunk once for the four query heads of a KV head writes the softmax
    # statistics the state update reads
    "bf16_gqa_split": wl.LLAVA.replace(cfg_id=126, batch=3, n_q_heads=8, n_kv_heads=2, head_dim=64,
                                       n_tokens=300, n_text=0, rank=48, r_lo=16, top_k=75, grid=None,
                                       inner_dim=128),
    # more selection workgroups than CUs: the 8-wavefront selector
    "bf16_many_wgs": wl.LLAVA.replace(cfg_id=123, batch=70, n_q_heads=16, n_kv_heads=16,
                                      head_dim=64, n_tokens=300, n_text=5, rank=32, r_lo=16,
                                      top_k=75, grid=None, inner_dim=300),
}
def _weight_rtol(w, s, q):
    """Per-head relative error bound of the GPU's attention weights (see above)."""
    if w.storage == "f32":
        return np.full(w.n_q_heads, 1e-4)
    d, G = w.head_dim, w.n_q_heads // w.n_kv_heads
    Uk = np.asarray(stored_u(w, s["U_k"]), np.float64)
    Bk = np.asarray(s["B_k"], np.float64)
    out = np.zeros(w.n_q_heads)
    for h in range(w.n_q_heads):
        g = h // G
        qt = Bk[:, g * d:(g + 1) * d] @ np.asarray(q[h * d:(h + 1) * d], np.float64)
        ds = 2.0 ** -8 * w.scale * np.max(np.abs(Uk * qt[None, :]).sum(axis=1))
        out[h] = 2.0 * np.expm1(ds) + 1e-5
    return out


def _queries(w, seqs, steps, seed):
    """Step 0 uses the workload's q; later steps draw fresh N(0,1) queries."""
    g = np.random.default_rng(seed)
    qs = [[s["q"] for s in seqs]]
    for _ in range(steps - 1):
        qs.append([g.standard_normal(w.n_q_heads * w.head_dim).astype(np.float32) for _ in seqs])
    return qs


def _oracle_with_sets(w, s, q, sets):
    """Oracle decode whose selected sets are forced to `sets` ([Hq][k] ids)."""
    keys = np.zeros((w.n_q_heads, w.n_tokens))
    for h in range(w.n_q_heads):
        keys[h, sets[h]] = 1.0
    return decode_ref(stored_u(w, s["U_k"]), s["B_k"], stored_u(w, s["U_v"]), s["B_v"], q,
                      w.n_kv_heads, w.head_dim,
                      w.r_lo, w.top_k, w.scale, s["text_k"] if w.n_text else None,
                      s["text_v"] if w.n_text else None, select_keys=keys)


def _run(gpu_lib, w, mode, alpha, steps, n_distinct=None, seed=5, splits=0, path=None):
    seqs = make_inputs(w, n_distinct)
    cache, q0, tk, tv = upload_decode(w, seqs, gpu_lib)
    B, Hq, N, k = w.batch, w.n_q_heads, w.n_tokens, w.top_k
    per_head = mode == "ema_head"
    imp = torch.zeros((B, Hq, N) if per_head else (B, N), dtype=torch.float32, device="cuda")
    scratch = torch.empty(B, Hq, N, dtype=torch.float32, device="cuda")
    qs = _queries(w, seqs, steps, seed)
    tol = TOL[w.storage]
    for t in range(steps):
        q = torch.from_numpy(np.stack([qs[t][b % len(seqs)] for b in range(B)])).cuda()
        before = imp.cpu().numpy().astype(np.float64)
        sel = torch.full((B, Hq, k), -1, dtype=torch.int32, device="cuda")
        if path is not None:
            cache.timing_enable(1)
        out = gpu_lib.decode(cache, q, r_lo=w.r_lo, top_k=k, scale=w.scale, text_k=tk, text_v=tv,
                             sel_out=sel, select=mode, ema_alpha=alpha, ema_first=(t == 0),
                             importance=imp, ema_scratch=scratch, splits=splits)
        if path is not None:
            ms, n = cache.timing_read()
            cache.timing_enable(0)
            assert n == 1
            if path == "decode":   # the single kernel, plus the fold of the per-token state
                assert ms["decode"] > 0 and ms["select"] == ms["attn"] == ms["combine"] == 0, ms
                assert (ms["ema"] > 0) == (mode == "ema_token"), ms
            else:
                assert ms["decode"] == 0 and min(ms["select"], ms["attn"], ms["ema"]) > 0, ms
        torch.cuda.synchronize()
        out, sel, after = out.cpu().numpy(), sel.cpu().numpy(), imp.cpu().numpy().astype(np.float64)
        for b in range(len(seqs)):
            s = seqs[b]
            if t == 0:
                plain = decode_ref(stored_u(w, s["U_k"]), s["B_k"], stored_u(w, s["U_v"]), s["B_v"],
                                   qs[t][b], w.n_kv_heads,
                                   w.head_dim, w.r_lo, k, w.scale, s["text_k"] if w.n_text else None,
                                   s["text_v"] if w.n_text else None)
                for h in range(Hq):
                    diff = set(sel[b, h].tolist()) ^ set(plain["top"][h].tolist())
                    band = band_mask(plain["s_lo"][h], k)
                    assert all(band[n] for n in diff), (t, b, h, sorted(diff)[:8])
            else:
                for h in range(Hq):
                    keys = before[b, h] if per_head else before[b]
                    assert sel[b, h].tolist() == select_top(keys, k).tolist(), (t, b, h)
            ref = _oracle_with_sets(w, s, qs[t][b], sel[b])
            err = float(np.max(np.abs(out[b] - ref["out"])))
            assert err <= tol, (t, b, err)
            p = ref["p"] if per_head else ref["p"].mean(axis=0)
            rt = _weight_rtol(w, s, qs[t][b])
            perr = ref["p"] * rt[:, None]                     # bound of each weight's error
            perr = perr if per_head else perr.mean(axis=0)
            want = p if t == 0 else alpha * before[b] + (1.0 - alpha) * p
            lim = (1.0 if t == 0 else 1.0 - alpha) * perr + 1e-6 * np.abs(want) + 1e-9
            got = after[b]
            bad = np.abs(got - want) > lim
            assert not bad.any(), (t, b, float(np.max(np.abs(got - want) / lim)))
        for b in range(len(seqs), B):   # replicas of a distinct sequence stay bit-identical
            o = b % len(seqs)
            assert np.array_equal(after[b], after[o]) and np.array_equal(sel[b], sel[o])
    cache.free()


@pytest.mark.parametrize("mode", ["ema_token", "ema_head"])
@pytest.mark.parametrize("name,alpha", [("bf16_text", 0.8), ("f32_gqa", 0.5), ("bf16_gqa_split", 0.6)])
def test_ema_selector_steps(gpu_lib, name, mode, alpha):
    _run(gpu_lib, SHAPES[name], mode, alpha, steps=4)


@pytest.mark.parametrize("mode", ["ema_token", "ema_head"])
@pytest.mark.parametrize("name,splits,path", [("bf16_single", 0, "decode"), ("bf16_single_3", 0, "decode"),
                                              ("bf16_single", 2, "split")])
def test_ema_selector_single_kernel(gpu_lib, name, splits, path, mode):
    """Shapes the single-kernel decode takes: the state is ranked, blended (per head) or
    folded from per-head-group sums (per token) there; an explicit split count runs the
    split-N path on the same shape."""
    _run(gpu_lib, SHAPES[name], mode, 0.8, steps=3, splits=splits, path=path)


@pytest.mark.parametrize("mode", ["ema_token", "ema_head"])
def test_ema_selector_many_workgroups(gpu_lib, mode):
    _run(gpu_lib, SHAPES["bf16_many_wgs"], mode, 0.7, steps=3, n_distinct=2)


def test_ema_alpha_zero_follows_last_weights(gpu_lib):
    _run(gpu_lib, SHAPES["bf16_text"], "ema_head", 0.0, steps=3)


@pytest.mark.parametrize("mode", ["ema_token", "ema_head"])
def test_ema_selector_full_layer(gpu_lib, mode):
    """The batch-32 LLaVA layer, three steps, three distinct sequences checked."""
    _run(gpu_lib, SHAPES["llava7b_layer"], mode, 0.9, steps=3, n_distinct=3)


def test_ema_argument_errors(gpu_lib):
    from rank_compressed_kv_ap_amd import binding as b
    w = SHAPES["bf16_text"]
    seqs = make_inputs(w, 1)
    cache, q, tk, tv = upload_decode(w.replace(batch=1), seqs, gpu_lib)
    with pytest.raises(b.APError):
        gpu_lib.decode(cache, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, select="ema_head",
                       ema_alpha=0.5)   # no state buffers
    imp = torch.zeros(1, w.n_q_heads, w.n_tokens, device="cuda")
    scratch = torch.empty_like(imp)
    for alpha in (1.0, -0.1, float("nan")):
        with pytest.raises(b.APError):
            gpu_lib.decode(cache, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, select="ema_head",
                           ema_alpha=alpha, importance=imp, ema_scratch=scratch)
    cache.free()
