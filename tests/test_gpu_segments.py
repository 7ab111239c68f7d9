"""GPU parity of decode over a factored text segment (needs an MI355X).

The text tokens are factored apart from the visual ones (their own cache, rank and
storage); the decode step attends over the visual segment, the text segment and the
dense tokens appended since, in one softmax.  The oracle (oracle.decode.decode_segments)
decompresses every segment explicitly at each token's rank and runs one dense softmax.
Bars: visual top-k sets exact outside the 1e-3 band; outputs within max-abs 2e-2 when
any segment is stored in bf16 or 4 bits, 1e-4 when all are fp32.  The cache-growth case
re-factors text + appended tokens with ap_compress on the GPU and checks each step
against the oracle run on the GPU's own downloaded factors.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, binding_storage, make_inputs, stored_u, torch_storage, torch_u
from oracle.decode import band_mask, decode_segments
from rank_compressed_kv_ap_amd import workloads as wl

pytestmark = pytest.mark.gpu

VIS = {
    "bf16": wl.LLAVA.replace(cfg_id=401, batch=3, n_q_heads=8, n_kv_heads=8, head_dim=64,
                             n_tokens=200, n_text=5, rank=48, r_lo=20, top_k=50, grid=None,
                             inner_dim=200),
    "int4": wl.LLAVA.replace(cfg_id=402, batch=2, n_q_heads=8, n_kv_heads=8, head_dim=64,
                             n_tokens=200, n_text=5, rank=48, r_lo=16, top_k=50, grid=None,
                             inner_dim=200, storage="int4"),
    "f32_gqa": wl.GQA.replace(cfg_id=403, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=32,
                              n_tokens=70, n_text=3, rank=40, r_lo=20, top_k=17, storage="f32",
                              inner_dim=64),
}


def text_workload(w, n_tok, rank, storage=None):
    """The text segment's factor law: the visual workload's shape with its own token
    count and rank (synthetic, seeded apart by cfg_id)."""
    return w.replace(cfg_id=w.cfg_id + 50, n_tokens=n_tok, rank=rank, n_text=0, grid=None,
                     frames=None, inner_dim=min(n_tok, w.width), storage=storage or w.storage)


def upload_cache(w, seqs, binding):
    B = w.batch
    idx = [b % len(seqs) for b in range(B)]

    def stack(key, dtype):
        return torch.from_numpy(np.stack([seqs[i][key] for i in idx])).to(dtype).cuda().contiguous()

    c = binding.compress(None, None, batch=B, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                         n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank,
                         storage=binding_storage(w))
    c.set_factors(stack("U_k", torch_u(w)), stack("B_k", torch_storage(w)), stack("U_v", torch_u(w)),
                  stack("B_v", torch_storage(w)))
    return c, stack


def seg_of(w, s, r_lo, top_k):
    return dict(U_k=stored_u(w, s["U_k"]), B_k=s["B_k"], U_v=stored_u(w, s["U_v"]), B_v=s["B_v"],
                r_lo=r_lo, top_k=top_k)


def check_set(got, want, s_lo, k, where):
    """Selected ids ascending, and equal to the oracle's outside the 1e-3 band of the
    k-th largest low-rank score."""
    assert np.all(np.diff(got) > 0), (where, "ids not strictly ascending")
    diff = set(got.tolist()) ^ set(want.tolist())
    if diff:
        band = band_mask(s_lo, k)
        assert all(band[n] for n in diff), (where, sorted(diff)[:8])
    return len(diff)


def seg_s_lo(w, f, q, h, r_lo):
    """A segment's low-rank scores for query head h (the ranking the oracle uses)."""
    g = h // (w.n_q_heads // w.n_kv_heads)
    cols = slice(g * w.head_dim, (g + 1) * w.head_dim)
    qh = q[h * w.head_dim:(h + 1) * w.head_dim]
    return w.scale * (f["U_k"][:, :r_lo] @ (f["B_k"][:r_lo, cols] @ qh))


def check(w, tw, vis, txt, out, sel, r_lo_t, k_t, dense=None, tsel=None):
    tol = max(TOL[w.storage], TOL[tw.storage])
    worst = 0.0
    for b in range(len(vis)):
        s, t = vis[b], txt[b]
        dk, dv = (s["text_k"], s["text_v"]) if dense is None else dense[b]
        ref = decode_segments([seg_of(w, s, w.r_lo, w.top_k), seg_of(tw, t, r_lo_t, k_t)], s["q"],
                              w.n_kv_heads, w.head_dim, w.scale, dk if len(dk) else None,
                              dv if len(dv) else None)
        err = float(np.max(np.abs(out[b] - ref["out"])))
        worst = max(worst, err)
        assert err <= tol, (b, err)
        for h in range(w.n_q_heads):
            if sel is not None:
                vs = seg_of(w, s, w.r_lo, w.top_k)
                check_set(sel[b, h], ref["top"][0][h], seg_s_lo(w, vs, s["q"], h, w.r_lo), w.top_k,
                          ("visual", b, h))
            if tsel is not None:
                ts = seg_of(tw, t, r_lo_t, k_t)
                check_set(tsel[b, h], ref["top"][1][h], seg_s_lo(w, ts, s["q"], h, r_lo_t), k_t,
                          ("text", b, h))
    return worst


@pytest.mark.parametrize("vis,text_storage,n_tok,rank,r_lo_t,k_t", [
    ("bf16", "bf16", 70, 16, 8, 20),      # text selected inside its segment, ragged token tail
    ("bf16", "bf16", 64, 16, 16, 0),      # text at full rank (r_lo = rank)
    ("int4", "bf16", 40, 32, 16, 10),     # 4-bit visual factors, bf16 text factors
    ("bf16", "int4", 100, 32, 16, 25),    # 4-bit text factors
    ("f32_gqa", "f32", 33, 12, 4, 33),    # fp32, GQA, every text token at full rank
    ("bf16", "bf16", 1100, 16, 8, 275),   # too large to stage in LDS: the three-kernel path
])
def test_text_segment_parity(gpu_lib, vis, text_storage, n_tok, rank, r_lo_t, k_t):
    w = VIS[vis]
    tw = text_workload(w, n_tok, rank, text_storage)
    vseqs = make_inputs(w)
    tseqs = [wl.gen_decode_inputs(tw, b) for b in range(w.batch)]
    c, stack = upload_cache(w, vseqs, gpu_lib)
    tc, _ = upload_cache(tw, tseqs, gpu_lib)
    q = stack("q", torch.float32)
    dt = torch_storage(w)
    tk, tv = stack("text_k", dt), stack("text_v", dt)
    sel = torch.full((w.batch, w.n_q_heads, w.top_k), -1, dtype=torch.int32, device="cuda")
    tsel = torch.full((w.batch, w.n_q_heads, k_t), -1, dtype=torch.int32, device="cuda")
    out = gpu_lib.decode(c, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk, text_v=tv,
                         sel_out=sel, text_cache=tc, text_r_lo=r_lo_t, text_top_k=k_t,
                         text_sel_out=tsel if k_t else None)
    torch.cuda.synchronize()
    err = check(w, tw, vseqs, tseqs, out.cpu().numpy(), sel.cpu().numpy(), r_lo_t, k_t,
                tsel=tsel.cpu().numpy())
    print(f"{vis} + text {text_storage}: max abs err {err:.3e}")
    c.free()
    tc.free()


def test_text_segment_full_layer(gpu_lib):
    """The batch-32 LLaVA layer with its 64 text tokens factored at rank 16 (the first 8
    components for the unselected half), no dense tokens left."""
    w = wl.LLAVA
    tw = text_workload(w, 64, 16)
    vseqs = make_inputs(w, 2)
    tseqs = [wl.gen_decode_inputs(tw, b) for b in range(2)]
    c, stack = upload_cache(w, vseqs, gpu_lib)
    tc, _ = upload_cache(tw.replace(batch=w.batch), tseqs, gpu_lib)
    q = stack("q", torch.float32)
    tsel = torch.full((w.batch, w.n_q_heads, 32), -1, dtype=torch.int32, device="cuda")
    out = gpu_lib.decode(c, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_cache=tc,
                         text_r_lo=8, text_top_k=32, text_sel_out=tsel)
    torch.cuda.synchronize()
    out, tsel = out.cpu().numpy(), tsel.cpu().numpy()
    empty = np.zeros((0, w.width), np.float32)
    check(w, tw, vseqs, tseqs, out, None, 8, 32, dense=[(empty, empty)] * 2, tsel=tsel)
    for b in range(2, w.batch):
        assert np.array_equal(out[b], out[b % 2]), b
        assert np.array_equal(tsel[b], tsel[b % 2]), b
    c.free()
    tc.free()


def test_cache_growth_with_refactoring(gpu_lib):
    """Decode steps that append 4 dense tokens each; after every second step the text
    tokens and the appended ones are factored again on the GPU (ap_compress) into a new
    text cache and the dense part starts empty.  Every step is checked against the
    oracle on the GPU's own downloaded text factors."""
    w = VIS["bf16"].replace(n_text=0)
    T0, rank_t, r_lo_t = 24, 16, 8
    vseqs = make_inputs(w)
    c, stack = upload_cache(w, vseqs, gpu_lib)
    rms = 1.0
    dense_all = [[wl.gen_text(w.replace(n_text=T0), b, which, rms) for which in (0, 1)]
                 for b in range(w.batch)]           # tokens of the text segment so far
    tail = [[np.zeros((0, w.width), np.float32)] * 2 for _ in range(w.batch)]
    tc = None

    def refactor():
        K = torch.from_numpy(np.stack([d[0] for d in dense_all])).to(torch.bfloat16).cuda()
        V = torch.from_numpy(np.stack([d[1] for d in dense_all])).to(torch.bfloat16).cuda()
        n = K.shape[1]
        return gpu_lib.compress(K.contiguous(), V.contiguous(), batch=w.batch, n_tokens=n,
                                n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
                                head_dim=w.head_dim, rank=min(rank_t, n), storage=torch.bfloat16,
                                seed=7 + n)

    tc = refactor()
    for step in range(6):
        new = [[wl.gen_text(w.replace(n_text=4), b, which, rms, step=step + 1) for which in (0, 1)]
               for b in range(w.batch)]
        for b in range(w.batch):
            for which in (0, 1):
                tail[b][which] = np.concatenate([tail[b][which], new[b][which]])
                dense_all[b][which] = np.concatenate([dense_all[b][which], new[b][which]])
        qn = [wl.gen_q(w, b, step=step + 1) for b in range(w.batch)]
        q = torch.from_numpy(np.stack(qn)).cuda()
        tk = torch.from_numpy(np.stack([t[0] for t in tail])).to(torch.bfloat16).cuda()
        tv = torch.from_numpy(np.stack([t[1] for t in tail])).to(torch.bfloat16).cuda()
        n_t = tc.n_tokens
        tsel = torch.full((w.batch, w.n_q_heads, n_t // 2), -1, dtype=torch.int32, device="cuda")
        out = gpu_lib.decode(c, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk, text_v=tv,
                             text_cache=tc, text_r_lo=r_lo_t, text_top_k=n_t // 2, text_sel_out=tsel)
        U_k, B_k, U_v, B_v = (x.float().cpu().numpy() for x in tc.get_factors())
        torch.cuda.synchronize()
        out, tsel = out.cpu().numpy(), tsel.cpu().numpy()
        for b in range(w.batch):
            s = vseqs[b % len(vseqs)]
            t = dict(U_k=U_k[b], B_k=B_k[b], U_v=U_v[b], B_v=B_v[b], r_lo=r_lo_t, top_k=n_t // 2)
            ref = decode_segments([seg_of(w, s, w.r_lo, w.top_k), t], qn[b], w.n_kv_heads,
                                  w.head_dim, w.scale, tail[b][0], tail[b][1])
            err = float(np.max(np.abs(out[b] - ref["out"])))
            assert err <= 2e-2, (step, b, err)
            for h in range(w.n_q_heads):
                check_set(tsel[b, h], ref["top"][1][h], seg_s_lo(w, t, qn[b], h, r_lo_t), n_t // 2,
                          ("text", step, b, h))
        if step % 2 == 1:     # re-factor text + appended tokens; the dense part restarts
            tc.free()
            tc = refactor()
            tail = [[np.zeros((0, w.width), np.float32)] * 2 for _ in range(w.batch)]
    assert tc.n_tokens == T0 + 6 * 4
    tc.free()
    c.free()


def test_text_segment_argument_errors(gpu_lib):
    from rank_compressed_kv_ap_amd import binding as bnd
    w = VIS["bf16"]
    vseqs = make_inputs(w, 1)
    c, stack = upload_cache(w, vseqs, gpu_lib)
    q = stack("q", torch.float32)
    bad_heads = gpu_lib.compress(None, None, batch=w.batch, n_tokens=16, n_kv_heads=4, n_q_heads=8,
                                 head_dim=w.head_dim, rank=8, storage=torch.bfloat16)
    good = gpu_lib.compress(None, None, batch=w.batch, n_tokens=16, n_kv_heads=w.n_kv_heads,
                            n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=8, storage=torch.bfloat16)
    cases = [dict(text_cache=bad_heads, text_r_lo=4, text_top_k=4),
             dict(text_cache=good, text_r_lo=0, text_top_k=4),
             dict(text_cache=good, text_r_lo=9, text_top_k=4),
             dict(text_cache=good, text_r_lo=4, text_top_k=17),
             dict(text_cache=c, text_r_lo=4, text_top_k=4)]
    for kw in cases:
        with pytest.raises(bnd.APError):
            gpu_lib.decode(c, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, **kw)
    for x in (bad_heads, good, c):
        x.free()
