"""GPU parity of ap_decode_attn against the CPU oracle (needs an MI355X).

Inputs: seeded factored caches from rank_compressed_kv_ap_amd.workloads, the
same storage-exact values on both sides.  Bar: top-k id sets equal except for
tokens whose low-rank score is within 1e-3 (relative) of the cutoff; outputs
within max-abs 2e-2 (bf16 storage) or 1e-4 (fp32 storage).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import check_against_oracle, make_inputs, run_decode, upload_decode
from rank_compressed_kv_ap_amd import workloads as wl

pytestmark = pytest.mark.gpu

# Small shapes that still span several tiles, with ragged token / rank / head tails.
SMALL = {
    "tiny_cfg": wl.TINY,
    "bf16_ragged": wl.LLAVA.replace(cfg_id=101, batch=3, n_q_heads=4, n_kv_heads=4, head_dim=64,
                                    n_tokens=100, n_text=5, rank=24, r_lo=8, top_k=25, grid=None,
                                    inner_dim=100),
    "f32_gqa_straddle": wl.GQA.replace(cfg_id=102, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=32,
                                       n_tokens=70, rank=40, r_lo=20, top_k=17, storage="f32",
                                       inner_dim=64),
    "bf16_48_heads": wl.LLAVA.replace(cfg_id=103, batch=2, n_q_heads=48, n_kv_heads=16, head_dim=16,
                                      n_tokens=64, n_text=3, rank=32, r_lo=16, top_k=16, grid=None,
                                      inner_dim=64),
    "bf16_rank128": wl.VIDEO.replace(cfg_id=104, batch=2, n_tokens=300, top_k=75, frames=None,
                                     inner_dim=300),
    "bf16_straddle_text": wl.LLAVA.replace(cfg_id=105, batch=2, n_q_heads=8, n_kv_heads=8,
                                           head_dim=64, n_tokens=200, n_text=70, rank=48, r_lo=20,
                                           top_k=50, grid=None, inner_dim=200),
    "f32_text_long": wl.TINY.replace(cfg_id=106, batch=2, n_text=300, n_tokens=90, top_k=22),
    # rank 64 with r_lo 16: the single-kernel decode with its panel split fixed at compile time
    "bf16_rank64_lo16": wl.LLAVA.replace(cfg_id=108, batch=2, n_q_heads=8, n_kv_heads=8, head_dim=64,
                                         n_tokens=300, n_text=10, rank=64, r_lo=16, top_k=75,
                                         grid=None, inner_dim=300),
    # query heads not a multiple of 4: the last head group of the single-kernel decode and
    # of the selector holds fewer heads (2 and 1)
    "bf16_6_heads_gqa": wl.LLAVA.replace(cfg_id=109, batch=3, n_q_heads=6, n_kv_heads=3, head_dim=64,
                                         n_tokens=150, n_text=7, rank=32, r_lo=16, top_k=40,
                                         grid=None, inner_dim=150),
    "bf16_5_heads": wl.LLAVA.replace(cfg_id=110, batch=2, n_q_heads=5, n_kv_heads=5, head_dim=32,
                                     n_tokens=97, n_text=0, rank=48, r_lo=16, top_k=30, grid=None,
                                     inner_dim=97),
    # one latent panel (r = 16): a single 16-row latent-query tile per head
    "bf16_rank16": wl.LLAVA.replace(cfg_id=111, batch=3, n_q_heads=8, n_kv_heads=4, head_dim=128,
                                    n_tokens=130, n_text=20, rank=16, r_lo=4, top_k=33, grid=None,
                                    inner_dim=130),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_parity_small(gpu_lib, name):
    w = SMALL[name]
    seqs = make_inputs(w)
    out, sel = run_decode(w, seqs, gpu_lib)
    err, flips = check_against_oracle(w, seqs, out, sel)
    print(f"{name}: max abs err {err:.3e}, band flips {flips}")


@pytest.mark.parametrize("name", ["bf16_6_heads_gqa", "bf16_5_heads", "bf16_rank16"])
def test_decode_partial_head_group_split_path(gpu_lib, name):
    """The same shapes through selection + split-N flash-decode + combine."""
    w = SMALL[name]
    seqs = make_inputs(w)
    out, sel = run_decode(w, seqs, gpu_lib, splits=2)
    check_against_oracle(w, seqs, out, sel)


@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_decode_split_count_does_not_change_result(gpu_lib, splits):
    w = SMALL["bf16_straddle_text"]
    seqs = make_inputs(w)
    out, sel = run_decode(w, seqs, gpu_lib, splits=splits)
    check_against_oracle(w, seqs, out, sel)


@pytest.mark.parametrize("top_k,r_lo", [(0, 8), (100, 8), (25, 24), (1, 1)])
def test_decode_edge_selection(gpu_lib, top_k, r_lo):
    w = SMALL["bf16_ragged"].replace(top_k=top_k, r_lo=r_lo)
    seqs = make_inputs(w)
    out, sel = run_decode(w, seqs, gpu_lib)
    check_against_oracle(w, seqs, out, sel)
    if top_k == w.n_tokens:
        assert np.array_equal(sel[0, 0], np.arange(w.n_tokens))


def test_decode_single_token(gpu_lib):
    for k in (0, 1):
        w = wl.TINY.replace(cfg_id=110, batch=2, n_tokens=1, rank=1, r_lo=1, top_k=k, inner_dim=1)
        seqs = make_inputs(w)
        out, sel = run_decode(w, seqs, gpu_lib)
        check_against_oracle(w, seqs, out, sel)


@pytest.mark.parametrize("name", ["bf16_ragged", "bf16_rank128", "f32_text_long"])
def test_decode_zero_query_ties_take_lowest_ids(gpu_lib, name):
    # every score ties: N <= 128 exercises exact ranking inside the boundary bin,
    # N = 300 the radix fallback over exact keys
    w = SMALL[name]
    seqs = make_inputs(w)
    for s in seqs:
        s["q"] = np.zeros_like(s["q"])
    out, sel = run_decode(w, seqs, gpu_lib)
    check_against_oracle(w, seqs, out, sel)
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            assert sel[b, h].tolist() == list(range(w.top_k))


@pytest.mark.parametrize("scale_row", [1e3, 1e6])
def test_decode_outlier_token(gpu_lib, scale_row):
    # one huge key row makes the score bound loose, so many tokens share a bin
    w = SMALL["bf16_rank128"]
    seqs = make_inputs(w)
    for s in seqs:
        s["U_k"][7] = wl.round_bf16(s["U_k"][7] * scale_row)
    out, sel = run_decode(w, seqs, gpu_lib)
    check_against_oracle(w, seqs, out, sel)


def test_decode_duplicated_tokens_tie_to_lower_ids(gpu_lib):
    # 40 identical key rows around the cutoff: the tied group is cut by index
    w = SMALL["bf16_straddle_text"]
    seqs = make_inputs(w)
    for s in seqs:
        s["U_k"][60:100] = s["U_k"][60]
    out, sel = run_decode(w, seqs, gpu_lib)
    check_against_oracle(w, seqs, out, sel)
    from gpu_helpers import oracle_decode
    for b, s in enumerate(seqs):
        ref = oracle_decode(w, s)
        for h in range(w.n_q_heads):
            got = set(sel[b, h].tolist())
            tied = set(range(60, 100))
            # inside the tied group the chosen ids are the lowest ones
            chosen = sorted(got & tied)
            if chosen and len(chosen) < len(tied):
                assert chosen == list(range(60, 60 + len(chosen))), (b, h, chosen[:5])


@pytest.mark.parametrize("name,splits", [("bf16_rank128", 0), ("bf16_straddle_text", 0),
                                         ("bf16_straddle_text", 3)])
def test_decode_is_deterministic(gpu_lib, name, splits):
    w = SMALL[name]
    seqs = make_inputs(w)
    cache, q, tk, tv = upload_decode(w, seqs, gpu_lib)
    outs = [gpu_lib.decode(cache, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk,
                           text_v=tv, splits=splits).cpu() for _ in range(3)]
    cache.free()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("name,splits,path", [("bf16_straddle_text", 0, "decode"),
                                              ("bf16_rank64_lo16", 0, "decode"),
                                              ("bf16_6_heads_gqa", 0, "decode"),
                                              ("bf16_5_heads", 0, "decode"),
                                              ("bf16_rank16", 0, "decode"),
                                              ("bf16_straddle_text", 2, "split"),
                                              ("bf16_rank128", 0, "split"),
                                              ("f32_text_long", 0, "split")])
def test_decode_path_taken(gpu_lib, name, splits, path):
    """splits == 0 on a covered shape runs the single-kernel decode; an explicit split
    count, rank 128 or fp32 factors run selection + split-N flash-decode + combine."""
    w = SMALL[name]
    seqs = make_inputs(w)
    cache, q, tk, tv = upload_decode(w, seqs, gpu_lib)
    cache.timing_enable(1)
    gpu_lib.decode(cache, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk, text_v=tv,
                   splits=splits)
    ms, n = cache.timing_read()
    cache.free()
    assert n == 1
    if path == "decode":
        assert ms["decode"] > 0 and ms["select"] == ms["attn"] == ms["combine"] == 0
    else:
        assert ms["decode"] == 0 and min(ms["select"], ms["attn"], ms["combine"]) > 0


def test_decode_more_selection_workgroups_than_cus(gpu_lib):
    """B * Hq / 4 > 256 workgroups: the selector runs 8 wavefronts per workgroup (two per
    CU); ragged token tail, text, replicas bit-identical."""
    w = wl.LLAVA.replace(cfg_id=107, batch=70, n_q_heads=16, n_kv_heads=16, head_dim=64,
                         n_tokens=300, n_text=5, rank=32, r_lo=16, top_k=75, grid=None,
                         inner_dim=300)
    seqs = make_inputs(w, 2)
    out, sel = run_decode(w, seqs, gpu_lib)
    check_against_oracle(w, seqs, out, sel)
    for b in range(2, w.batch):
        assert np.array_equal(out[b], out[b % 2]) and np.array_equal(sel[b], sel[b % 2]), b


@pytest.mark.parametrize("n_text", [0, 7])
def test_decode_many_selection_workgroups_of_16_wavefronts(gpu_lib, n_text):
    """B * Hq / 4 > 256 workgroups whose four heads' tokens need more than 8 steps of 8
    wavefronts (N > 4096): the selector keeps 16 wavefronts per workgroup and runs two
    rounds of workgroups; grouped-query heads, a ragged token tail, with and without text."""
    w = wl.GQA.replace(cfg_id=113, batch=33, n_q_heads=32, n_kv_heads=8, head_dim=32,
                       n_tokens=4200, n_text=n_text, rank=32, r_lo=16, top_k=1050, inner_dim=256)
    seqs = make_inputs(w, 2)
    out, sel = run_decode(w, seqs, gpu_lib)
    check_against_oracle(w, seqs, out, sel)
    for b in range(2, w.batch):
        assert np.array_equal(out[b], out[b % 2]) and np.array_equal(sel[b], sel[b % 2]), b


@pytest.mark.parametrize("cfg,n_distinct,splits", [(2, 3, 0), (2, 3, 16), (3, 2, 0), (4, 2, 0),
                                                   (5, 2, 0)])
def test_decode_parity_full_configs(gpu_lib, cfg, n_distinct, splits):
    """Full batch at the workload's real shape (splits 0: the single-kernel decode where
    the shape allows; 16: the split-N path); distinct sequences are checked against
    the oracle and every replica must equal its original bit for bit."""
    w = wl.WORKLOADS[cfg]
    seqs = make_inputs(w, n_distinct)
    out, sel = run_decode(w, seqs, gpu_lib, splits=splits)
    err, flips = check_against_oracle(w, seqs, out, sel)
    for b in range(len(seqs), w.batch):
        o = b % len(seqs)
        assert np.array_equal(out[b], out[o]) and np.array_equal(sel[b], sel[o]), f"replica {b}"
    print(f"cfg {cfg} splits {splits}: max abs err {err:.3e}, band flips {flips}")


def test_empty_batch_is_a_noop(gpu_lib):
    c = gpu_lib.compress(None, None, batch=0, n_tokens=8, n_kv_heads=1, n_q_heads=1, head_dim=16,
                         rank=4, storage=torch.bfloat16)
    q = torch.zeros(0, 16, device="cuda")
    gpu_lib.decode(c, q, r_lo=2, top_k=2, scale=0.25)
    c.free()


def test_factor_roundtrip(gpu_lib):
    w = SMALL["bf16_ragged"]
    seqs = make_inputs(w)
    cache, q, tk, tv = upload_decode(w, seqs, gpu_lib)
    U_k, B_k, U_v, B_v = cache.get_factors()
    for b in range(w.batch):
        s = seqs[b % len(seqs)]
        assert np.array_equal(U_k[b].float().cpu().numpy(), s["U_k"])
        assert np.array_equal(U_v[b].float().cpu().numpy(), s["U_v"])
        assert np.array_equal(B_k[b].float().cpu().numpy(), s["B_k"])
        assert np.array_equal(B_v[b].float().cpu().numpy(), s["B_v"])
    cache.free()


def _decode_once(gpu_lib, w, cache, q, tk, tv, with_sel, timed=False):
    sel = None
    if with_sel:
        sel = torch.full((w.batch, w.n_q_heads, w.top_k), -1, dtype=torch.int32, device="cuda")
    if timed:
        cache.timing_enable(1)
    out = gpu_lib.decode(cache, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk, text_v=tv,
                         sel_out=sel, splits=0)
    ms = None
    if timed:
        ms, n = cache.timing_read()
        assert n == 1
        cache.timing_enable(0)
    torch.cuda.synchronize()
    return out.cpu(), (sel.cpu().numpy() if sel is not None else None), ms


@pytest.mark.parametrize("name", ["llava_full", "bf16_straddle_text", "bf16_rank64_lo16",
                                  "bf16_6_heads_gqa", "bf16_rank16"])
def test_decode_without_sel_out_is_the_checked_call(gpu_lib, name):
    """The call the benchmark times: splits = 0 and no sel_out, through the single-kernel
    decode.  Its output is compared with the oracle, and it must equal bit for bit the
    output of the same call with sel_out (whose sets are checked as well)."""
    w = wl.WORKLOADS[2] if name == "llava_full" else SMALL[name]
    seqs = make_inputs(w, 3)
    cache, q, tk, tv = upload_decode(w, seqs, gpu_lib)
    out0, _, ms = _decode_once(gpu_lib, w, cache, q, tk, tv, with_sel=False, timed=True)
    assert ms["decode"] > 0 and ms["select"] == ms["attn"] == ms["combine"] == 0, ms
    out1, sel, _ = _decode_once(gpu_lib, w, cache, q, tk, tv, with_sel=True)
    cache.free()
    assert torch.equal(out0, out1)
    out0 = out0.numpy()
    err, _ = check_against_oracle(w, seqs, out0, None)
    check_against_oracle(w, seqs, out1.numpy(), sel)
    for b in range(len(seqs), w.batch):
        assert np.array_equal(out0[b], out0[b % len(seqs)]), f"replica {b}"
    print(f"{name}: max abs err {err:.3e} without sel_out")


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_split_path_bench_call_without_sel_out(gpu_lib, cfg):
    """The call `bench.py --cfg N` times on the other workloads at full size: splits = 0
    and no sel_out, through the three-kernel path (the default split count).  Its output
    is compared with the oracle, and it equals bit for bit the same call with sel_out."""
    w = wl.WORKLOADS[cfg]
    seqs = make_inputs(w, 2)
    cache, q, tk, tv = upload_decode(w, seqs, gpu_lib)
    out0, _, ms = _decode_once(gpu_lib, w, cache, q, tk, tv, with_sel=False, timed=True)
    assert ms["decode"] == 0 and ms["select"] > 0 and ms["attn"] > 0 and ms["combine"] > 0, ms
    out1, sel, _ = _decode_once(gpu_lib, w, cache, q, tk, tv, with_sel=True)
    cache.free()
    assert torch.equal(out0, out1)
    err, _ = check_against_oracle(w, seqs, out0.numpy(), None)
    for b in range(len(seqs), w.batch):
        assert np.array_equal(out0.numpy()[b], out0.numpy()[b % len(seqs)]), f"replica {b}"
    print(f"cfg {cfg}: max abs err {err:.3e} without sel_out")
