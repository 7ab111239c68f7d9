"""GPU parity of 4-bit token factors (AP_INT4 caches; needs an MI355X).

* Codes: the library quantizes float32 U on loading; the stored values code * scale
  (read back through ap_cache_get_factors) must equal oracle.quant's bit for bit: the
  same integer decisions from the same float32 inputs, including planted midpoint ties,
  zero columns, an outlier row and ragged token / rank tails.
* Decode: the oracle attends over the oracle's 4-bit round trip of the same U (equal
  to the library's, checked above) with the usual bars: top-k sets exact outside the
  1e-3 band, outputs within max-abs 2e-2.
* Compress: the relative reconstruction error of the stored factors (4-bit U, bf16 B)
  within 1e-3 (relative) of the oracle's randomized factorisation followed by the
  oracle's quantizer, with the same test matrix.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import check_against_oracle, make_inputs, run_decode, upload_decode
from oracle.factorize import round_to_storage, rsvd
from oracle.quant import quantize_dequant_u4
from rank_compressed_kv_ap_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = {
    "ragged": wl.LLAVA.replace(cfg_id=301, batch=3, n_q_heads=4, n_kv_heads=4, head_dim=64,
                               n_tokens=100, n_text=5, rank=24, r_lo=8, top_k=25, grid=None,
                               inner_dim=100, storage="int4"),
    "gqa_straddle": wl.GQA.replace(cfg_id=302, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=32,
                                   n_tokens=70, rank=40, r_lo=20, top_k=17, inner_dim=64,
                                   storage="int4"),
    "rank128": wl.VIDEO.replace(cfg_id=303, batch=2, n_tokens=300, top_k=75, frames=None,
                                inner_dim=300, storage="int4"),
    "text_straddle": wl.LLAVA.replace(cfg_id=304, batch=2, n_q_heads=8, n_kv_heads=8, head_dim=64,
                                      n_tokens=200, n_text=70, rank=48, r_lo=20, top_k=50,
                                      grid=None, inner_dim=200, storage="int4"),
    "heads48": wl.LLAVA.replace(cfg_id=305, batch=2, n_q_heads=48, n_kv_heads=16, head_dim=16,
                                n_tokens=64, n_text=3, rank=32, r_lo=16, top_k=16, grid=None,
                                inner_dim=64, storage="int4"),
}


def _planted(U):
    """Midpoint ties (block 1, column 1 has maximum 7: scale exactly 1), a zero
    column and an outlier row, on top of the generator's values."""
    U = U.copy()
    N, r = U.shape
    if N > 40 and r > 2:
        U[32:40, 1] = [7.0, 0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 6.5]
        U[40:min(N, 64), 1] = np.clip(U[40:min(N, 64), 1], -3.0, 3.0)
        U[:, r - 1] = 0.0
        U[5] = U[5] * np.float32(1e3)
    return U.astype(np.float32)


@pytest.mark.parametrize("name", ["ragged", "gqa_straddle", "rank128"])
def test_int4_codes_match_oracle(gpu_lib, name):
    w = SHAPES[name]
    seqs = make_inputs(w)
    for s in seqs:
        s["U_k"] = _planted(s["U_k"])
    cache, _, _, _ = upload_decode(w, seqs, gpu_lib)
    U_k, B_k, U_v, B_v = cache.get_factors()
    torch.cuda.synchronize()
    assert U_k.dtype == torch.float32 and B_k.dtype == torch.bfloat16
    for b in range(w.batch):
        s = seqs[b % len(seqs)]
        for got, U in ((U_k[b], s["U_k"]), (U_v[b], s["U_v"])):
            want = quantize_dequant_u4(U)
            assert np.array_equal(got.cpu().numpy().astype(np.float64), want), b
        assert np.array_equal(B_k[b].float().cpu().numpy(), s["B_k"])
    p, factor_bytes, _ = cache.info()
    nblk, NP = (w.n_tokens + 31) // 32, (w.rank + 15) // 16
    B_bytes = 2 * w.batch * 16 * NP * w.width * 2
    assert factor_bytes == 2 * w.batch * nblk * NP * 256 + w.batch * nblk * 2 * 16 * NP * 2 + B_bytes
    cache.free()


@pytest.mark.parametrize("name", list(SHAPES))
def test_int4_decode_parity_small(gpu_lib, name):
    w = SHAPES[name]
    seqs = make_inputs(w)
    out, sel = run_decode(w, seqs, gpu_lib)
    err, flips = check_against_oracle(w, seqs, out, sel)
    print(f"{name}: max abs err {err:.3e}, band flips {flips}")


# Shapes the single-kernel decode takes with 4-bit codes: r = 64 (four panels), r_lo =
# 16, head_dim a multiple of 32, two or three steps per wavefront.
FUSED = {
    "gqa6_text_tail": wl.LLAVA.replace(cfg_id=306, batch=3, n_q_heads=6, n_kv_heads=2, head_dim=64,
                                       n_tokens=300, n_text=20, rank=64, r_lo=16, top_k=75,
                                       grid=None, inner_dim=300, storage="int4"),
    "three_steps": wl.LLAVA.replace(cfg_id=307, batch=2, n_q_heads=4, n_kv_heads=4, head_dim=32,
                                    n_tokens=2100, n_text=0, rank=64, r_lo=16, top_k=500,
                                    grid=None, inner_dim=256, storage="int4"),
}


def _decode_timed(gpu_lib, w, cache, q, tk, tv, with_sel, splits=0):
    sel = None
    if with_sel:
        sel = torch.full((w.batch, w.n_q_heads, w.top_k), -1, dtype=torch.int32, device="cuda")
    cache.timing_enable(1)
    out = gpu_lib.decode(cache, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk, text_v=tv,
                         sel_out=sel, splits=splits)
    ms, n = cache.timing_read()
    cache.timing_enable(0)
    torch.cuda.synchronize()
    assert n == 1
    return out.cpu().numpy(), (sel.cpu().numpy() if sel is not None else None), ms


@pytest.mark.parametrize("name", list(FUSED))
def test_int4_single_kernel_parity(gpu_lib, name):
    """4-bit codes through the single-kernel decode: that kernel alone runs; output and
    top-k sets match the oracle; the call without sel_out (the one the benchmark times)
    gives the same output bit for bit; the split-N path agrees with the oracle too."""
    w = FUSED[name]
    seqs = make_inputs(w)
    cache, q, tk, tv = upload_decode(w, seqs, gpu_lib)
    out, sel, ms = _decode_timed(gpu_lib, w, cache, q, tk, tv, with_sel=True)
    assert ms["decode"] > 0 and ms["select"] == ms["attn"] == ms["combine"] == 0, ms
    err, flips = check_against_oracle(w, seqs, out, sel)
    out0, _, _ = _decode_timed(gpu_lib, w, cache, q, tk, tv, with_sel=False)
    assert np.array_equal(out0, out)
    out3, sel3, ms3 = _decode_timed(gpu_lib, w, cache, q, tk, tv, with_sel=True, splits=3)
    assert ms3["decode"] == 0 and ms3["attn"] > 0, ms3
    check_against_oracle(w, seqs, out3, sel3)
    cache.free()
    print(f"{name}: max abs err {err:.3e}, band flips {flips}")


@pytest.mark.parametrize("top_k,r_lo", [(0, 8), (100, 8), (25, 24), (1, 1)])
def test_int4_decode_edge_selection(gpu_lib, top_k, r_lo):
    w = SHAPES["ragged"].replace(top_k=top_k, r_lo=r_lo)
    seqs = make_inputs(w)
    out, sel = run_decode(w, seqs, gpu_lib)
    check_against_oracle(w, seqs, out, sel)


def test_int4_zero_query_ties_take_lowest_ids(gpu_lib):
    w = SHAPES["rank128"]
    seqs = make_inputs(w)
    for s in seqs:
        s["q"] = np.zeros_like(s["q"])
    out, sel = run_decode(w, seqs, gpu_lib)
    check_against_oracle(w, seqs, out, sel)
    assert all(sel[b, h].tolist() == list(range(w.top_k)) for b in range(w.batch) for h in range(w.n_q_heads))


@pytest.mark.parametrize("splits", [1, 3])
def test_int4_split_count_does_not_change_result(gpu_lib, splits):
    w = SHAPES["text_straddle"]
    seqs = make_inputs(w)
    a, sa = run_decode(w, seqs, gpu_lib, splits=splits)
    check_against_oracle(w, seqs, a, sa)


@pytest.mark.parametrize("cfg,n_distinct", [(2, 2), (3, 2)])
def test_int4_full_configs(gpu_lib, cfg, n_distinct):
    """The batch-32 LLaVA layer and the batch-64 GQA layer with 4-bit U: distinct
    sequences against the oracle, replicas bit-identical."""
    w = wl.WORKLOADS[cfg].replace(storage="int4")
    seqs = make_inputs(w, n_distinct)
    out, sel = run_decode(w, seqs, gpu_lib)
    err, flips = check_against_oracle(w, seqs, out, sel)
    for b in range(len(seqs), w.batch):
        o = b % len(seqs)
        assert np.array_equal(out[b], out[o]) and np.array_equal(sel[b], sel[o]), f"replica {b}"
    print(f"cfg {cfg} int4: max abs err {err:.3e}, band flips {flips}")


def test_int4_moving_average_selector(gpu_lib):
    """The importance-state selector on a 4-bit cache: state and output per step."""
    from test_gpu_ema import _run
    _run(gpu_lib, SHAPES["text_straddle"], "ema_head", 0.7, steps=3)


@pytest.mark.parametrize("name,shape", [
    ("ragged", wl.LLAVA.replace(cfg_id=311, batch=2, n_q_heads=4, n_kv_heads=4, head_dim=64,
                                n_tokens=100, rank=24, grid=None, inner_dim=100, storage="int4")),
    ("rank64", wl.GQA.replace(cfg_id=312, batch=2, n_q_heads=8, n_kv_heads=8, head_dim=64,
                              n_tokens=500, rank=64, inner_dim=256, storage="int4")),
])
def test_int4_compress_parity(gpu_lib, name, shape):
    w = shape
    K = [wl.gen_kv(w, b, 0) for b in range(w.batch)]
    V = [wl.gen_kv(w, b, 1) for b in range(w.batch)]
    om = [(wl.gen_omega(w, b, 0), wl.gen_omega(w, b, 1)) for b in range(w.batch)]
    k = torch.from_numpy(np.stack(K)).to(torch.bfloat16).cuda()
    v = torch.from_numpy(np.stack(V)).to(torch.bfloat16).cuda()
    omega = torch.from_numpy(np.stack([np.stack(o) for o in om]).astype(np.float32)).cuda()
    c = gpu_lib.compress(k, v, batch=w.batch, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                         n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank, storage="int4",
                         oversample=w.oversample, power_iters=w.power_iters, omega=omega)
    U_k, B_k, U_v, B_v = (x.float().cpu().numpy().astype(np.float64) for x in c.get_factors())
    c.free()
    for b in range(w.batch):
        for which, A, U, B in ((0, K[b], U_k[b], B_k[b]), (1, V[b], U_v[b], B_v[b])):
            Ur, Br, _ = rsvd(A, w.rank, om[b][which], w.power_iters, "f32")
            Uq = quantize_dequant_u4(Ur.astype(np.float32))
            Bq = round_to_storage(Br, "bf16")
            e_ora = np.linalg.norm(A - Uq @ Bq) / np.linalg.norm(A)
            e_gpu = np.linalg.norm(A - U @ B) / np.linalg.norm(A)
            assert abs(e_gpu - e_ora) <= 1e-3 * e_ora, (name, b, which, e_gpu, e_ora)
            print(f"{name} b{b} {'KV'[which]}: error {e_gpu:.6e} (oracle {e_ora:.6e})")
