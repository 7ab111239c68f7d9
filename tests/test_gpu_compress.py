"""GPU parity of ap_compress against the oracle's randomized factorisation
(needs an MI355X).

Both sides factor the same storage-exact K and V with the same test matrix Omega
(seeded Gaussian from rank_compressed_kv_ap_amd.workloads, or the library's own
Philox random signs, which oracle/philox.py reproduces bit for bit).  Bar: the
relative Frobenius reconstruction error ||A - U B|| / ||A|| of every factored
matrix within 1e-3 (relative) of the oracle's; singular values within 2e-3 of the
largest; B's rows orthonormal to the storage precision.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import torch_storage
from oracle.factorize import rsvd
from oracle.philox import sign_omega
from rank_compressed_kv_ap_amd import workloads as wl

pytestmark = pytest.mark.gpu

ERR_RTOL = 1e-3
SIG_RTOL = 2e-3
ORTH_TOL = {"bf16": 3e-2, "f32": 1e-4}


def rel_err(A, U, B):
    return float(np.linalg.norm(A - U @ B) / np.linalg.norm(A))


def host_inputs(w, n_distinct):
    S = min(w.batch, n_distinct)
    K = [wl.gen_kv(w, b, 0) for b in range(S)]
    V = [wl.gen_kv(w, b, 1) for b in range(S)]
    om = [(wl.gen_omega(w, b, 0), wl.gen_omega(w, b, 1)) for b in range(S)]
    return K, V, om


def gpu_compress(w, K, V, binding, om=None, seed=0, oversample=None, power_iters=None):
    """Factor the whole batch (sequence b = distinct input b % S) and download."""
    dt = torch_storage(w)
    S = len(K)
    idx = torch.tensor([b % S for b in range(w.batch)], device="cuda")
    k = torch.from_numpy(np.stack(K)).to(dt).cuda()[idx].contiguous()
    v = torch.from_numpy(np.stack(V)).to(dt).cuda()[idx].contiguous()
    omega = None
    if om is not None:
        omega = torch.from_numpy(np.stack([np.stack(o) for o in om]).astype(np.float32)).cuda()
        omega = omega[idx].contiguous()
    c = binding.compress(k, v, batch=w.batch, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                         n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank, storage=dt,
                         oversample=w.oversample if oversample is None else oversample,
                         power_iters=w.power_iters if power_iters is None else power_iters,
                         seed=seed, omega=omega)
    U_k, B_k, U_v, B_v = c.get_factors()
    sk, sv = c.get_sigma()
    torch.cuda.synchronize()
    del k, v, omega
    res = [x.float().cpu().numpy().astype(np.float64) for x in (U_k, B_k, U_v, B_v, sk, sv)]
    return c, res


def check_matrix(w, A, U, B, sig, omega, power_iters, label):
    Ur, Br, s = rsvd(A, w.rank, omega, power_iters, w.storage)
    e_ora, e_gpu = rel_err(A, Ur, Br), rel_err(A, U, B)
    assert abs(e_gpu - e_ora) <= ERR_RTOL * e_ora, f"{label}: error {e_gpu:.6e} vs oracle {e_ora:.6e}"
    assert np.all(np.isfinite(U)) and np.all(np.isfinite(B))
    assert np.max(np.abs(sig - s[:w.rank])) <= SIG_RTOL * s[0], f"{label}: singular values"
    assert np.all(np.diff(sig) <= 0), f"{label}: singular values not descending"
    G = B @ B.T
    assert np.max(np.abs(G - np.eye(w.rank))) <= ORTH_TOL[w.storage], f"{label}: B rows not orthonormal"
    return e_gpu, e_ora


SMALL = {
    "tiny_cfg": (wl.TINY, {}),
    "bf16_ragged": (wl.LLAVA.replace(cfg_id=201, batch=3, n_q_heads=4, n_kv_heads=4, head_dim=64,
                                     n_tokens=100, rank=24, grid=None, inner_dim=100), {}),
    "bf16_odd_width": (wl.GQA.replace(cfg_id=202, batch=2, n_q_heads=3, n_kv_heads=3, head_dim=21,
                                      n_tokens=77, rank=20, inner_dim=63), {}),
    "bf16_ell_is_n": (wl.LLAVA.replace(cfg_id=203, batch=2, n_q_heads=2, n_kv_heads=2, head_dim=64,
                                       n_tokens=40, rank=30, grid=None, inner_dim=40), {}),
    "f32_ragged": (wl.TINY.replace(cfg_id=204, batch=2, n_kv_heads=3, n_q_heads=3, head_dim=32,
                                   n_tokens=150, rank=12, inner_dim=96), {}),
    "bf16_no_power_no_oversample": (wl.GQA.replace(cfg_id=205, batch=2, n_q_heads=4, n_kv_heads=4,
                                                   head_dim=32, n_tokens=300, rank=32,
                                                   inner_dim=128, oversample=0, power_iters=0), {}),
    "bf16_rank128": (wl.VIDEO.replace(cfg_id=206, batch=1, n_kv_heads=2, n_q_heads=2, n_tokens=600,
                                      frames=None, inner_dim=256, oversample=0), {}),
    # rank 128 with the default oversampling: ell = 144, nine 16-column tiles; the core
    # SVD's rotation rows are split over two workgroups per matrix
    "bf16_rank128_ell144": (wl.VIDEO.replace(cfg_id=210, batch=2, n_kv_heads=2, n_q_heads=4, n_tokens=700,
                                             frames=None, inner_dim=256), {}),
    # ell = 136: nine tiles with a ragged last one (ell < ellp)
    "bf16_ell136": (wl.VIDEO.replace(cfg_id=211, batch=2, n_kv_heads=3, n_q_heads=3, n_tokens=400,
                                     rank=120, frames=None, inner_dim=300), {}),
    # fp32 at ell = 144
    "f32_ell144": (wl.TINY.replace(cfg_id=212, batch=1, n_kv_heads=4, n_q_heads=4, head_dim=64,
                                   n_tokens=300, rank=128, inner_dim=200), {}),
    # fp32 over several 128-row tiles and 16-wide k steps of the MFMA products, with a
    # ragged row tile (1000 rows) and a ragged k step (N = 1000 in A^T Q)
    "f32_wide": (wl.TINY.replace(cfg_id=213, batch=1, n_kv_heads=8, n_q_heads=8, head_dim=128,
                                 n_tokens=1000, rank=64, inner_dim=200), {}),
    # fp32 with widths and token counts not multiples of 4 (element-wise operand loads)
    "f32_odd": (wl.TINY.replace(cfg_id=214, batch=2, n_kv_heads=3, n_q_heads=3, head_dim=21,
                                n_tokens=131, rank=16, inner_dim=50), {}),
    # 576 tokens: A X over four and a half 128-row tiles, eight matrices
    "bf16_rows576": (wl.LLAVA.replace(cfg_id=215, batch=4, n_q_heads=4, n_kv_heads=4, head_dim=64,
                                      n_tokens=576, rank=32, grid=None, inner_dim=256), {}),
    # 8 matrices: the product kernels deal each matrix's row tiles to one XCD
    "bf16_eight_matrices": (wl.LLAVA.replace(cfg_id=209, batch=4, n_q_heads=4, n_kv_heads=4, head_dim=64,
                                             n_tokens=300, rank=24, grid=None, inner_dim=120), {}),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_compress_parity_small(gpu_lib, name):
    w, _ = SMALL[name]
    K, V, om = host_inputs(w, w.batch)
    c, (U_k, B_k, U_v, B_v, sk, sv) = gpu_compress(w, K, V, gpu_lib, om=om)
    c.free()
    for b in range(w.batch):
        for which, A, U, B, sg in ((0, K[b], U_k[b], B_k[b], sk[b]), (1, V[b], U_v[b], B_v[b], sv[b])):
            e_gpu, e_ora = check_matrix(w, A, U, B, sg, om[b][which], w.power_iters, f"b{b}/{'KV'[which]}")
    print(f"{name}: last error {e_gpu:.6e} (oracle {e_ora:.6e})")


def test_compress_seeded_signs_match_oracle_generator(gpu_lib):
    """omega == NULL: the device's Philox random signs equal oracle/philox.py's, so
    passing those signs explicitly gives bit-identical factors."""
    w = SMALL["bf16_ragged"][0]
    K, V, _ = host_inputs(w, w.batch)
    seed = 0x1234_5678_9ABC
    c1, r1 = gpu_compress(w, K, V, gpu_lib, seed=seed)
    c1.free()
    om = [(sign_omega(seed, 2 * b, w.width, w.ell), sign_omega(seed, 2 * b + 1, w.width, w.ell))
          for b in range(w.batch)]
    c2, r2 = gpu_compress(w, K, V, gpu_lib, om=om)
    c2.free()
    for x, y in zip(r1, r2):
        assert np.array_equal(x, y)
    U_k, B_k, U_v, B_v, sk, sv = r1
    for b in range(w.batch):
        check_matrix(w, K[b], U_k[b], B_k[b], sk[b], om[b][0], w.power_iters, f"b{b}/K")
        check_matrix(w, V[b], U_v[b], B_v[b], sv[b], om[b][1], w.power_iters, f"b{b}/V")


@pytest.mark.parametrize("storage,bound", [("f32", 1e-5), ("bf16", 1e-2)])
def test_compress_recovers_exact_low_rank(gpu_lib, storage, bound):
    # A of exact rank 5, factored at r = 8: only rounding error remains
    w = wl.TINY.replace(cfg_id=207, batch=2, n_tokens=130, storage=storage, rank=8)
    g = np.random.default_rng(7)
    K = [wl.to_storage(g.standard_normal((w.n_tokens, 5)) @ g.standard_normal((5, w.width)), storage)
         for _ in range(w.batch)]
    V = [wl.to_storage(g.standard_normal((w.n_tokens, 5)) @ g.standard_normal((5, w.width)), storage)
         for _ in range(w.batch)]
    c, (U_k, B_k, U_v, B_v, sk, sv) = gpu_compress(w, K, V, gpu_lib, seed=3)
    c.free()
    for b in range(w.batch):
        assert rel_err(K[b], U_k[b], B_k[b]) <= bound
        assert rel_err(V[b], U_v[b], B_v[b]) <= bound
        assert np.all(sk[b][5:] <= 1e-3 * sk[b][0]) and np.all(sv[b][5:] <= 1e-3 * sv[b][0])


def test_compress_zero_matrix_gives_zero_factors(gpu_lib):
    w = SMALL["bf16_ragged"][0]
    K = [np.zeros((w.n_tokens, w.width), np.float32) for _ in range(w.batch)]
    V = [wl.gen_kv(w, b, 1) for b in range(w.batch)]
    c, (U_k, B_k, U_v, B_v, sk, sv) = gpu_compress(w, K, V, gpu_lib, seed=1)
    c.free()
    assert np.all(np.isfinite(U_k)) and np.all(np.isfinite(B_k)) and np.all(np.isfinite(sk))
    assert np.max(np.abs(U_k)) == 0.0
    assert np.max(sk) <= 1e-12   # what the Cholesky shift leaves of an all-zero Gram
    for b in range(w.batch):   # the V half of the same call is unaffected
        assert rel_err(V[b], U_v[b], B_v[b]) < 1.0


def test_compress_empty_batch(gpu_lib):
    w = SMALL["bf16_ragged"][0].replace(batch=0)
    k = torch.zeros(0, w.n_tokens, w.width, dtype=torch.bfloat16, device="cuda")
    c = gpu_lib.compress(k, k, batch=0, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                         n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank,
                         storage=torch.bfloat16)
    c.free()


@pytest.mark.parametrize("cfg,n_distinct", [(2, 2), (3, 2), (4, 1), (5, 2)])
def test_compress_full_configs_then_decode(gpu_lib, cfg, n_distinct):
    """Full batch at the workload's real shape, with the default p = 16, q = 2 (the
    long-video layer: r = 128, ell = 144), distinct sequences tiled over it: they match
    the oracle's factorisation, replicas equal their originals bit for bit, and one
    decode step on the GPU's own factors matches the oracle's decode of those factors."""
    from gpu_helpers import check_against_oracle
    w = wl.WORKLOADS[cfg]
    assert w.oversample == 16 and w.power_iters == 2
    K, V, om = host_inputs(w, n_distinct)
    c, (U_k, B_k, U_v, B_v, sk, sv) = gpu_compress(w, K, V, gpu_lib, om=om)
    S = len(K)
    for b in range(S):
        check_matrix(w, K[b], U_k[b], B_k[b], sk[b], om[b][0], w.power_iters, f"b{b}/K")
        check_matrix(w, V[b], U_v[b], B_v[b], sv[b], om[b][1], w.power_iters, f"b{b}/V")
    for b in range(S, w.batch):
        o = b % S
        assert np.array_equal(U_k[b], U_k[o]) and np.array_equal(B_v[b], B_v[o]), f"replica {b}"
    # one decode step over the compressed cache
    seqs = []
    for b in range(S):
        s = dict(U_k=U_k[b], B_k=B_k[b], U_v=U_v[b], B_v=B_v[b], q=wl.gen_q(w, b))
        if w.n_text:
            s["text_k"] = wl.gen_text(w, b, 0, wl.factor_rms(U_k[b], B_k[b]))
            s["text_v"] = wl.gen_text(w, b, 1, wl.factor_rms(U_v[b], B_v[b]))
        seqs.append(s)
    idx = [b % S for b in range(w.batch)]
    dt = torch_storage(w)
    q = torch.from_numpy(np.stack([seqs[i]["q"] for i in idx])).float().cuda()
    tk = tv = None
    if w.n_text:
        tk = torch.from_numpy(np.stack([seqs[i]["text_k"] for i in idx])).to(dt).cuda()
        tv = torch.from_numpy(np.stack([seqs[i]["text_v"] for i in idx])).to(dt).cuda()
    sel = torch.full((w.batch, w.n_q_heads, w.top_k), -1, dtype=torch.int32, device="cuda")
    out = gpu_lib.decode(c, q, r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk, text_v=tv,
                         sel_out=sel)
    torch.cuda.synchronize()
    c.free()
    check_against_oracle(w, seqs, out.cpu().numpy(), sel.cpu().numpy())


def test_recompress_equals_fresh_compress(gpu_lib):
    """ap_recompress into a cache built from other inputs gives the factors a fresh
    ap_compress of the new inputs gives, bit for bit."""
    w = SMALL["bf16_ragged"][0]
    K1, V1, _ = host_inputs(w, w.batch)
    w2 = w.replace(cfg_id=208)
    K2, V2, om2 = host_inputs(w2, w2.batch)
    c_ref, ref = gpu_compress(w, K2, V2, gpu_lib, om=om2)
    c_ref.free()
    c, _ = gpu_compress(w, K1, V1, gpu_lib, seed=9)
    dt = torch_storage(w)
    k = torch.from_numpy(np.stack(K2)).to(dt).cuda()
    v = torch.from_numpy(np.stack(V2)).to(dt).cuda()
    om = torch.from_numpy(np.stack([np.stack(o) for o in om2]).astype(np.float32)).cuda()
    c.recompress(k, v, omega=om)
    U_k, B_k, U_v, B_v = c.get_factors()
    sk, sv = c.get_sigma()
    torch.cuda.synchronize()
    got = [x.float().cpu().numpy().astype(np.float64) for x in (U_k, B_k, U_v, B_v, sk, sv)]
    c.free()
    for x, y in zip(got, ref):
        assert np.array_equal(x, y)
