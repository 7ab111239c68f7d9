"""The allocation-free re-factorisation (ap_recompress_noalloc) against ap_recompress
(needs an MI355X).

Its factorisation workspace is the library's fixed device array; the kernels are the
same, so the factors and singular values must equal ap_recompress's bit for bit.  Two
calls in a row, the second with a smaller shape (the fixed array keeps the first
call's contents, which must not leak into the second), an fp32 call with the caller's
test matrix, and a shape too large for the array, refused before anything runs.
"""
import numpy as np
import pytest
import torch

from rank_compressed_kv_ap_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _inputs(w, dt):
    K = np.stack([wl.gen_kv(w, b, 0) for b in range(w.batch)])
    V = np.stack([wl.gen_kv(w, b, 1) for b in range(w.batch)])
    return (torch.from_numpy(K).to(dt).cuda().contiguous(),
            torch.from_numpy(V).to(dt).cuda().contiguous())


def _cache(binding, w, dt):
    return binding.compress(None, None, batch=w.batch, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                            n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank, storage=dt,
                            oversample=w.oversample, power_iters=w.power_iters)


def _download(c):
    out = list(c.get_factors()) + list(c.get_sigma())
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in out]


def _both(binding, w, dt, seed=0, omega=None):
    """Factors from ap_recompress and from ap_recompress_noalloc of the same inputs."""
    k, v = _inputs(w, dt)
    ref, fix = _cache(binding, w, dt), _cache(binding, w, dt)
    ref.recompress(k, v, seed=seed, omega=omega)
    fix.recompress_noalloc(k, v, seed=seed, omega=omega)
    a, b = _download(ref), _download(fix)
    ref.free()
    fix.free()
    return a, b


SHAPE_A = wl.LLAVA.replace(cfg_id=301, batch=3, n_q_heads=4, n_kv_heads=4, head_dim=64,
                           n_tokens=300, rank=24, grid=None, inner_dim=200)
SHAPE_B = wl.GQA.replace(cfg_id=302, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         n_tokens=100, rank=16, inner_dim=100)


def test_noalloc_equals_recompress_two_calls_second_smaller(gpu_lib):
    for w, seed in ((SHAPE_A, 11), (SHAPE_B, 12)):
        a, b = _both(gpu_lib, w, torch.bfloat16, seed=seed)
        for x, y in zip(a, b):
            assert x.shape == y.shape and np.array_equal(x, y), w.name
        # the factors are a real factorisation of the inputs, not zeros
        U_k, B_k = a[0], a[1]
        K = np.stack([wl.gen_kv(w, bb, 0) for bb in range(w.batch)]).astype(np.float64)
        err = np.linalg.norm(K - U_k.astype(np.float64) @ B_k.astype(np.float64)) / np.linalg.norm(K)
        assert err < 0.5, err


def test_noalloc_f32_with_caller_omega(gpu_lib):
    w = wl.TINY.replace(cfg_id=303, batch=2, n_tokens=90, rank=12)
    om = np.stack([np.stack([wl.gen_omega(w, b, 0), wl.gen_omega(w, b, 1)]) for b in range(w.batch)])
    omega = torch.from_numpy(om.astype(np.float32)).cuda().contiguous()
    a, b = _both(gpu_lib, w, torch.float32, omega=omega)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_noalloc_refuses_a_shape_beyond_the_fixed_workspace(gpu_lib):
    from rank_compressed_kv_ap_amd import binding as bnd
    # 64 matrices of 2880 x 4096 at ell = 80 need about 370 MB of workspace
    w = wl.LLAVA.replace(cfg_id=304, batch=32)
    c = gpu_lib.compress(None, None, batch=w.batch, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                         n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank,
                         storage=torch.bfloat16)
    before = _download(c)
    k = torch.zeros(w.batch, w.n_tokens, w.width, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bnd.APError) as ei:
        c.recompress_noalloc(k, k, seed=1)
    assert ei.value.status == bnd.AP_ERR_UNSUPPORTED
    assert "bytes" in str(ei.value)
    after = _download(c)
    c.free()
    for x, y in zip(before, after):
        assert np.array_equal(x, y)
    # the fixed workspace still serves a shape that fits, after the refusal
    a, b = _both(gpu_lib, SHAPE_B, torch.bfloat16, seed=5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
