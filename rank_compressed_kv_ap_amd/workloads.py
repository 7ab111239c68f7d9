"""Seeded synthetic workloads for compressed-KV decode attention.

This module only *draws inputs*: Gaussian factors, a power-law spectrum, the
patch-grid smoothing and frame correlation that shape them, text tokens,
queries and random test matrices.  It holds none of the method's arithmetic
(no SVD, no projection, no selection, no softmax) and is the only code shared
by the CPU oracle, the tests and the benchmark.

The shapes stand in for the workloads of the AttentionPack summaries
("Attention-aware Inference Optimizations for Large Vision-Language Models with
Memory-efficient Decoding", gist.science es/fr/de, §4 Resultados / Résultats /
Ergebnisse): LLaVA-1.5-7B-like layers (32 heads of 128, a few thousand visual
tokens per image), a grouped-query variant and a long video context of 64
frames.  No dataset or model weights are used; every value is synthetic.

Seeding: one ``numpy.random.Generator(PCG64(SeedSequence([0xA77E, cfg, b,
tensor_id, step])))`` per tensor, so any sequence of a batch can be drawn on
its own.  tensor_id: 0 K, 1 V, 2 text K, 3 text V, 4 query, 5 Omega_K,
6 Omega_V, 16 factored K, 17 factored V.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SEED_ROOT = 0xA77E
TID_K, TID_V, TID_TEXT_K, TID_TEXT_V, TID_Q, TID_OMEGA_K, TID_OMEGA_V = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload shape and the law its K/V are drawn from."""

    name: str
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int          # N visual tokens (compressed)
    n_text: int            # T text tokens (kept dense)
    rank: int              # r
    r_lo: int              # low rank used for unselected tokens
    top_k: int             # tokens per (sequence, query head) at full rank
    storage: str           # "f32", "bf16" or "int4" (4-bit U; K, V, text, B in bf16)
    inner_dim: int         # m: number of spectral components drawn
    sigma_exp: float       # sigma_i = i ** -sigma_exp
    sigma_cut: int         # sigma_i = 0 for i > sigma_cut (0: no cut)
    noise: float           # iid N(0, noise^2) added after the low-rank part
    grid: Optional[tuple]  # (rows, cols) patch grid smoothed by a 3x3 box filter
    frames: Optional[tuple]  # (frames, patches_per_frame, rho) AR(1) across frames
    oversample: int = 16
    power_iters: int = 2
    decode_steps: int = 1

    @property
    def width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def ell(self) -> int:
        return min(self.rank + self.oversample, self.n_tokens, self.width)

    def sigmas(self) -> np.ndarray:
        i = np.arange(1, self.inner_dim + 1, dtype=np.float64)
        s = i ** (-self.sigma_exp)
        if self.sigma_cut:
            s[self.sigma_cut:] = 0.0
        return s

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _wl(**kw) -> Workload:
    return Workload(**kw)


TINY = _wl(name="tiny", cfg_id=1, batch=1, n_q_heads=4, n_kv_heads=4, head_dim=64,
           n_tokens=256, n_text=0, rank=16, r_lo=4, top_k=64, storage="f32",
           inner_dim=32, sigma_exp=1.0, sigma_cut=32, noise=0.01, grid=None, frames=None)
LLAVA = _wl(name="llava7b_layer", cfg_id=2, batch=32, n_q_heads=32, n_kv_heads=32,
            head_dim=128, n_tokens=2880, n_text=64, rank=64, r_lo=16, top_k=720,
            storage="bf16", inner_dim=2880, sigma_exp=0.8, sigma_cut=0, noise=0.02,
            grid=(48, 60), frames=None)
GQA = _wl(name="gqa", cfg_id=3, batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
          n_tokens=8192, n_text=0, rank=64, r_lo=16, top_k=2048, storage="bf16",
          inner_dim=1024, sigma_exp=0.8, sigma_cut=0, noise=0.02, grid=None, frames=None)
VIDEO = _wl(name="long_video", cfg_id=4, batch=4, n_q_heads=32, n_kv_heads=32,
            head_dim=128, n_tokens=32768, n_text=0, rank=128, r_lo=32, top_k=8192,
            storage="bf16", inner_dim=4096, sigma_exp=0.8, sigma_cut=0, noise=0.02,
            grid=None, frames=(64, 512, 0.9))
E2E = _wl(name="compress_decode_e2e", cfg_id=5, batch=256, n_q_heads=32, n_kv_heads=32,
          head_dim=128, n_tokens=4096, n_text=0, rank=64, r_lo=16, top_k=1024,
          storage="bf16", inner_dim=4096, sigma_exp=0.8, sigma_cut=0, noise=0.02,
          grid=None, frames=None, decode_steps=16)

WORKLOADS = {w.cfg_id: w for w in (TINY, LLAVA, GQA, VIDEO, E2E)}


def rng(cfg_id: int, b: int, tensor_id: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([SEED_ROOT, cfg_id, b, tensor_id, step])))


# ---------------------------------------------------------------- rounding
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returned as float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def to_storage(x: np.ndarray, storage: str) -> np.ndarray:
    """Values exactly as a device buffer of the storage dtype holds them (float32).
    A 4-bit cache keeps its dense tensors (K, V, text, B) in bf16."""
    if storage == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if storage in ("bf16", "int4"):
        return round_bf16(x)
    raise ValueError(storage)


def u_storage(storage: str) -> str:
    """Rounding of the token factor U handed to the library: a 4-bit cache takes U as
    float32 values and chooses its codes itself."""
    return "f32" if storage == "int4" else storage


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """uint16 payload of float32 values that are already bfloat16-exact."""
    return (np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- structure
def _box3(X: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """3x3 box filter over a rows x cols token grid (row-major token order).

    Edge tokens average only the neighbours that lie inside the grid.
    """
    n = rows * cols
    G = X[:n].reshape(rows, cols, -1)
    acc = np.zeros_like(G)
    cnt = np.zeros((rows, cols, 1))
    for di in (-1, 0, 1):
        for dj in (-1, 0, 1):
            i0, i1 = max(0, -di), rows - max(0, di)
            j0, j1 = max(0, -dj), cols - max(0, dj)
            acc[i0:i1, j0:j1] += G[i0 + di:i1 + di, j0 + dj:j1 + dj]
            cnt[i0:i1, j0:j1] += 1.0
    out = X.copy()
    out[:n] = (acc / cnt).reshape(n, -1)
    return out


def _ar1_frames(g: np.random.Generator, frames: int, patches: int, rho: float,
                m: int) -> np.ndarray:
    """Rows of the left factor, correlated across frames by AR(1) per patch."""
    X = np.empty((frames * patches, m))
    X[:patches] = g.standard_normal((patches, m))
    a = math.sqrt(1.0 - rho * rho)
    for f in range(1, frames):
        X[f * patches:(f + 1) * patches] = (rho * X[(f - 1) * patches:f * patches]
                                            + a * g.standard_normal((patches, m)))
    return X


def _left_factor(w: Workload, g: np.random.Generator, m: int, n_tokens: int) -> np.ndarray:
    if w.frames is not None and n_tokens == w.frames[0] * w.frames[1]:
        G1 = _ar1_frames(g, w.frames[0], w.frames[1], w.frames[2], m)
    else:
        G1 = g.standard_normal((n_tokens, m))
    if w.grid is not None and n_tokens >= w.grid[0] * w.grid[1]:
        G1 = _box3(G1, w.grid[0], w.grid[1])
    return G1


def gen_kv(w: Workload, b: int, which: int, step: int = 0) -> np.ndarray:
    """One heads-merged visual K (which=0) or V (which=1) matrix [N, W].

    A = G1 diag(sigma) G2^T (+ smoothing / frame correlation on G1's rows)
    + iid N(0, noise^2), rounded once to the storage dtype (float32 values).
    """
    g = rng(w.cfg_id, b, TID_K if which == 0 else TID_V, step)
    m = w.inner_dim
    G1 = _left_factor(w, g, m, w.n_tokens)
    G2 = g.standard_normal((w.width, m))
    A = (G1 * w.sigmas()[None, :]) @ G2.T
    if w.noise:
        A += w.noise * g.standard_normal(A.shape)
    return to_storage(A, w.storage)


def gen_factors(w: Workload, b: int, which: int, step: int = 0):
    """A compressed cache drawn directly in factored form.

    U = G1[:, :r] diag(sigma_1..r) (same row structure as gen_kv) and
    B = G2[:, :r]^T, each rounded to the storage dtype (U to float32 for a 4-bit
    cache, which quantizes it on loading).  U @ B is the rank-r
    part of the workload's K (which=0) or V (which=1) law; no factorisation
    is run to produce it.  Returns float32 arrays U [N, r], B [r, W].
    """
    g = rng(w.cfg_id, b, 16 + which, step)
    r = w.rank
    G1 = _left_factor(w, g, r, w.n_tokens)
    G2 = g.standard_normal((w.width, r))
    s = w.sigmas()[:r]
    U = G1 * s[None, :]
    return to_storage(U, u_storage(w.storage)), to_storage(G2.T, w.storage)


def gen_text(w: Workload, b: int, which: int, rms: float, step: int = 0) -> np.ndarray:
    """Dense text tokens [T, W]: iid N(0,1) scaled to the given RMS, rounded."""
    g = rng(w.cfg_id, b, TID_TEXT_K if which == 0 else TID_TEXT_V, step)
    X = rms * g.standard_normal((w.n_text, w.width))
    return to_storage(X, w.storage)


def factor_rms(U: np.ndarray, B: np.ndarray) -> float:
    """RMS of the entries of U @ B, from the r x r Gram products (no N x W product)."""
    U = U.astype(np.float64)
    B = B.astype(np.float64)
    fro2 = float(np.sum((U.T @ U) * (B @ B.T)))
    return math.sqrt(fro2 / (U.shape[0] * B.shape[1]))


def gen_q(w: Workload, b: int, step: int = 0) -> np.ndarray:
    """Query [Hq * d] ~ N(0, 1), float32."""
    return rng(w.cfg_id, b, TID_Q, step).standard_normal(w.n_q_heads * w.head_dim).astype(np.float32)


def gen_omega(w: Workload, b: int, which: int) -> np.ndarray:
    """Random test matrix Omega [W, ell] ~ N(0,1), rounded to the storage dtype."""
    g = rng(w.cfg_id, b, TID_OMEGA_K if which == 0 else TID_OMEGA_V)
    return to_storage(g.standard_normal((w.width, w.ell)), w.storage)


def gen_decode_inputs(w: Workload, b: int, step: int = 0) -> dict:
    """Everything one sequence's decode step reads, as float32 storage-exact arrays."""
    Uk, Bk = gen_factors(w, b, 0)
    Uv, Bv = gen_factors(w, b, 1)
    out = dict(U_k=Uk, B_k=Bk, U_v=Uv, B_v=Bv, q=gen_q(w, b, step))
    if w.n_text:
        out["text_k"] = gen_text(w, b, 0, factor_rms(Uk, Bk))
        out["text_v"] = gen_text(w, b, 1, factor_rms(Uv, Bv))
    else:
        out["text_k"] = np.zeros((0, w.width), np.float32)
        out["text_v"] = np.zeros((0, w.width), np.float32)
    return out
