"""Randomized low-rank factorisation of a heads-merged K or V — oracle only.

What is factored ([fr §2.A], [es §2.A], [de §2.A]): per sequence, the visual
keys (and separately the values) of all heads are concatenated along the
hidden axis into one N x (H*d) matrix and replaced by a compressed matrix
K* (N x R) and a decompression matrix D_k (R x H*d), so that K ~= K* D_k.
Storage falls from N*H*d to N*R + R*H*d values ([fr §2.A "Gain"]).

The summaries name an SVD but no algorithm.  The factorisation here is the
randomized subspace iteration of Halko, Martinsson & Tropp (SIAM Review 2011,
range finder with q power iterations, then the SVD of the small projected
matrix), with a Gaussian test matrix Omega of ell = r + p columns supplied by
the caller.  Reading chosen for the summaries' open points:
  * the singular values are folded into the compressed matrix:
    U = Q Uc[:, :r] diag(s_r) (N x r), B = Vc[:, :r]^T (r x W), so B has
    orthonormal rows and the components are ordered by decreasing s;
  * every product with A is re-orthonormalised (modified Gram–Schmidt, run
    twice); a column that vanishes under projection (rank-deficient input)
    is set to zero rather than normalised;
  * U and B are rounded once to the storage dtype at the end.

Pins: exact recovery of a rank-k matrix when ell >= k, error never below the
Eckart–Young optimum, and within 1% of it on the workloads' spectra
(tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

from .jacobi import jacobi_svd


def round_to_storage(x: np.ndarray, storage: str) -> np.ndarray:
    """Round float64 values to float32 or bfloat16 (nearest, ties to even).

    Returned as float64 holding exactly the representable values.
    """
    x = np.asarray(x, dtype=np.float64)
    f32 = x.astype(np.float32)
    if storage == "f32":
        return f32.astype(np.float64)
    if storage != "bf16":
        raise ValueError(storage)
    bits = f32.view(np.uint32).astype(np.int64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) >> 16) << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def orth_mgs2(Y: np.ndarray, drop_tol: float = 1e-12) -> np.ndarray:
    """Orthonormal basis of range(Y) by modified Gram–Schmidt applied twice.

    A column whose norm after projection is at most drop_tol times its norm
    before projection is replaced by zeros (the input was rank deficient).
    """
    Q = np.array(Y, dtype=np.float64, copy=True)
    n = Q.shape[1]
    for _ in range(2):
        for j in range(n):
            before = np.linalg.norm(Q[:, j])
            for i in range(j):
                Q[:, j] -= (Q[:, i] @ Q[:, j]) * Q[:, i]
            after = np.linalg.norm(Q[:, j])
            if before == 0.0 or after <= drop_tol * before:
                Q[:, j] = 0.0
            else:
                Q[:, j] /= after
    return Q


def rsvd(A: np.ndarray, r: int, omega: np.ndarray, power_iters: int = 2,
         storage: str | None = None):
    """Rank-r factors of A (N x W) from the test matrix omega (W x ell).

    Steps (HMT 2011, subspace iteration):
      Q  = orth(A Omega)
      repeat power_iters times:  Qt = orth(A^T Q);  Q = orth(A Qt)
      C  = Q^T A                          (ell x W)
      C  = Uc diag(s) Vc^T                (one-sided Jacobi SVD)
      U  = Q Uc[:, :r] diag(s[:r]),  B = Vc[:, :r]^T
    Returns (U, B, s) with s the ell singular values of C; U and B are rounded
    to ``storage`` when it is given.
    """
    A = np.asarray(A, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    ell = omega.shape[1]
    if not (1 <= r <= ell):
        raise ValueError("need 1 <= r <= ell")
    Q = orth_mgs2(A @ omega)
    for _ in range(power_iters):
        Qt = orth_mgs2(A.T @ Q)
        Q = orth_mgs2(A @ Qt)
    C = Q.T @ A
    Uc, s, Vc = jacobi_svd(C)
    U = (Q @ Uc[:, :r]) * s[None, :r]
    B = Vc[:, :r].T
    if storage is not None:
        U = round_to_storage(U, storage)
        B = round_to_storage(B, storage)
    return U, B, s
