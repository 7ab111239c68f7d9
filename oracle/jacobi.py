"""One-sided (Hestenes) Jacobi SVD in float64 — oracle, test infrastructure only.

The summaries say the heads-merged K and V matrices are factored by a singular
value decomposition ([es §2.A], [fr §2.A "Mécanisme"], [de §2.A "Technik"]).
The oracle computes that SVD with the textbook one-sided Jacobi method
(Hestenes 1958): plane rotations are applied to pairs of columns until every
pair is numerically orthogonal; the column norms are then the singular values.

Pins (tests/test_oracle_pins.py): singular values against numpy.linalg.svd,
orthogonality of both factors, exact reconstruction, Eckart–Young truncation
error, exact recovery of a rank-k matrix.
"""
from __future__ import annotations

import numpy as np


def _rotate_columns(X: np.ndarray, V: np.ndarray, tol: float, max_sweeps: int) -> None:
    """Orthogonalise the columns of X in place, accumulating the rotations in V."""
    n = X.shape[1]
    for _ in range(max_sweeps):
        rotated = False
        for i in range(n - 1):
            for j in range(i + 1, n):
                xi, xj = X[:, i], X[:, j]
                alpha = float(xi @ xi)
                beta = float(xj @ xj)
                gamma = float(xi @ xj)
                if gamma == 0.0 or abs(gamma) <= tol * np.sqrt(alpha * beta):
                    continue
                rotated = True
                # angle that zeroes the (i, j) inner product
                zeta = (beta - alpha) / (2.0 * gamma)
                t = np.copysign(1.0, zeta) / (abs(zeta) + np.sqrt(1.0 + zeta * zeta))
                c = 1.0 / np.sqrt(1.0 + t * t)
                s = c * t
                new_i = c * xi - s * xj
                new_j = s * xi + c * xj
                X[:, i], X[:, j] = new_i, new_j
                vi, vj = V[:, i].copy(), V[:, j].copy()
                V[:, i] = c * vi - s * vj
                V[:, j] = s * vi + c * vj
        if not rotated:
            return
    raise RuntimeError("Jacobi SVD did not converge")


def jacobi_svd(A: np.ndarray, tol: float = 1e-15, max_sweeps: int = 80):
    """SVD A = U diag(s) V^T of an m x n matrix by one-sided Jacobi.

    Returns U (m x p), s (p, descending), V (n x p) with p = min(m, n).  Zero
    singular values get a zero column in U.  Each singular pair is signed so
    that the entry of largest magnitude in its left vector is positive (this
    only fixes the sign freedom; it does not change U diag(s) V^T).
    """
    A = np.asarray(A, dtype=np.float64)
    m, n = A.shape
    if m < n:
        Ut, s, Vt = jacobi_svd(A.T, tol, max_sweeps)
        return Vt, s, Ut
    X = A.copy()
    V = np.eye(n)
    _rotate_columns(X, V, tol, max_sweeps)
    s = np.sqrt(np.einsum("ij,ij->j", X, X))
    order = np.argsort(-s, kind="stable")
    s, X, V = s[order], X[:, order], V[:, order]
    U = np.zeros_like(X)
    nz = s > 0
    U[:, nz] = X[:, nz] / s[nz]
    for j in range(n):
        if not nz[j]:
            continue
        if U[np.argmax(np.abs(U[:, j])), j] < 0:
            U[:, j] = -U[:, j]
            V[:, j] = -V[:, j]
    return U, s, V
