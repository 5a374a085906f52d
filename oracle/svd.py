"""Exact polar factors for checking the iterations.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The polar factor of X = U Sigma V^T is U V^T ([Gram-NS], "Algorithm
advantages: from standard Newton-Schulz to Gram Newton-Schulz";
[NanoGPT-Muon], "From SGD to Muon": the closest (semi-)orthogonal matrix).

``jacobi_svd`` is a one-sided (Hestenes) Jacobi SVD written here so the
smallest pins do not depend on LAPACK; ``polar_eigh`` uses the symmetric
eigensolver of numpy on the Gram matrix for sizes where Jacobi is too slow:
for a full-rank wide X, polar(X) = (X X^T)^{-1/2} X.
"""

from __future__ import annotations

import numpy as np


def jacobi_svd(a: np.ndarray, tol: float = 1e-15, max_sweeps: int = 80):
    """One-sided Jacobi SVD of a (rows >= cols required; transpose otherwise).

    Repeatedly rotates pairs of columns (p, q) of a working copy W = A V until
    every pair is orthogonal to working precision.  Then the column norms of
    W are the singular values and W / sigma are the left singular vectors.
    Returns (U, sigma, V) with A = U diag(sigma) V^T, sigma unsorted.
    """
    w = np.array(a, dtype=np.float64, copy=True)
    rows, cols = w.shape
    if rows < cols:
        raise ValueError("jacobi_svd expects rows >= cols")
    v = np.eye(cols)
    for _ in range(max_sweeps):
        rotated = False
        for p in range(cols - 1):
            for q in range(p + 1, cols):
                alpha = float(w[:, p] @ w[:, p])
                beta = float(w[:, q] @ w[:, q])
                gamma = float(w[:, p] @ w[:, q])
                if abs(gamma) <= tol * np.sqrt(alpha * beta) or gamma == 0.0:
                    continue
                rotated = True
                zeta = (beta - alpha) / (2.0 * gamma)
                t = np.sign(zeta) / (abs(zeta) + np.sqrt(1.0 + zeta * zeta))
                if zeta == 0.0:
                    t = 1.0
                cs = 1.0 / np.sqrt(1.0 + t * t)
                sn = cs * t
                wp = w[:, p].copy()
                w[:, p] = cs * wp - sn * w[:, q]
                w[:, q] = sn * wp + cs * w[:, q]
                vp = v[:, p].copy()
                v[:, p] = cs * vp - sn * v[:, q]
                v[:, q] = sn * vp + cs * v[:, q]
        if not rotated:
            break
    sigma = np.sqrt(np.sum(w * w, axis=0))
    u = w / np.where(sigma > 0, sigma, 1.0)[None, :]
    return u, sigma, v


def polar_jacobi(m: np.ndarray) -> np.ndarray:
    """U V^T from ``jacobi_svd``; full rank assumed (tiny inputs only)."""
    x = np.asarray(m, dtype=np.float64)
    if x.shape[0] >= x.shape[1]:
        u, _, v = jacobi_svd(x)
        return u @ v.T
    u, _, v = jacobi_svd(x.T)
    return (u @ v.T).T


def polar_eigh(m: np.ndarray) -> np.ndarray:
    """U V^T via the eigendecomposition of the smaller Gram matrix.

    For wide X (n <= m): X X^T = U S^2 U^T, so U V^T = U S^{-1} U^T X.
    Full rank assumed.
    """
    x = np.asarray(m, dtype=np.float64)
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T
    evals, evecs = np.linalg.eigh(x @ x.T)
    inv_sqrt = 1.0 / np.sqrt(np.maximum(evals, np.finfo(np.float64).tiny))
    out = (evecs * inv_sqrt[None, :]) @ (evecs.T @ x)
    return out.T if transposed else out


def orthogonalization_mse(approx: np.ndarray, m: np.ndarray,
                          exact: np.ndarray = None) -> float:
    """Mean squared singular-value error of an orthogonalization of m.

    Reading of the ROOT page's "MSE": ``||NS(M) - polar(M)||_F^2 / min(r, c)``,
    i.e. the squared Frobenius error per singular value.  (The per-entry mean
    would be thousands of times smaller than the page's 0.0499 at
    2048 x 2048; this normalization reproduces the printed figure.)
    """
    if exact is None:
        exact = polar_eigh(m)
    d = np.asarray(approx, dtype=np.float64) - exact
    return float(np.sum(d * d) / min(exact.shape))
