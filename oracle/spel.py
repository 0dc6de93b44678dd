"""SPEL projector update on the Stiefel manifold, fp64, algorithm steps.

Source: *Learned Subspace Compression for Communication-Efficient Pipeline
Parallelism*, Section 3.3, Eq. (4) tangent projection g - A sym(A^T g) with
sym(M) = (M + M^T)/2, Eq. (5) heavy-ball momentum, Eq. (6) spectral LMO
direction d = Polar(m), Eq. (7) retraction A <- Polar(A - alpha d), in the
order of Algorithm 1, step 4.

The pages name Polar Express for Polar(.) but print no coefficients.  Here
the polar map is fixed to the cubic Newton-Schulz iteration
X <- 1.5 X - 0.5 X (X^T X), 8 iterations, with the Gram matrix X^T X formed
first.  Readings taken where the pages are silent:
  * the LMO input is scaled by its Frobenius norm (all singular values <= 1,
    inside the iteration's convergence region 0 < s < sqrt(3)); a zero
    momentum gives a zero direction;
  * the retraction input A - alpha d is NOT rescaled (its singular values lie
    in [1 - alpha, 1 + alpha] when ||d||_2 <= 1);
  * the momentum buffer starts at zero.

Test infrastructure only: see the package docstring.
"""
from __future__ import annotations

import numpy as np


def sym(M) -> np.ndarray:
    """sym(M) = (M + M^T) / 2 (Section 3.3, below Eq. (7))."""
    M = np.asarray(M, dtype=np.float64)
    return 0.5 * (M + M.T)


def tangent_project(A, g) -> np.ndarray:
    """Eq. (4): g_R = g - A sym(A^T g)."""
    A = np.asarray(A, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    return g - A @ sym(A.T @ g)


def momentum(m, gR, beta: float) -> np.ndarray:
    """Eq. (5): m <- beta m + (1 - beta) g_R."""
    return beta * np.asarray(m, dtype=np.float64) + (1.0 - beta) * np.asarray(gR, dtype=np.float64)


def newton_schulz(X, iters: int) -> np.ndarray:
    """Cubic Newton-Schulz polar iteration: X <- 1.5 X - 0.5 X (X^T X)."""
    X = np.array(X, dtype=np.float64, copy=True)
    for _ in range(int(iters)):
        gram = X.T @ X
        X = 1.5 * X - 0.5 * (X @ gram)
    return X


def lmo_direction(m, iters: int) -> np.ndarray:
    """Eq. (6): d = Polar(m), computed as NS(m / ||m||_F); zero if m == 0."""
    m = np.asarray(m, dtype=np.float64)
    f = float(np.sqrt(np.sum(m * m)))
    if f == 0.0:
        return np.zeros_like(m)
    return newton_schulz(m / f, iters)


def retract(A, D, alpha: float, iters: int) -> np.ndarray:
    """Eq. (7): A <- Polar(A - alpha d), the input taken unscaled."""
    return newton_schulz(np.asarray(A, dtype=np.float64) - alpha * np.asarray(D, dtype=np.float64), iters)


def spel_step(A, g, m, alpha: float, beta: float, iters: int = 8):
    """One SPEL step (Algorithm 1, step 4).  Returns (A_new, m_new, d, g_R)."""
    gR = tangent_project(A, g)
    m_new = momentum(m, gR, beta)
    D = lmo_direction(m_new, iters)
    A_new = retract(A, D, alpha, iters)
    return A_new, m_new, D, gR
