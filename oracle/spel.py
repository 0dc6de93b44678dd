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


# ------------------------------------------------------------ Polar Express --
# Section 3.3 and Table 8 name Polar Express (the paper's reference [2]) for the
# polar map, with 5 LMO steps and 7 retraction steps, but print no
# coefficients.  Reading taken here (the published method as this oracle
# understands it): step t applies the odd quintic p_t(x) = a x + b x^3 + c x^5
# to the singular values, X <- X (a I + b S + c S^2) with S = X^T X, where p_t
# is the best uniform approximation of 1 on the current singular-value
# interval [l_t, u_t] (Remez exchange on four alternation points), and the
# next interval is p_t's range there, [1 - E_t, 1 + E_t].  The input is scaled
# by its Frobenius norm (all singular values <= 1) and the first interval is
# [ell, 1].  Once an interval is narrower than 1e-4 the limit polynomial
# (15 x - 10 x^3 + 3 x^5) / 8 is used: there the exchange system is
# ill-conditioned, and the limit quintic's error is already O(width^3).


def _remez_odd_quintic(lo: float, hi: float, iters: int = 60):
    """Minimax odd quintic a x + b x^3 + c x^5 for the constant 1 on [lo, hi]:
    returns ((a, b, c), E), E the maximum error |1 - p|."""
    # start from four evenly spread points of the interval
    xs = np.array([lo, lo + 0.25 * (hi - lo), lo + 0.75 * (hi - lo), hi])
    coef, E = None, None
    for _ in range(iters):
        M = np.array([[x, x ** 3, x ** 5, (-1.0) ** i] for i, x in enumerate(xs)])
        a, b, c, e = np.linalg.solve(M, np.ones(4))
        coef, E = (a, b, c), abs(e)
        # interior alternation points: the critical points of p, 5 c y^2 + 3 b y + a = 0, y = x^2
        disc = 9.0 * b * b - 20.0 * a * c
        if c == 0.0 or disc < 0.0:
            break
        ys = sorted(((-3.0 * b - np.sqrt(disc)) / (10.0 * c), (-3.0 * b + np.sqrt(disc)) / (10.0 * c)))
        inner = [np.sqrt(y) for y in ys if y > 0.0 and lo < np.sqrt(y) < hi]
        if len(inner) != 2:
            break
        new = np.array([lo, inner[0], inner[1], hi])
        done = np.max(np.abs(new - xs)) <= 1e-15 * hi
        xs = new
        if done:
            break
    return coef, E


def polar_express_coefficients(ell: float, steps: int):
    """The greedy minimax schedule: [(a, b, c)] and the errors [E_t]."""
    lo, hi = float(ell), 1.0
    coefs, errs = [], []
    for _ in range(int(steps)):
        if hi - lo < 1e-4:
            a, b, c = 15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0
            p = lambda x: a * x + b * x ** 3 + c * x ** 5
            E = max(abs(1.0 - p(lo)), abs(1.0 - p(hi)))
        else:
            (a, b, c), E = _remez_odd_quintic(lo, hi)
        coefs.append((a, b, c))
        errs.append(E)
        lo, hi = 1.0 - E, 1.0 + E
    return coefs, errs


def polar_express(X, steps: int, ell: float = 1e-3) -> np.ndarray:
    """Polar(X) by the Polar Express schedule: X / ||X||_F, then X <- X (a I +
    b S + c S^2) for each step; zero for a zero X."""
    X = np.asarray(X, dtype=np.float64)
    f = float(np.sqrt(np.sum(X * X)))
    if f == 0.0:
        return np.zeros_like(X)
    X = X / f
    I = np.eye(X.shape[1])
    for a, b, c in polar_express_coefficients(ell, steps)[0]:
        S = X.T @ X
        X = X @ (a * I + b * S + c * (S @ S))
    return X


def spel_step_polar_express(A, g, m, alpha: float, beta: float, lmo_steps: int = 5, ret_steps: int = 7,
                            ell: float = 1e-3):
    """One SPEL step with the Polar Express polar map: Eq. (4)-(5) as in
    spel_step, Eq. (6) d = PE(m, lmo_steps), Eq. (7) A <- PE(A - alpha d,
    ret_steps) (both inputs scaled by their Frobenius norms).  Returns
    (A_new, m_new, d, g_R)."""
    gR = tangent_project(A, g)
    m_new = momentum(m, gR, beta)
    D = polar_express(m_new, lmo_steps, ell)
    A_new = polar_express(np.asarray(A, dtype=np.float64) - alpha * D, ret_steps, ell)
    return A_new, m_new, D, gR
