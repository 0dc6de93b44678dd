"""The algebra behind the r x r (Gram-space) form of the cubic Newton-Schulz
polar map that spel_step uses for r <= 256: with S_k = X_k^T X_k,
T_k = 1.5 I - 0.5 S_k,
    X_k = X_0 Q_k,  Q_{k+1} = Q_k T_k,  S_{k+1} = 2.25 S_k - 1.5 S_k^2 + 0.25 S_k^3,
so n steps of X <- X (1.5 I - 0.5 X^T X) equal X_0 Q_n.  Checked here in fp64
against the oracle's d x r iteration (Section 3.3, Eq. (6)-(7)), for well- and
ill-conditioned inputs, so that the GPU path's fp32 parity (tests/test_gpu_spel.py)
rests on an identity rather than on a coincidence of rounding."""
import numpy as np
import pytest

from oracle import spel


def gram_space_ns(X, n):
    S = X.T @ X
    r = S.shape[0]
    Q = np.eye(r)
    for _ in range(n):
        Q = 1.5 * Q - 0.5 * Q @ S
        S2 = S @ S
        S = 2.25 * S - 1.5 * S2 + 0.25 * S2 @ S
    return X @ Q


@pytest.mark.parametrize("d,r,n,cond", [(256, 32, 8, 10.0), (1024, 128, 8, 1e3), (96, 96, 5, 1e2),
                                        (512, 64, 1, 1e4), (300, 40, 13, 1.0)])
def test_gram_space_iteration_equals_newton_schulz(d, r, n, cond):
    rng = np.random.default_rng(d + r + n)
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    V, _ = np.linalg.qr(rng.standard_normal((r, r)))
    s = np.geomspace(1.0, 1.0 / cond, r)
    X = (U * s) @ V.T
    X /= np.linalg.norm(X)  # the LMO's scaling: every singular value <= 1
    ref = spel.newton_schulz(X, n)
    got = gram_space_ns(X, n)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_gram_space_iterates_commute_with_the_gram_matrix():
    # Q_k and S_k are polynomials in S_0: they commute with it and are symmetric
    rng = np.random.default_rng(5)
    X = rng.standard_normal((200, 24))
    X /= np.linalg.norm(X)
    S0 = X.T @ X
    S, Q = S0.copy(), np.eye(24)
    for _ in range(6):
        Q = 1.5 * Q - 0.5 * Q @ S
        S2 = S @ S
        S = 2.25 * S - 1.5 * S2 + 0.25 * S2 @ S
        for M in (Q, S):
            assert np.abs(M @ S0 - S0 @ M).max() <= 1e-12
            assert np.abs(M - M.T).max() <= 1e-12
