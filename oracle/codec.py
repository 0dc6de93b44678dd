"""MAPL boundary codec, forward and backward, as plain fp64 definitions.

Source: *Learned Subspace Compression for Communication-Efficient Pipeline
Parallelism*, Section 3.2, Eq. (1) (compression), Eq. (2) (reconstruction) and
Eq. (3) (factorised anchor E_small[ids] P with E_small in R^{V x r} and
P in R^{r x d}); Section 3.1 "Setup" (the backward pass transmits the gradient
of the boundary activation) and Section 3.2 (the gradient is routed through
the same projector A).  Tokens are flattened: N = B*T rows.

Anchor variants (Table 6, the anchor-rank ablation of Appendix G, and the
no-anchor "Subspace" rows): the anchor's rank ra may differ from the
projector's rank r (E_small [V][ra], P [ra][d]); the full-rank anchor is the
table E in R^{V x d}, i.e. ra = d with P = I; and "no anchor" is
E_small = P = None, which these functions read as an anchor term of zero.

Test infrastructure only: see the package docstring.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def anchor(tids, E_small, P) -> np.ndarray:
    """Eq. (3): the factorised anchor E_small[tids] @ P, shape [N][d]."""
    return _f64(E_small)[np.asarray(tids, dtype=np.int64)] @ _f64(P)


def _residual(X, tids, E_small, P) -> np.ndarray:
    """X minus the anchor; without an anchor (E_small None) X itself."""
    X = _f64(X)
    return X if E_small is None else X - anchor(tids, E_small, P)


def compress(X, tids, E_small, P, A) -> np.ndarray:
    """Eq. (1): Z = (X - E_small[tids] P) A, shape [N][r]."""
    return _residual(X, tids, E_small, P) @ _f64(A)


def reconstruct(Z, tids, E_small, P, A) -> np.ndarray:
    """Eq. (2): Xhat = Z A^T + E_small[tids] P, shape [N][d].  E_small and P
    are the receiving stage's anchor (E_{p+1}, P_{p+1} in Eq. (2))."""
    Xh = _f64(Z) @ _f64(A).T
    return Xh if E_small is None else Xh + anchor(tids, E_small, P)


def reconstruct_bwd(gXhat, Z, A):
    """Backward of Eq. (2) with respect to Z and A, given G = dL/dXhat:
    gZ = G A  ([N][r]) and gA_rec = G^T Z  ([d][r]).  The anchor term does not
    depend on Z or A."""
    G = _f64(gXhat)
    return G @ _f64(A), G.T @ _f64(Z)


def compress_bwd(gZ, X, tids, E_small, P, A):
    """Backward of Eq. (1) with respect to X and A, given gZ = dL/dZ:
    gX = gZ A^T ([N][d]) and gA_cmp = (X - E_small[tids] P)^T gZ ([d][r])."""
    gZ = _f64(gZ)
    R = _residual(X, tids, E_small, P)
    return gZ @ _f64(A).T, R.T @ gZ


def anchor_grad(gZ, tids, P, A, V, gXhat=None, P_recv=None) -> np.ndarray:
    """Gradient of the loss with respect to the trainable anchor table
    E_small ([V][ra], ra = P's row count), Eq. (3) being trainable.  From
    Eq. (1): d/dE[t] of -(E[t] P) A is -gZ_n (P A)^T, scatter-added to row
    tids[n].  If the receiver's G = dL/dXhat is given, Eq. (2) adds
    G_n P_recv^T to row tids[n] of the receiver's table (returned separately
    by calling this with gZ = 0).  Sum over tokens in token order."""
    tids = np.asarray(tids, dtype=np.int64)
    out = np.zeros((V, _f64(P).shape[0]), dtype=np.float64)
    rows = -(_f64(gZ) @ (_f64(P) @ _f64(A)).T)
    if gXhat is not None:
        rows = rows + _f64(gXhat) @ _f64(P_recv).T
    np.add.at(out, tids, rows)
    return out


def bytes_per_token(width: int, bytes_per_value: int = 2) -> int:
    """Boundary payload per token: one `width`-wide row of values.  The token
    id travels alongside and is excluded, as in the paper's Table 1."""
    return int(width) * int(bytes_per_value)


def compression_ratio(d: int, r: int) -> float:
    """Section 3.2: the codec's exact compression ratio r/d (equal dtypes)."""
    return bytes_per_token(r) / bytes_per_token(d)
