"""Pins of the fp64 oracle against things other than itself.

Each check ties an oracle function to brute-force loops, a closed form (via
the SVD), a library routine for a special case, an invariant the MAPL paper
states, or a number the paper prints (tests/golden).  A plausible slip in the
oracle -- a dropped term, a wrong sign, a transposed operand, a wrong
coefficient -- fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.cluster.vq

import synth
from oracle import codec, rvq, spel


# ----------------------------------------------------------------- helpers --

def micro_codec(seed=0, N=7, d=8, r=3, V=5, ra=None):
    """A tiny boundary; the anchor rank ra defaults to r (Eq. (3))."""
    ra = r if ra is None else ra
    rng = np.random.default_rng(seed)
    A = synth.orthonormal_columns(rng, d, r)
    P = synth.orthonormal_rows(rng, ra, d)
    E = rng.standard_normal((V, ra)) * 0.3
    tids = rng.integers(0, V, size=N).astype(np.int32)
    X = rng.standard_normal((N, d))
    G = rng.standard_normal((N, d))
    gZ = rng.standard_normal((N, r))
    return dict(A=A, P=P, E=E, tids=tids, X=X, G=G, gZ=gZ, N=N, d=d, r=r, V=V, ra=ra)


def loop_anchor(n, i, m):
    return sum(m["E"][m["tids"][n]][k] * m["P"][k][i] for k in range(m["ra"]))


# anchor ranks of the pins: Eq. (3)'s ra = r, and Appendix G's anchor rank as a
# separate choice below and above r
RA_CASES = [None, 2, 5]


def loop_compress(m, X=None):
    X = m["X"] if X is None else X
    N, d, r = m["N"], m["d"], m["r"]
    Z = np.zeros((N, r))
    for n in range(N):
        for j in range(r):
            Z[n, j] = sum((X[n][i] - loop_anchor(n, i, m)) * m["A"][i][j] for i in range(d))
    return Z


def loop_reconstruct(m, Z):
    N, d, r = m["N"], m["d"], m["r"]
    Xh = np.zeros((N, d))
    for n in range(N):
        for i in range(d):
            Xh[n, i] = sum(Z[n][j] * m["A"][i][j] for j in range(r)) + loop_anchor(n, i, m)
    return Xh


# ------------------------------------------------------------ codec pins --

@pytest.mark.parametrize("ra", RA_CASES)
def test_codec_forward_matches_brute_force_loops(ra):
    m = micro_codec(1, ra=ra)
    Z = codec.compress(m["X"], m["tids"], m["E"], m["P"], m["A"])
    np.testing.assert_allclose(Z, loop_compress(m), rtol=0, atol=1e-12)
    Xh = codec.reconstruct(Z, m["tids"], m["E"], m["P"], m["A"])
    np.testing.assert_allclose(Xh, loop_reconstruct(m, Z), rtol=0, atol=1e-12)


@pytest.mark.parametrize("ra", RA_CASES)
def test_codec_backward_matches_brute_force_loops(ra):
    m = micro_codec(2, ra=ra)
    N, d, r = m["N"], m["d"], m["r"]
    Z = codec.compress(m["X"], m["tids"], m["E"], m["P"], m["A"])
    gZ, gA_rec = codec.reconstruct_bwd(m["G"], Z, m["A"])
    gX, gA_cmp = codec.compress_bwd(m["gZ"], m["X"], m["tids"], m["E"], m["P"], m["A"])
    for n in range(N):
        for j in range(r):
            assert abs(gZ[n, j] - sum(m["G"][n][i] * m["A"][i][j] for i in range(d))) < 1e-12
        for i in range(d):
            assert abs(gX[n, i] - sum(m["gZ"][n][j] * m["A"][i][j] for j in range(r))) < 1e-12
    for i in range(d):
        for j in range(r):
            ref_rec = sum(m["G"][n][i] * Z[n][j] for n in range(N))
            ref_cmp = sum((m["X"][n][i] - loop_anchor(n, i, m)) * m["gZ"][n][j] for n in range(N))
            assert abs(gA_rec[i, j] - ref_rec) < 1e-12
            assert abs(gA_cmp[i, j] - ref_cmp) < 1e-12


def _central_diff(f, x, h=1e-3):
    g = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


def test_backward_equals_finite_differences_of_forward():
    """Both maps are linear in X, Z and A, so central differences are exact up
    to fp64 rounding; they pin every backward output to the forward maps."""
    m = micro_codec(3)
    Z0 = codec.compress(m["X"], m["tids"], m["E"], m["P"], m["A"])
    L_rec_A = lambda A: float(np.sum(m["G"] * codec.reconstruct(Z0, m["tids"], m["E"], m["P"], A)))
    L_rec_Z = lambda Z: float(np.sum(m["G"] * codec.reconstruct(Z, m["tids"], m["E"], m["P"], m["A"])))
    L_cmp_A = lambda A: float(np.sum(m["gZ"] * codec.compress(m["X"], m["tids"], m["E"], m["P"], A)))
    L_cmp_X = lambda X: float(np.sum(m["gZ"] * codec.compress(X, m["tids"], m["E"], m["P"], m["A"])))
    gZ, gA_rec = codec.reconstruct_bwd(m["G"], Z0, m["A"])
    gX, gA_cmp = codec.compress_bwd(m["gZ"], m["X"], m["tids"], m["E"], m["P"], m["A"])
    np.testing.assert_allclose(gA_rec, _central_diff(L_rec_A, m["A"]), atol=1e-9)
    np.testing.assert_allclose(gZ, _central_diff(L_rec_Z, Z0), atol=1e-9)
    np.testing.assert_allclose(gA_cmp, _central_diff(L_cmp_A, m["A"]), atol=1e-9)
    np.testing.assert_allclose(gX, _central_diff(L_cmp_X, m["X"]), atol=1e-9)


@pytest.mark.parametrize("ra", RA_CASES)
def test_anchor_grad_equals_finite_differences(ra):
    m = micro_codec(4, ra=ra)
    def L(E):
        Z = codec.compress(m["X"], m["tids"], E, m["P"], m["A"])
        return float(np.sum(m["gZ"] * Z))
    gE = codec.anchor_grad(m["gZ"], m["tids"], m["P"], m["A"], m["V"])
    np.testing.assert_allclose(gE, _central_diff(L, m["E"]), atol=1e-9)
    def L2(E):
        return float(np.sum(m["G"] * codec.reconstruct(np.zeros((m["N"], m["r"])), m["tids"], E, m["P"], m["A"])))
    gE2 = codec.anchor_grad(np.zeros((m["N"], m["r"])), m["tids"], m["P"], m["A"], m["V"],
                            gXhat=m["G"], P_recv=m["P"])
    np.testing.assert_allclose(gE2, _central_diff(L2, m["E"]), atol=1e-9)


@pytest.mark.parametrize("ra", RA_CASES)
def test_anchor_grad_adjoint_identity_and_loops(ra):
    """Eq. (1) and (2) are affine in E_small, so for any table perturbation dE
    the pairing <gE, dE> equals the change of <gZ, Z> (sender) and of
    <gXhat, Xhat> (receiver) exactly; and the scatter is checked against
    explicit per-token loops, with repeated ids."""
    m = micro_codec(6, N=9, V=4, ra=ra)
    rng = np.random.default_rng(60)
    dE = rng.standard_normal(m["E"].shape)
    gE = codec.anchor_grad(m["gZ"], m["tids"], m["P"], m["A"], m["V"])
    dZ = (codec.compress(m["X"], m["tids"], m["E"] + dE, m["P"], m["A"])
          - codec.compress(m["X"], m["tids"], m["E"], m["P"], m["A"]))
    assert abs(np.sum(gE * dE) - np.sum(m["gZ"] * dZ)) < 1e-12 * (1 + abs(np.sum(gE * dE)))
    Zr = rng.standard_normal((m["N"], m["r"]))
    gE2 = codec.anchor_grad(np.zeros((m["N"], m["r"])), m["tids"], m["P"], m["A"], m["V"], gXhat=m["G"],
                            P_recv=m["P"])
    dXh = (codec.reconstruct(Zr, m["tids"], m["E"] + dE, m["P"], m["A"])
           - codec.reconstruct(Zr, m["tids"], m["E"], m["P"], m["A"]))
    assert abs(np.sum(gE2 * dE) - np.sum(m["G"] * dXh)) < 1e-12 * (1 + abs(np.sum(gE2 * dE)))
    # loops: row v collects -gZ[n] (P A)^T over the tokens with id v, plus G[n] P^T
    both = codec.anchor_grad(m["gZ"], m["tids"], m["P"], m["A"], m["V"], gXhat=m["G"], P_recv=m["P"])
    want = np.zeros((m["V"], m["ra"]))
    for n in range(m["N"]):
        v = m["tids"][n]
        for k in range(m["ra"]):
            pa = [sum(m["P"][k][i] * m["A"][i][j] for i in range(m["d"])) for j in range(m["r"])]
            want[v][k] -= sum(m["gZ"][n][j] * pa[j] for j in range(m["r"]))
            want[v][k] += sum(m["G"][n][i] * m["P"][k][i] for i in range(m["d"]))
    assert len(set(m["tids"].tolist())) < m["N"]  # some id repeats
    np.testing.assert_allclose(both, want, atol=1e-12)


def test_no_anchor_is_the_plain_projection():
    """Table 6's "no anchor" row: without E_small and P the maps are Z = X A
    and Xhat = Z A^T (checked by loops), the same as with an all-zero table,
    and the backward's gA is X^T gZ."""
    m = micro_codec(7)
    N, d, r = m["N"], m["d"], m["r"]
    Z = codec.compress(m["X"], None, None, None, m["A"])
    for n in range(N):
        for j in range(r):
            assert abs(Z[n, j] - sum(m["X"][n][i] * m["A"][i][j] for i in range(d))) < 1e-12
    zero = np.zeros_like(m["E"])
    np.testing.assert_array_equal(Z, codec.compress(m["X"], m["tids"], zero, m["P"], m["A"]))
    Xh = codec.reconstruct(Z, None, None, None, m["A"])
    for n in range(N):
        for i in range(d):
            assert abs(Xh[n, i] - sum(Z[n][j] * m["A"][i][j] for j in range(r))) < 1e-12
    gX, gA = codec.compress_bwd(m["gZ"], m["X"], None, None, None, m["A"])
    for i in range(d):
        for j in range(r):
            assert abs(gA[i, j] - sum(m["X"][n][i] * m["gZ"][n][j] for n in range(N))) < 1e-12
    np.testing.assert_allclose(gX, m["gZ"] @ m["A"].T, atol=1e-12)


def test_full_anchor_is_a_row_gather():
    """Table 6's fully trainable anchor: E in R^{V x d} with P = I.  The
    anchor is then the gathered row E[t] itself, Eq. (1) subtracts it before
    the projection, and its table gradient scatters -gZ A^T (sender) and gXhat
    (receiver) rows by id -- each checked by explicit loops."""
    m = micro_codec(8, N=9, V=4)
    N, d, r, V = m["N"], m["d"], m["r"], m["V"]
    rng = np.random.default_rng(80)
    E = rng.standard_normal((V, d))
    I = np.eye(d)
    t = m["tids"]
    np.testing.assert_array_equal(codec.anchor(t, E, I), E[t])
    Z = codec.compress(m["X"], t, E, I, m["A"])
    for n in range(N):
        for j in range(r):
            want = sum((m["X"][n][i] - E[t[n]][i]) * m["A"][i][j] for i in range(d))
            assert abs(Z[n, j] - want) < 1e-12
    Xh = codec.reconstruct(Z, t, E, I, m["A"])
    for n in range(N):
        for i in range(d):
            assert abs(Xh[n, i] - (sum(Z[n][j] * m["A"][i][j] for j in range(r)) + E[t[n]][i])) < 1e-12
    gE = codec.anchor_grad(m["gZ"], t, I, m["A"], V, gXhat=m["G"], P_recv=I)
    want = np.zeros((V, d))
    for n in range(N):
        for i in range(d):
            want[t[n]][i] += m["G"][n][i] - sum(m["gZ"][n][j] * m["A"][i][j] for j in range(r))
    np.testing.assert_allclose(gE, want, atol=1e-12)


def test_stiefel_projector_inputs_and_idempotence():
    """A^T A = I (Section 3.2) for the generated projector; Z A^T A = Z."""
    inp = synth.codec_inputs(1, 64, 256, 32, 1000, "f32")
    A, P = inp["A64"], inp["P64"]
    assert np.abs(A.T @ A - np.eye(32)).max() < 1e-13
    assert np.abs(P @ P.T - np.eye(32)).max() < 1e-13
    X = inp["X"].double().numpy()
    Z = codec.compress(X, inp["tids"].numpy(), inp["E"].double().numpy(), P, A)
    np.testing.assert_allclose(Z @ A.T @ A, Z, atol=1e-12)


def test_exact_round_trip_when_residual_in_span():
    """Section 3.2: A^T inverts A on its column space, so with equal anchors a
    residual inside span(A) round-trips exactly."""
    rng = np.random.default_rng(5)
    inp = synth.codec_inputs(1, 128, 256, 32, 1000, "f32")
    A, P = inp["A64"], inp["P64"]
    E = inp["E"].double().numpy()
    t = inp["tids"].numpy()
    W = rng.standard_normal((128, 32))
    X = codec.anchor(t, E, P) + W @ A.T
    Z = codec.compress(X, t, E, P, A)
    np.testing.assert_allclose(Z, W, atol=1e-12)
    np.testing.assert_allclose(codec.reconstruct(Z, t, E, P, A), X, atol=1e-12)


def _golden_rows(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "payload_bytes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            rows.append(dict(kind=p[0], d=int(p[1]), r=None if p[2] == "-" else int(p[2]),
                             G=None if p[3] == "-" else int(p[3]),
                             R=None if p[4] == "-" else int(p[4]),
                             K=None if p[5] == "-" else int(p[5]),
                             bytes=int(p[6]), ratio=int(p[7])))
    return rows


def test_payload_sizes_match_paper(golden_dir):
    rows = _golden_rows(golden_dir)
    assert len(rows) == 12
    for row in rows:
        base = codec.bytes_per_token(row["d"])
        if row["kind"] == "uncompressed":
            got = base
        elif row["kind"] == "mapl":
            got = codec.bytes_per_token(row["r"])
            assert codec.compression_ratio(row["d"], row["r"]) == row["r"] / row["d"]
        else:
            got = rvq.bytes_per_token(row["G"], row["R"], row["K"])
        assert got == row["bytes"], row
        assert base / got == row["ratio"], row


# ------------------------------------------------------------- spel pins --

def _ns_closed_form(M, iters):
    """NS applied to the singular values: U f^k(S) V^T, f(s) = 1.5 s - 0.5 s^3."""
    U, S, Vt = np.linalg.svd(M, full_matrices=False)
    s = S.copy()
    for _ in range(iters):
        s = 1.5 * s - 0.5 * s ** 3
    return (U * s) @ Vt


@pytest.mark.parametrize("shape,smin,smax", [((40, 6), 0.05, 0.9), ((64, 16), 0.3, 1.3),
                                             ((2048, 256), 0.01, 0.1)])
def test_newton_schulz_equals_singular_value_closed_form(shape, smin, smax):
    rng = np.random.default_rng(6)
    d, r = shape
    U = synth.orthonormal_columns(rng, d, r)
    V = synth.orthonormal_columns(rng, r, r)
    s = np.linspace(smin, smax, r)
    M = (U * s) @ V.T
    for iters in (1, 3, 8):
        np.testing.assert_allclose(spel.newton_schulz(M, iters), _ns_closed_form(M, iters), atol=1e-12)


def test_newton_schulz_converges_to_svd_polar_and_fixes_stiefel():
    rng = np.random.default_rng(7)
    U = synth.orthonormal_columns(rng, 48, 8)
    V = synth.orthonormal_columns(rng, 8, 8)
    M = (U * np.linspace(0.3, 1.3, 8)) @ V.T
    np.testing.assert_allclose(spel.newton_schulz(M, 8), U @ V.T, atol=1e-12)
    Q = synth.orthonormal_columns(rng, 48, 8)
    np.testing.assert_allclose(spel.newton_schulz(Q, 8), Q, atol=1e-14)


def test_tangent_projection_properties():
    rng = np.random.default_rng(8)
    A = synth.orthonormal_columns(rng, 50, 7)
    g = rng.standard_normal((50, 7))
    gR = spel.tangent_project(A, g)
    # lies in the tangent space: sym(A^T gR) = 0
    assert np.abs(spel.sym(A.T @ gR)).max() < 1e-14
    # idempotent
    np.testing.assert_allclose(spel.tangent_project(A, gR), gR, atol=1e-14)
    # removes exactly the normal component: normal vectors A S (S symmetric) vanish
    S = rng.standard_normal((7, 7)); S = S + S.T
    assert np.abs(spel.tangent_project(A, A @ S)).max() < 1e-13
    # orthogonal projection: g - gR is orthogonal to every tangent vector
    D = spel.tangent_project(A, rng.standard_normal((50, 7)))
    assert abs(np.sum((g - gR) * D)) < 1e-12
    # skew part and the orthogonal-complement part pass through unchanged
    K = rng.standard_normal((7, 7)); K = K - K.T
    Y = rng.standard_normal((50, 7)); Y = Y - A @ (A.T @ Y)
    np.testing.assert_allclose(spel.tangent_project(A, A @ K + Y), A @ K + Y, atol=1e-13)


def _loop_spel(A, g, m, alpha, beta, iters):
    d, r = A.shape
    def mm(X, Y):
        return [[sum(X[i][k] * Y[k][j] for k in range(len(Y))) for j in range(len(Y[0]))]
                for i in range(len(X))]
    def T(X):
        return [list(c) for c in zip(*X)]
    A = A.tolist(); g = g.tolist(); m = m.tolist()
    S = mm(T(A), g)
    gR = [[g[i][j] - sum(A[i][k] * 0.5 * (S[k][j] + S[j][k]) for k in range(r)) for j in range(r)]
          for i in range(d)]
    m = [[beta * m[i][j] + (1 - beta) * gR[i][j] for j in range(r)] for i in range(d)]
    f = math.sqrt(sum(v * v for row in m for v in row))
    def ns(X):
        for _ in range(iters):
            Gm = mm(T(X), X)
            XG = mm(X, Gm)
            X = [[1.5 * X[i][j] - 0.5 * XG[i][j] for j in range(r)] for i in range(d)]
        return X
    D = ns([[v / f for v in row] for row in m])
    An = ns([[A[i][j] - alpha * D[i][j] for j in range(r)] for i in range(d)])
    return np.array(An), np.array(m), np.array(D)


def test_spel_step_matches_brute_force_loops():
    rng = np.random.default_rng(9)
    A = synth.orthonormal_columns(rng, 6, 2)
    g = rng.standard_normal((6, 2))
    m0 = rng.standard_normal((6, 2)) * 0.1
    An, mn, D, _ = spel.spel_step(A, g, m0, 0.05, 0.9, 8)
    An2, mn2, D2 = _loop_spel(A, g, m0, 0.05, 0.9, 8)
    np.testing.assert_allclose(mn, mn2, atol=1e-14)
    np.testing.assert_allclose(D, D2, atol=1e-13)
    np.testing.assert_allclose(An, An2, atol=1e-13)


def test_spel_step_at_1b_shape_stays_on_stiefel_and_matches_svd_polar():
    inp = synth.spel_inputs(5, 2048, 256)
    A = inp["A"].double().numpy()
    g = inp["g"].double().numpy()
    An, mn, D, gR = spel.spel_step(A, g, np.zeros_like(A), 1e-3, 0.9, 8)
    np.testing.assert_allclose(mn, 0.1 * gR, atol=1e-18)
    assert np.abs(An.T @ An - np.eye(256)).max() < 1e-12
    # the retraction equals the SVD polar factor of A - alpha d
    U, _, Vt = np.linalg.svd(A - 1e-3 * D, full_matrices=False)
    np.testing.assert_allclose(An, U @ Vt, atol=1e-13)
    # the LMO direction is the singular-value closed form of NS8(m/||m||_F)
    np.testing.assert_allclose(D, _ns_closed_form(mn / np.linalg.norm(mn), 8), atol=1e-12)


# ------------------------------------------------------ Polar Express pins --

def _pe_interval_grid(lo, hi, n=400001):
    return np.linspace(lo, hi, n)


def test_polar_express_polynomials_are_minimax():
    """Chebyshev's alternation theorem: p_t is the best uniform approximation
    of 1 on [l_t, u_t] by odd quintics (a 3-dimensional Haar space) exactly
    when 1 - p_t reaches its maximum E_t with alternating signs at 4 points;
    and the next interval is p_t's range, [1 - E_t, 1 + E_t]."""
    coefs, errs = spel.polar_express_coefficients(1e-3, 7)
    lo, hi = 1e-3, 1.0
    for (a, b, c), E in zip(coefs, errs):
        if hi - lo < 1e-4:
            break
        x = _pe_interval_grid(lo, hi)
        e = 1.0 - (a * x + b * x ** 3 + c * x ** 5)
        assert np.max(np.abs(e)) <= E * (1 + 1e-8) + 1e-15
        # alternation: scan the sign pattern of the near-extremal points
        peaks = np.where(np.abs(e) >= E * (1 - 1e-6))[0]
        signs = [np.sign(e[peaks[0]])]
        for i in peaks[1:]:
            if np.sign(e[i]) != signs[-1]:
                signs.append(np.sign(e[i]))
        assert len(signs) >= 4, (lo, hi, signs)
        p = 1.0 - e
        assert abs(p.min() - (1 - E)) <= 1e-9 * max(E, 1e-12) + 1e-14
        assert abs(p.max() - (1 + E)) <= 1e-9 * max(E, 1e-12) + 1e-14
        lo, hi = 1.0 - E, 1.0 + E


def test_polar_express_narrow_interval_tends_to_the_limit_quintic():
    """As the interval shrinks to {1}, the minimax quintic tends to the one
    with p(1) = 1, p'(1) = p''(1) = 0: (15 x - 10 x^3 + 3 x^5) / 8."""
    (a, b, c), E = spel._remez_odd_quintic(1 - 1e-4, 1 + 1e-4)
    np.testing.assert_allclose([a, b, c], [15 / 8, -10 / 8, 3 / 8], atol=1e-6)
    assert E < 1e-10


def test_polar_express_matches_the_singular_value_closed_form():
    """For X = U diag(s) V^T the schedule acts on singular values only:
    PE(X) = U diag(phi(s / ||X||_F)) V^T, phi the composition of the scalar
    quintics; and after 7 steps from ell = 1e-3 it is the SVD polar factor
    U V^T to within the last error bound."""
    rng = np.random.default_rng(71)
    U, _ = np.linalg.qr(rng.standard_normal((48, 12)))
    V, _ = np.linalg.qr(rng.standard_normal((12, 12)))
    s = np.geomspace(1.0, 2e-3, 12) * 3.0
    X = U @ np.diag(s) @ V.T
    coefs, errs = spel.polar_express_coefficients(1e-3, 7)
    y = s / np.sqrt(np.sum(s * s))
    for a, b, c in coefs:
        y = a * y + b * y ** 3 + c * y ** 5
    np.testing.assert_allclose(spel.polar_express(X, 7), U @ np.diag(y) @ V.T, atol=1e-12)
    np.testing.assert_allclose(spel.polar_express(X, 7), U @ V.T, atol=2 * errs[-1] + 1e-12)
    assert np.all(np.abs(y - 1) <= errs[-1] * (1 + 1e-6))
    # five steps (the LMO's) leave every singular value within E_5 of 1
    y5 = s / np.sqrt(np.sum(s * s))
    for a, b, c in coefs[:5]:
        y5 = a * y5 + b * y5 ** 3 + c * y5 ** 5
    assert np.all(np.abs(y5 - 1) <= errs[4] * (1 + 1e-9))


def test_polar_express_step_shares_the_tangent_and_momentum_steps():
    inp = synth.spel_inputs(72, 96, 16, 1e-3)
    A, g, m = (inp[k].double().numpy() for k in ("A", "g", "m"))
    A1, m1, D1, gR1 = spel.spel_step(A, g, m, 0.05, 0.9, 8)
    A2, m2, D2, gR2 = spel.spel_step_polar_express(A, g, m, 0.05, 0.9, 5, 7)
    np.testing.assert_array_equal(m1, m2)
    np.testing.assert_array_equal(gR1, gR2)
    np.testing.assert_allclose(A2.T @ A2, np.eye(16), atol=1e-8)
    z = spel.polar_express(np.zeros((8, 4)), 5)
    assert not np.any(z)


def test_spel_degenerate_cases():
    rng = np.random.default_rng(10)
    A = synth.orthonormal_columns(rng, 30, 4)
    S = rng.standard_normal((4, 4)); S = S + S.T
    # a purely normal gradient projects to rounding noise only
    _, _, _, gR = spel.spel_step(A, A @ S, np.zeros((30, 4)), 0.1, 0.9, 8)
    assert np.abs(gR).max() < 1e-13
    # a zero gradient with zero momentum: no direction, and A (already on the
    # manifold) is a fixed point of the retraction
    An, mn, D, gR = spel.spel_step(A, np.zeros((30, 4)), np.zeros((30, 4)), 0.1, 0.9, 8)
    assert np.all(mn == 0) and np.all(D == 0)
    np.testing.assert_allclose(An, A, atol=1e-14)
    # LMO is invariant to the momentum's scale
    m = rng.standard_normal((30, 4))
    np.testing.assert_allclose(spel.lmo_direction(m, 8), spel.lmo_direction(7.5 * m, 8), atol=1e-14)
    assert np.all(spel.lmo_direction(np.zeros((30, 4)), 8) == 0)


# -------------------------------------------------------------- rvq pins --

def _loop_rvq(Z, C, G, K, R):
    N, r = Z.shape
    w = r // G
    res = [list(map(float, row)) for row in Z]
    codes = np.zeros((N, R, G), dtype=np.int64)
    for rho in range(R):
        book = C[rho if C.shape[0] > 1 else 0]
        for n in range(N):
            for g in range(G):
                best, bk = None, -1
                for k in range(K):
                    dist = sum((res[n][g * w + j] - book[g][k][j]) ** 2 for j in range(w))
                    if best is None or dist < best:   # strict: keeps the lowest index on ties
                        best, bk = dist, k
                codes[n, rho, g] = bk
                for j in range(w):
                    res[n][g * w + j] -= book[g][bk][j]
    return codes, np.array(res)


@pytest.mark.parametrize("R_c", [1, 3])
def test_rvq_matches_brute_force_loops(R_c):
    rng = np.random.default_rng(11)
    N, r, G, K, R = 7, 4, 2, 4, 3
    C = rng.standard_normal((R_c, G, K, r // G))
    Z = rng.standard_normal((N, r))
    out = rvq.encode(Z, C, G, K, R)
    codes, res = _loop_rvq(Z, C, G, K, R)
    np.testing.assert_array_equal(out["codes"], codes)
    np.testing.assert_allclose(out["residual"], res, atol=1e-13)
    np.testing.assert_allclose(rvq.decode(codes, C, G, K, R) + res, Z, atol=1e-13)


def _loop_dists(res_rows, book_g):
    """Squared distances of each residual row to each codeword, by explicit loops."""
    out = np.zeros((len(res_rows), len(book_g)))
    for n, x in enumerate(res_rows):
        for k, c in enumerate(book_g):
            out[n, k] = sum((float(x[j]) - float(c[j])) ** 2 for j in range(len(c)))
    return out


@pytest.mark.parametrize("R_c", [1, 3])
def test_rvq_teacher_forcing_follows_the_teacher_and_reports_exact_distances(R_c):
    """With teacher codes, each round's residual is Z minus the TEACHER's
    codewords of the earlier rounds (not the oracle's own), d_teacher is the
    teacher codeword's distance, and codes / d1 / d2 are the argmin and the two
    smallest distances on that residual -- all checked by explicit loops.  The
    teacher picks the second-nearest codeword in round 0, so its residual
    differs from the oracle's own."""
    rng = np.random.default_rng(31)
    N, G, K, w, R = 9, 3, 6, 2, 3
    C = rng.standard_normal((R_c, G, K, w))
    Z = rng.standard_normal((N, G * w))
    own = rvq.encode(Z, C, G, K, R)
    teacher = own["codes"].copy()
    for n in range(N):
        for g in range(G):
            dd = _loop_dists([Z[n, g * w:(g + 1) * w]], C[0, g])[0]
            teacher[n, 0, g] = int(np.argsort(dd, kind="stable")[1])   # second nearest
    teacher[:, 1:, :] = rng.integers(0, K, size=(N, R - 1, G))
    out = rvq.encode(Z, C, G, K, R, teacher=teacher)
    res = Z.copy()
    for rho in range(R):
        book = C[rho if R_c > 1 else 0]
        for g in range(G):
            sl = slice(g * w, (g + 1) * w)
            D = _loop_dists(res[:, sl], book[g])
            srt = np.sort(D, axis=1)
            np.testing.assert_array_equal(out["codes"][:, rho, g], np.argmin(D, axis=1))
            np.testing.assert_allclose(out["d1"][:, rho, g], srt[:, 0], rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(out["d2"][:, rho, g], srt[:, 1], rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(out["d_teacher"][:, rho, g], D[np.arange(N), teacher[:, rho, g]],
                                       rtol=1e-12, atol=1e-15)
            res[:, sl] = res[:, sl] - book[g][teacher[:, rho, g]]
    # the final residual is Z minus the teacher's codewords, exactly as decode forms them
    np.testing.assert_allclose(out["residual"], res, atol=1e-13)
    np.testing.assert_allclose(rvq.decode(teacher, C, G, K, R) + out["residual"], Z, atol=1e-13)
    # round 0 is judged on Z itself: the teacher's second-nearest pick is never the argmin
    assert np.all(out["d_teacher"][:, 0, :] >= out["d1"][:, 0, :])
    assert np.all(out["d_teacher"][:, 0, :] == out["d2"][:, 0, :])


def test_rvq_teacher_equal_to_own_codes_changes_nothing():
    rng = np.random.default_rng(32)
    N, G, K, w, R = 40, 4, 16, 4, 2
    C = rng.standard_normal((R, G, K, w))
    Z = rng.standard_normal((N, G * w))
    own = rvq.encode(Z, C, G, K, R)
    tf = rvq.encode(Z, C, G, K, R, teacher=own["codes"])
    for key in ("codes", "d1", "d2", "residual", "energy"):
        np.testing.assert_array_equal(tf[key], own[key])
    np.testing.assert_array_equal(tf["d_teacher"], own["d1"])


def test_rvq_single_codeword_and_odd_codebook_sizes():
    """K = 1 gives code 0 and d2 = inf; for K not a multiple of anything the
    argmin still matches explicit loops (the kernels pad K)."""
    rng = np.random.default_rng(33)
    N, G, w = 11, 2, 4
    Z = rng.standard_normal((N, G * w))
    one = rvq.encode(Z, rng.standard_normal((1, G, 1, w)), G, 1, 2)
    assert np.all(one["codes"] == 0) and np.all(np.isinf(one["d2"]))
    for K in (5, 33):
        C = rng.standard_normal((1, G, K, w))
        out = rvq.encode(Z, C, G, K, 1)
        for g in range(G):
            D = _loop_dists(Z[:, g * w:(g + 1) * w], C[0, g])
            np.testing.assert_array_equal(out["codes"][:, 0, g], np.argmin(D, axis=1))


def test_rvq_codeword_inputs_come_back_with_zero_residual():
    rng = np.random.default_rng(12)
    N, G, K, w = 50, 4, 16, 8
    C = rng.standard_normal((1, G, K, w))
    k_true = rng.integers(0, K, size=(N, G))
    Z = np.concatenate([C[0, g][k_true[:, g]] for g in range(G)], axis=1)
    out = rvq.encode(Z, C, G, K, 1)
    np.testing.assert_array_equal(out["codes"][:, 0, :], k_true)
    assert np.all(out["residual"] == 0.0)


def test_rvq_duplicate_codewords_pick_lowest_index():
    rng = np.random.default_rng(13)
    G, K, w = 1, 8, 4
    C = rng.standard_normal((1, G, K, w))
    C[0, 0, 6] = C[0, 0, 2]
    Z = C[0, 0, 2][None, :] + 1e-3 * rng.standard_normal((5, w))
    out = rvq.encode(Z, C, G, K, 1)
    assert np.all(out["codes"][:, 0, 0] == 2)


def test_rvq_single_round_single_group_is_textbook_vq():
    rng = np.random.default_rng(14)
    obs = rng.standard_normal((300, 6))
    book = rng.standard_normal((20, 6))
    ref, dist = scipy.cluster.vq.vq(obs, book)
    out = rvq.encode(obs, book[None, None], 1, 20, 1)
    np.testing.assert_array_equal(out["codes"][:, 0, 0], ref)
    np.testing.assert_allclose(np.sqrt(out["d1"][:, 0, 0]), dist, rtol=1e-12)


def test_rvq_energy_and_decode_identity_at_config_like_shape():
    rng = np.random.default_rng(15)
    N, r, G, K, R = 512, 256, 8, 256, 2
    Z = rng.standard_normal((N, r))
    for R_c in (1, 2):
        C = rng.standard_normal((R_c, G, K, r // G)) / math.sqrt(32)
        out = rvq.encode(Z, C, G, K, R)
        e = out["energy"]
        assert all(e[i + 1] <= e[i] for i in range(R))
        assert np.all(out["grew"] == 0)
        np.testing.assert_allclose(rvq.decode(out["codes"], C, G, K, R) + out["residual"], Z, atol=1e-12)
        assert np.all(out["d1"] <= out["d2"])


def test_stream_apply_overwrites_exactly_the_streamed_codewords():
    C = synth.rvq_codebooks(4, 2, 8, 256, 32).numpy()
    sender = C + np.float32(1e-2) * np.random.default_rng(16).standard_normal(C.shape).astype(np.float32)
    idx = np.array([3, 700, 4095], dtype=np.int64)
    vals = sender.reshape(-1, 32)[idx]
    out = rvq.stream_apply(C, idx, vals)
    flat_o, flat_c, flat_s = out.reshape(-1, 32), C.reshape(-1, 32), sender.reshape(-1, 32)
    assert np.array_equal(flat_o[idx], flat_s[idx])
    keep = np.setdiff1d(np.arange(flat_c.shape[0]), idx)
    assert np.array_equal(flat_o[keep], flat_c[keep])
    full = rvq.stream_apply(C, np.arange(flat_c.shape[0]), flat_s)
    assert np.array_equal(full, sender)


# -------------------------------------------------- input recipe checks --

def test_lowrank_generator_keeps_99_percent_in_rank_250():
    """Section 3.1, Figure 3: rank ~250 keeps >= 99 % of the boundary energy."""
    rng = synth.stream(3, 4)
    X = synth.low_rank_plus_noise(rng, 2048, 1024)
    s = np.linalg.svd(X, compute_uv=False)
    energy = np.cumsum(s ** 2) / np.sum(s ** 2)
    assert energy[249] >= 0.99
    assert energy[200] < 0.99


def test_generators_are_seeded_and_in_range():
    a = synth.codec_inputs(2, 256, 1024, 128, 32000, "bf16")
    b = synth.codec_inputs(2, 256, 1024, 128, 32000, "bf16")
    assert all(torch_equal(a[k], b[k]) for k in ("X", "E", "P", "A", "gXhat", "tids"))
    t = a["tids"].numpy()
    assert t.min() >= 0 and t.max() < 32000
    assert np.bincount(t).argmax() == 0   # Zipf: id 0 is the most frequent


def torch_equal(x, y):
    return bool((x.view(-1) == y.view(-1)).all()) if x.dtype.is_floating_point else bool((x == y).all())
