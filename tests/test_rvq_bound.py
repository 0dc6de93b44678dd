"""The error bounds behind the VQ encode's candidate filters (rvq_encode),
checked on the CPU.  Both kernels score codeword k approximately, a_k ~ s_k =
||c_k||^2 - 2 <res, c_k> (res kept in fp64), and rescore exactly every k with
a_k <= min_j a_j + 2 delta; that finds the exact argmin (Section 3.5's nearest
codeword) if |a_k - s_k| <= delta.  Each kernel's delta is a proven bound
(derived beside the kernel); the worst case needs every rounding error to
line up with the operands' signs, so on these inputs the emulated error stays
under half of it, and an error above that would point at a mistake in the
emulation or the derivation.

* w >= 16: a_k = nrm_k + <bf16(fp32(-2 res)), bf16(c_k)> (nrm_k the fp32
  ||c_k||^2; bf16 products exact, fp32 sums), delta = 2^-6 (1 + 2^-6) ||res|| max ||c|| + 2^-14 max ||c||^2 + 1e-30.
* w < 16: a_k = fp32 sums starting at nrm_k (the fp32 ||c_k||^2) of the fp32
  products fp32(-2 res_j) c_kj, delta = (2 w + 4) 2^-23 (max ||c||^2 +
  2 ||res|| max ||c||) + 1e-30; a token whose second-smallest score exceeds
  its smallest by more than 2 delta keeps that codeword without rescoring.

The scores are emulated in numpy in two summation orders (the hardware's order
inside a matrix-core instruction is not documented) on random and adversarial
inputs."""
import numpy as np
import pytest
import torch


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def norms_f32(C):
    nrm = np.zeros(C.shape[0], np.float32)
    for j in range(C.shape[1]):
        nrm = np.float32(nrm + C[:, j] * C[:, j])
    return nrm


def emulate_bf16(res, C, reverse=False):
    """bf16 scores a [n][K] as the w >= 16 kernel forms them: the accumulator starts at nrm_k
    (the fp32 ||c_k||^2) and adds the exact bf16 products in fp32 (dims in order or reversed)."""
    nrm = norms_f32(C)
    rb, cb = bf16(f32(-2.0 * res)), bf16(C)
    a = np.broadcast_to(nrm[None, :], (res.shape[0], C.shape[0])).astype(np.float32)
    dims = range(C.shape[1] - 1, -1, -1) if reverse else range(C.shape[1])
    for j in dims:
        a = np.float32(a + np.outer(rb[:, j], cb[:, j]).astype(np.float32))
    return a, nrm


def emulate_f32(res, C, reverse=False):
    """fp32 scores a [n][K] as the w < 16 kernel forms them: the accumulator starts at
    nrm_k and adds each rounded product (dims in order or reversed)."""
    nrm = norms_f32(C)
    b = f32(-2.0 * res)
    a = np.broadcast_to(nrm[None, :], (res.shape[0], C.shape[0])).astype(np.float32)
    dims = range(C.shape[1] - 1, -1, -1) if reverse else range(C.shape[1])
    for j in dims:
        a = np.float32(a + np.float32(np.outer(b[:, j], C[:, j])))
    return a, nrm


def exact_scores(res, C):
    return (C.astype(np.float64) ** 2).sum(1)[None, :] - 2.0 * res @ C.astype(np.float64).T


def delta_bf16(res, nrm):
    rn = np.sqrt(np.float32((res ** 2).sum(1)))
    nmax = np.float32(nrm.max())
    return np.float32(2.0 ** -6 * (1 + 2.0 ** -6)) * rn * np.sqrt(nmax) + np.float32(2.0 ** -14) * nmax + np.float32(1e-30)


def delta_f32(res, nrm, w):
    rn = np.sqrt(np.float32((res ** 2).sum(1)))
    nmax = np.float32(nrm.max())
    return np.float32(2 * w + 4) * np.float32(2.0 ** -23) * (nmax + 2 * rn * np.sqrt(nmax)) + np.float32(1e-30)


def make_case(w, kind, seed):
    rng = np.random.default_rng(seed)
    K, n = 256, 512
    C = rng.normal(0.0, 1.0 / np.sqrt(w), (K, w)).astype(np.float32)
    res = rng.normal(0.0, 1.0, (n, w))
    if kind == "near":        # residuals a hair away from codewords: near-ties and cancellation
        res = C[rng.integers(0, K, n)].astype(np.float64) + rng.normal(0.0, 1e-3, (n, w))
    elif kind == "round1":    # a second-round residual: bf16 z minus an fp32 codeword, exact in fp64
        z = bf16(C[rng.integers(0, K, n)] + rng.normal(0.0, 0.05, (n, w)).astype(np.float32)).astype(np.float64)
        res = z - C[rng.integers(0, K, n)].astype(np.float64)
    elif kind == "scaled_up":
        res *= 1e4
        C *= np.float32(30.0)
    elif kind == "scaled_down":
        res *= 1e-5
        C *= np.float32(1e-3)
    elif kind == "spread_norms":
        C *= np.geomspace(1e-3, 10.0, K, dtype=np.float32)[:, None]
    return res, C


KINDS = ("gauss", "near", "round1", "scaled_up", "scaled_down", "spread_norms")


@pytest.mark.parametrize("w,kind", [(w, k) for w in (16, 32, 64) for k in KINDS])
def test_bf16_scores_stay_within_half_the_kernels_delta(w, kind):
    res, C = make_case(w, kind, w * 7 + len(kind))
    s = exact_scores(res, C)
    for reverse in (False, True):
        a, nrm = emulate_bf16(res, C, reverse)
        delta = delta_bf16(res, nrm).astype(np.float64)
        err = np.abs(a.astype(np.float64) - s)
        assert np.all(err <= 0.5 * delta[:, None]), float((err / delta[:, None]).max())
        kstar = s.argmin(1)
        lim = a.min(1).astype(np.float64) + 2.0 * delta
        assert np.all(a[np.arange(len(res)), kstar] <= lim)   # the exact argmin is a candidate


@pytest.mark.parametrize("w,kind", [(w, k) for w in (2, 4, 8) for k in KINDS])
def test_f32_scores_stay_within_half_the_kernels_delta(w, kind):
    res, C = make_case(w, kind, w * 11 + len(kind))
    s = exact_scores(res, C)
    n = len(res)
    for reverse in (False, True):
        a, nrm = emulate_f32(res, C, reverse)
        delta = delta_f32(res, nrm, w).astype(np.float64)
        err = np.abs(a.astype(np.float64) - s)
        assert np.all(err <= 0.5 * delta[:, None]), float((err / delta[:, None]).max())
        # the one-pass shortcut: a margin of more than 2 delta between the two smallest
        # scores means the smallest score's codeword is the exact argmin
        srt = np.sort(a, axis=1).astype(np.float64)
        sure = srt[:, 1] - srt[:, 0] > 2.0 * delta
        kbest = np.argmin(a, axis=1)
        assert np.all(kbest[sure] == s.argmin(1)[sure])
        kstar = s.argmin(1)
        assert np.all(a[np.arange(n), kstar] <= srt[:, 0] + 2.0 * delta)
