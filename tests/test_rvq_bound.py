"""The error bound behind the bf16-scored VQ encode (rvq_encode, group width
w >= 16), checked on the CPU: the kernel scores codeword k as
    a_k = <bf16(-2 res), bf16(c_k)> + hi_k + lo_k
(bf16 products exact, fp32 sums; hi_k + lo_k the two-part bf16 split of the
fp32 ||c_k||^2) and rescores exactly every k with a_k <= min_j a_j + 2 delta,
    delta = 2^-6 ||res|| max ||c|| + 2^-14 max ||c||^2 + 1e-30.
That is safe if |a_k - s_k| <= delta for the exact s_k = ||c_k||^2 - 2 <res, c_k>
(the kernel's delta is twice the proven bound).  Here the scores are emulated
in numpy (bf16 by round-to-nearest-even through torch, sums in float32 in two
orders) on random and adversarial inputs, and the exact argmin (Section 3.5's
nearest codeword) must always be a candidate."""
import numpy as np
import pytest
import torch


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def emulate(res, C, reverse=False):
    """bf16 scores a [n][K] as the kernel forms them (fp32 sums, in dim order or reversed)."""
    nrm = np.zeros(C.shape[0], np.float32)
    for j in range(C.shape[1]):
        nrm = np.float32(nrm + C[:, j] * C[:, j])
    hi = bf16(nrm)
    lo = bf16(nrm - hi)
    rb, cb = bf16(-2.0 * res), bf16(C)
    a = np.zeros((res.shape[0], C.shape[0]), np.float32)
    dims = range(C.shape[1] - 1, -1, -1) if reverse else range(C.shape[1])
    for j in dims:
        a = np.float32(a + np.outer(rb[:, j], cb[:, j]).astype(np.float32))
    return np.float32(np.float32(a + hi[None, :]) + lo[None, :]), nrm


def kernel_delta(res, nrm):
    rn = np.sqrt(np.float32((res.astype(np.float32) ** 2).sum(1)))
    nmax = np.float32(nrm.max())
    return np.float32(2.0 ** -6) * rn * np.sqrt(nmax) + np.float32(2.0 ** -14) * nmax + np.float32(1e-30)


CASES = []
for w in (16, 32, 64):
    for kind in ("gauss", "near", "scaled_up", "scaled_down", "spread_norms"):
        CASES.append((w, kind))


@pytest.mark.parametrize("w,kind", CASES)
def test_bf16_scores_stay_within_half_the_kernels_delta(w, kind):
    rng = np.random.default_rng(w * 7 + len(kind))
    K, n = 256, 512
    C = rng.normal(0.0, 1.0 / np.sqrt(w), (K, w)).astype(np.float32)
    res = rng.normal(0.0, 1.0, (n, w)).astype(np.float32)
    if kind == "near":        # residuals a hair away from codewords: near-ties and cancellation
        res = (C[rng.integers(0, K, n)] + rng.normal(0.0, 1e-3, (n, w))).astype(np.float32)
    elif kind == "scaled_up":
        res *= np.float32(1e4)
        C *= np.float32(30.0)
    elif kind == "scaled_down":
        res *= np.float32(1e-5)
        C *= np.float32(1e-3)
    elif kind == "spread_norms":
        C *= np.geomspace(1e-3, 10.0, K, dtype=np.float32)[:, None]
    s = (C.astype(np.float64) ** 2).sum(1)[None, :] - 2.0 * res.astype(np.float64) @ C.astype(np.float64).T
    for reverse in (False, True):
        a, nrm = emulate(res, C, reverse)
        delta = kernel_delta(res, nrm).astype(np.float64)
        err = np.abs(a.astype(np.float64) - s)
        assert np.all(err <= 0.5 * delta[:, None]), float((err / delta[:, None]).max())
        # the exact argmin is a candidate
        kstar = s.argmin(1)
        lim = a.min(1).astype(np.float64) + 2.0 * delta
        assert np.all(a[np.arange(n), kstar] <= lim)
