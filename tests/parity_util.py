"""Shared helpers of the GPU parity tests (comparison rules only).

Floating-point outputs are compared twice: by the relative L2 error of the
whole tensor against the class tolerance, and row by row (a token row of a
codec output, a row of gA or of a spel matrix), so that one wrong row cannot
hide in the norm of a large tensor.  VQ codes are compared index by index."""
import numpy as np
import torch

BF16_TOL = 1e-2   # relative L2 for every output of a bf16 configuration
F32_TOL = 1e-5    # relative L2 for fp32 outputs
ROW_FACTOR = 4.0  # a row's own relative L2 may reach this multiple of the class tolerance
TIE_REL = 1e-6    # VQ codes may differ only where the oracle's top-2 gap is below this (relative to d1)


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a device or host tensor to float64 NumPy."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_l2(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(y - ref))
    return num / den if den > 0 else num


def row_rel_l2(y, ref) -> np.ndarray:
    """Relative L2 error of each row (last axis) of y against ref.  A row whose
    reference norm is below 1e-3 of the median row norm is measured against
    that floor instead (a near-zero row is judged by its absolute error)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.ndim < 2:
        y, ref = y.reshape(1, -1), ref.reshape(1, -1)
    y = y.reshape(-1, ref.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    floor = 1e-3 * float(np.median(den)) if den.size else 0.0
    den = np.maximum(den, max(floor, 1e-300))
    return num / den


def assert_close(y, ref, tol, what, row_factor=ROW_FACTOR):
    """Whole-tensor relative L2 within tol, and every row's within row_factor * tol."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape or y.size == ref.size, f"{what}: shape {y.shape} vs {ref.shape}"
    y = y.reshape(ref.shape)
    assert np.all(np.isfinite(y) == np.isfinite(ref)), f"{what}: non-finite values differ"
    e = rel_l2(y, ref)
    assert e <= tol, f"{what}: relative L2 error {e:.3e} > {tol:.1e} (max abs {np.max(np.abs(y - ref)):.3e})"
    if ref.size:
        rows = row_rel_l2(y, ref)
        worst = int(np.argmax(rows))
        assert rows[worst] <= row_factor * tol, (
            f"{what}: row {worst} has relative L2 error {rows[worst]:.3e} > {row_factor * tol:.1e} "
            f"(whole tensor {e:.3e})")
    return e


def check_codes(gpu_codes: np.ndarray, ora: dict, what: str):
    """VQ index rule: every code equals the oracle's argmin, except where the
    oracle's top-2 gap is a near-tie, (d2 - d1) <= TIE_REL * d1; there the
    GPU's codeword must be within TIE_REL * d1 of the best distance.  `ora`
    must come from a teacher-forced oracle run on the GPU's own codes (each
    round is then judged on its own).  Returns the number of mismatches."""
    gpu_codes = gpu_codes.astype(np.int64)
    mism = gpu_codes != ora["codes"]
    n_mis = int(mism.sum())
    if n_mis:
        d1, d2, dt = ora["d1"][mism], ora["d2"][mism], ora["d_teacher"][mism]
        margin = TIE_REL * d1
        near = (d2 - d1) <= margin
        ok = dt <= d1 + margin
        bad = int(np.count_nonzero(~(near & ok)))
        assert bad == 0, f"{what}: {bad} of {n_mis} code mismatches are not near-ties"
    return n_mis
