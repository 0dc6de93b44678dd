"""Shared helpers of the GPU parity tests (comparison rules only)."""
import numpy as np
import torch

BF16_TOL = 1e-2   # relative L2 for every output of a bf16 configuration
F32_TOL = 1e-5    # relative L2 for fp32 outputs
TIE_REL = 1e-6    # VQ codes may differ only where the oracle's top-2 gap is below this (relative)


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a device or host tensor to float64 NumPy."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_l2(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(y - ref))
    return num / den if den > 0 else num


def assert_close(y, ref, tol, what):
    e = rel_l2(y, ref)
    assert e <= tol, f"{what}: relative L2 error {e:.3e} > {tol:.1e} (max abs {np.max(np.abs(np.asarray(y, np.float64) - ref)):.3e})"
    return e


def check_codes(gpu_codes: np.ndarray, ora: dict, what: str):
    """VQ index rule: equal to the oracle's argmin, except at near-ties.  The
    GPU scores codewords in fp32 as ||c||^2 - 2<z, c> (the squared distance
    less ||z||^2), whose rounding error scales with the size of those terms,
    not with the distance itself; so a near-tie is a top-2 gap below TIE_REL
    times max(d1, ||z||^2 + max ||c||^2) (the oracle's `scale`), and there the
    GPU's choice must be within the same margin of the best distance.  `ora`
    must come from a teacher-forced oracle run on the GPU's own codes (so each
    round is judged on its own)."""
    gpu_codes = gpu_codes.astype(np.int64)
    mism = gpu_codes != ora["codes"]
    n_mis = int(mism.sum())
    if n_mis:
        d1, d2, dt = ora["d1"][mism], ora["d2"][mism], ora["d_teacher"][mism]
        margin = TIE_REL * np.maximum(np.maximum(d1, ora["scale"][mism]), 1e-30)
        near = (d2 - d1) <= margin
        ok = dt <= d1 + margin
        bad = int(np.count_nonzero(~(near & ok)))
        assert bad == 0, f"{what}: {bad} of {n_mis} code mismatches are not near-ties"
    return n_mis
