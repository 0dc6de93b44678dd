"""Seeded input generators (inputs only; no codec arithmetic lives here).

Every tensor is drawn from its own stream
``np.random.default_rng(SeedSequence([cfg_seed, tensor_id, sub]))`` in fp64
and then cast to the configuration's storage dtype.  The cast goes fp64 ->
fp32 (round to nearest even) and, for bf16, fp32 -> bf16 (round to nearest
even, done by torch).  Whatever bits come out are what both the oracle and the
GPU path read, so the exact rounding route of the cast does not affect parity.

Shapes and distributions follow the boundary workloads of the MAPL paper
(Learned Subspace Compression for Communication-Efficient Pipeline
Parallelism): widths of the 150M and 1B LLaMA stages (Appendix E.1), context
2048 and vocabulary 32000 (Section 4.1), and the rank-250 / 99 % energy
structure of boundary activations (Section 3.1, Figure 3).  N(mu, s) below
takes s as the *variance*.
"""
from __future__ import annotations

import math

import numpy as np
import torch

# tensor ids inside one configuration's seed space
TID_A, TID_P, TID_E, TID_TIDS, TID_X, TID_GXHAT, TID_C, TID_G, TID_STREAM = range(9)

# The five workloads.  N = B*T boundary tokens.
CONFIGS = {
    "tiny": dict(seed=1, B=1, T=128, d=256, r=32, V=1000, dtype="f32"),
    "150m": dict(seed=2, B=8, T=2048, d=1024, r=128, V=32000, dtype="bf16"),
    "sweep": dict(seed=3, B=8, T=2048, d=1024, ranks=(64, 256, 512), V=32000,
                  dtype="bf16", x_kind="lowrank"),
    "rvq": dict(seed=4, B=8, T=2048, d=1024, r=256, V=32000, G=8, K=256, R=2,
                dtype="bf16", codebook_var=1.0 / 32.0),
    "1b": dict(seed=5, B=4, T=2048, d=2048, r=256, V=32000, dtype="bf16",
               spel=dict(alpha=1e-3, beta=0.9, ns_iters=8, g_var=1e-3)),
}


def stream(cfg_seed: int, tensor_id: int, sub: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for one tensor of one configuration."""
    return np.random.default_rng(np.random.SeedSequence([int(cfg_seed), int(tensor_id), int(sub)]))


def gaussian(rng: np.random.Generator, shape, var: float = 1.0) -> np.ndarray:
    """fp64 samples of N(0, var)."""
    return rng.standard_normal(shape) * math.sqrt(var)


def orthonormal_columns(rng: np.random.Generator, d: int, r: int) -> np.ndarray:
    """fp64 d x r matrix with orthonormal columns: Q of the QR factorisation of
    a Gaussian d x r matrix, columns sign-fixed so that diag(R) > 0."""
    q, rr = np.linalg.qr(rng.standard_normal((d, r)))
    s = np.sign(np.diag(rr))
    s[s == 0] = 1.0
    return q * s[None, :]


def orthonormal_rows(rng: np.random.Generator, r: int, d: int) -> np.ndarray:
    """fp64 r x d matrix with orthonormal rows (the transpose of an
    independent orthonormal_columns draw)."""
    return np.ascontiguousarray(orthonormal_columns(rng, d, r).T)


def zipf_tids(rng: np.random.Generator, n: int, V: int, s: float = 1.1) -> np.ndarray:
    """int32 token ids in [0, V): finite-support Zipf p(k) ~ k^-s for
    k = 1..V, mapped to id k-1, drawn by inverse CDF from seeded uniforms."""
    k = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-s))
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int32)


def low_rank_plus_noise(rng: np.random.Generator, n: int, d: int, rank: int = 250,
                        signal_frac: float = 0.99) -> np.ndarray:
    """fp64 n x d matrix: a rank-`rank` Gaussian factor product carrying
    `signal_frac` of the energy plus isotropic Gaussian noise carrying the rest
    (total energy n*d)."""
    rank = min(rank, n, d)
    f1 = rng.standard_normal((n, rank))
    f2 = rng.standard_normal((rank, d))
    s = f1 @ f2
    s *= math.sqrt(signal_frac * n * d / float(np.sum(s * s)))
    w = rng.standard_normal((n, d))
    w *= math.sqrt((1.0 - signal_frac) * n * d / float(np.sum(w * w)))
    return s + w


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Cast fp64 values to the storage dtype ('f32' or 'bf16') as a CPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def codec_inputs(cfg_seed: int, N: int, d: int, r: int, V: int, dtype: str,
                 x_kind: str = "gauss", with_grad: bool = True,
                 e_var: float = 0.02, ra: int = None, anchor: str = "factorised") -> dict:
    """Inputs of one boundary: X [N][d], tids [N], E_small [V][ra], P [ra][d]
    (orthonormal rows; ra defaults to r), A [d][r] and, optionally, the
    upstream gradient gXhat [N][d] ~ N(0,1).

    anchor = "none": E and P are None (ra = 0); anchor = "full": E is [V][d]
    and P is None, standing for the d x d identity (ra = d).

    Returns CPU tensors in `dtype` (tids int32) plus the fp64 pre-cast A and P
    under 'A64' and 'P64', and the anchor rank under 'ra'.
    """
    if anchor == "none":
        ra = 0
    elif anchor == "full":
        ra = d
    elif anchor == "factorised":
        ra = r if ra is None else ra
    else:
        raise ValueError(f"unknown anchor kind {anchor!r}")
    A64 = orthonormal_columns(stream(cfg_seed, TID_A), d, r)
    P64 = orthonormal_rows(stream(cfg_seed, TID_P), ra, d) if anchor == "factorised" else None
    E = gaussian(stream(cfg_seed, TID_E), (V, ra), e_var) if ra > 0 else None
    tids = zipf_tids(stream(cfg_seed, TID_TIDS), N, V)
    if x_kind == "gauss":
        X = gaussian(stream(cfg_seed, TID_X), (N, d))
    elif x_kind == "lowrank":
        X = low_rank_plus_noise(stream(cfg_seed, TID_X), N, d)
    else:
        raise ValueError(f"unknown x_kind {x_kind!r}")
    out = dict(
        X=to_dtype(X, dtype), tids=torch.from_numpy(tids), E=None if E is None else to_dtype(E, dtype),
        P=None if P64 is None else to_dtype(P64, dtype), A=to_dtype(A64, dtype), A64=A64, P64=P64,
        N=N, d=d, r=r, V=V, ra=ra, anchor=anchor, dtype=dtype,
    )
    if with_grad:
        out["gXhat"] = to_dtype(gaussian(stream(cfg_seed, TID_GXHAT), (N, d)), dtype)
    return out


def rvq_codebooks(cfg_seed: int, R_c: int, G: int, K: int, w: int,
                  var: float = 1.0 / 32.0, sub: int = 0) -> torch.Tensor:
    """fp32 codebooks [R_c][G][K][w] with entries ~ N(0, var)."""
    c = gaussian(stream(cfg_seed, TID_C, sub), (R_c, G, K, w), var)
    return to_dtype(c, "f32")


def stream_packets(cfg_seed: int, call: int, sender: torch.Tensor) -> tuple:
    """One streaming-sync packet: for each (round-codebook, group) one codeword
    index drawn uniformly (a 1/K fraction of the K entries), returned as flat
    codeword indices q in [0, R_c*G*K) (int32) and the sender's values [n][w]
    (fp32, copied bit-exactly)."""
    R_c, G, K, w = sender.shape
    rng = stream(cfg_seed, TID_STREAM, call)
    per = max(1, math.ceil(K * (1.0 / K)))
    idx = []
    for rc in range(R_c):
        for g in range(G):
            ks = rng.choice(K, size=per, replace=False)
            idx.extend(int((rc * G + g) * K + k) for k in ks)
    idx_t = torch.tensor(idx, dtype=torch.int32)
    vals = sender.reshape(R_c * G * K, w)[idx_t.long()].clone()
    return idx_t, vals


def spel_inputs(cfg_seed: int, d: int, r: int, g_var: float = 1e-3) -> dict:
    """Projector-update inputs: A fp32 [d][r] with orthonormal columns, the
    Euclidean gradient g ~ N(0, g_var) fp32 and a zero momentum buffer."""
    A64 = orthonormal_columns(stream(cfg_seed, TID_A, 1), d, r)
    g = gaussian(stream(cfg_seed, TID_G), (d, r), g_var)
    return dict(A=to_dtype(A64, "f32"), g=to_dtype(g, "f32"),
                m=torch.zeros((d, r), dtype=torch.float32), A64=A64, d=d, r=r)
