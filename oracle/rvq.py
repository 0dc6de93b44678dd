"""Residual multi-codebook VQ of the projected boundary activation, fp64.

Source: *Learned Subspace Compression for Communication-Efficient Pipeline
Parallelism*, Section 3.5 "Composing with vector quantization": Z is split
into G groups and quantised over R rounds, each round quantising the residual
left by the previous one, against a per-stage codebook; "Codebook
Synchronization" and Appendix F: the sender streams a random subset of
codewords (a 1/K fraction per micro-batch) and the receiver overwrites them.
Appendix E.4 gives K = 256 and R = 2.

Readings taken where the pages are silent:
  * G is the number of groups; group g covers columns [g w, (g+1) w) with
    w = r / G;
  * codebooks are stored [R_c][G][K][w]: R_c = 1 is one codebook shared by all
    rounds (the literal per-stage C_p), R_c = R gives each round its own;
  * the distance is squared Euclidean, computed directly as sum (z - c)^2,
    and exact ties go to the lowest codeword index;
  * decoding sums the chosen codewords of all rounds in round order.

Test infrastructure only: see the package docstring.
"""
from __future__ import annotations

import math

import numpy as np


def _round_book(C: np.ndarray, rho: int) -> np.ndarray:
    R_c = C.shape[0]
    return C[rho if R_c > 1 else 0]


def encode(Z, C, G: int, K: int, R: int, teacher=None, chunk: int = 2048) -> dict:
    """Residual VQ encode.

    Z [N][r]; C [R_c][G][K][w] with R_c in {1, R}.  Returns a dict with
      codes    int64 [N][R][G]: argmin over k of sum_j (res_j - C_k,j)^2,
               lowest k on exact ties;
      d1, d2   the smallest and second-smallest distances per (n, rho, g)
               (d2 = inf when K = 1);
      d_teacher distance of the teacher's codeword (if `teacher` is given);
      energy   [R+1] total residual energy before round 0 and after each round;
      grew     [R] count of (n, g) whose group residual energy increased;
      residual the final residual [N][r].
    With `teacher` (int [N][R][G]) the residual of round rho is formed from the
    teacher's codes of earlier rounds (teacher forcing); the returned codes are
    still the oracle's own argmin of each round.
    """
    res = np.array(Z, dtype=np.float64, copy=True)
    C = np.asarray(C, dtype=np.float64)
    N, r = res.shape
    if r % G:
        raise ValueError("r must be a multiple of G")
    w = r // G
    if C.shape[1:] != (G, K, w) or C.shape[0] not in (1, R):
        raise ValueError(f"codebook shape {C.shape} does not match G={G} K={K} w={w} R={R}")
    codes = np.zeros((N, R, G), dtype=np.int64)
    d1 = np.zeros((N, R, G))
    d2 = np.full((N, R, G), np.inf)
    d_t = np.zeros((N, R, G)) if teacher is not None else None
    energy = [float(np.sum(res * res))]
    grew = []
    for rho in range(R):
        books = _round_book(C, rho)
        n_grew = 0
        for g in range(G):
            cb = books[g]
            sub = res[:, g * w:(g + 1) * w]  # view: updated in place below
            for s in range(0, N, chunk):
                e = min(N, s + chunk)
                diff = sub[s:e, None, :] - cb[None, :, :]
                D = np.sum(diff * diff, axis=2)          # [n][K]
                k1 = np.argmin(D, axis=1)                # first minimum = lowest index
                codes[s:e, rho, g] = k1
                part = np.partition(D, 1, axis=1) if K > 1 else D
                d1[s:e, rho, g] = part[:, 0]
                if K > 1:
                    d2[s:e, rho, g] = part[:, 1]
                chosen = k1 if teacher is None else np.asarray(teacher[s:e, rho, g], dtype=np.int64)
                if d_t is not None:
                    d_t[s:e, rho, g] = D[np.arange(e - s), chosen]
                before = np.sum(sub[s:e] * sub[s:e], axis=1)
                sub[s:e] -= cb[chosen]
                after = np.sum(sub[s:e] * sub[s:e], axis=1)
                n_grew += int(np.count_nonzero(after > before))
        energy.append(float(np.sum(res * res)))
        grew.append(n_grew)
    return dict(codes=codes, d1=d1, d2=d2, d_teacher=d_t, energy=np.array(energy),
                grew=np.array(grew), residual=res)


def decode(codes, C, G: int, K: int, R: int) -> np.ndarray:
    """Residual VQ decode: Zq[n, group g] = sum over rounds rho (in order) of
    the codeword codes[n][rho][g] of round rho's codebook for group g."""
    codes = np.asarray(codes, dtype=np.int64)
    C = np.asarray(C, dtype=np.float64)
    N = codes.shape[0]
    w = C.shape[3]
    out = np.zeros((N, G * w), dtype=np.float64)
    for rho in range(R):
        books = _round_book(C, rho)
        for g in range(G):
            out[:, g * w:(g + 1) * w] += books[g][codes[:, rho, g]]
    return out


def stream_apply(C, idx, vals) -> np.ndarray:
    """Appendix F streaming sync on the receiver: overwrite whole codewords.
    `idx` holds flat codeword indices q in [0, R_c*G*K); `vals` is [n][w]."""
    C = np.array(C, copy=True)
    R_c, G, K, w = C.shape
    flat = C.reshape(R_c * G * K, w)
    flat[np.asarray(idx, dtype=np.int64)] = np.asarray(vals, dtype=C.dtype)
    return flat.reshape(R_c, G, K, w)


def bytes_per_token(G: int, R: int, K: int) -> float:
    """Payload of the VQ codes per token: G R ceil(log2 K) bits."""
    return G * R * math.ceil(math.log2(K)) / 8.0
