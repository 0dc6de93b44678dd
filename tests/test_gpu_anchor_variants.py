"""GPU parity of the anchor variants of Appendix G (Table 6) against the fp64
oracle, through the C ABI: no anchor (ra = 0), a factorised anchor whose rank
ra differs from the projector's rank r, and the fully trainable anchor
E in R^{V x d} with P = I (passed as no P, ra = d).

Each case runs the forward pair, both backward maps and (when there is a
table) both anchor-table gradients, at sizes that span several tiles and end
in a ragged tile.  Tolerances as elsewhere: relative L2 1e-2 for bf16 outputs,
1e-5 for fp32 outputs and for the fp32 table gradient read teacher-forced."""
import numpy as np
import pytest
import torch

import learned_activation_compression_amd as lac
import synth
from oracle import codec
from parity_util import BF16_TOL, F32_TOL, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def oracle_anchor(inp):
    """(E, P) for the oracle: None for no anchor, the d x d identity for the
    full-rank anchor."""
    if inp["anchor"] == "none":
        return None, None
    E = np64(inp["E"])
    P = np.eye(inp["d"]) if inp["anchor"] == "full" else np64(inp["P"])
    return E, P


def run_and_check(inp, tol):
    g = to_dev(inp)
    V, r = inp["V"], inp["r"]
    X, t, A = np64(inp["X"]), inp["tids"].numpy(), np64(inp["A"])
    E, P = oracle_anchor(inp)
    # forward pair
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    Xh = lac.mapl_reconstruct(Z, g["tids"], g["E"], g["P"], g["A"])
    torch.cuda.synchronize()
    Z_ref = codec.compress(X, t, E, P, A)
    assert_close(np64(Z), Z_ref, tol, "Z")
    assert_close(np64(Xh), codec.reconstruct(np64(Z), t, E, P, A), tol, "Xhat (teacher-forced)")
    assert_close(np64(Xh), codec.reconstruct(Z_ref, t, E, P, A), tol, "Xhat (end to end)")
    # backward maps
    gZ, gA_rec = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
    gX, gA_cmp = lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"])
    gA_sum = gA_rec.clone()
    lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"], gA=gA_sum, accumulate=True)
    torch.cuda.synchronize()
    gZ_ref, gA_rec_ref = codec.reconstruct_bwd(np64(inp["gXhat"]), np64(Z), A)
    assert_close(np64(gZ), gZ_ref, tol, "gZ")
    assert_close(np64(gA_rec), gA_rec_ref, tol, "gA_rec")
    gX_ref, gA_cmp_ref = codec.compress_bwd(np64(gZ), X, t, E, P, A)
    assert_close(np64(gX), gX_ref, tol, "gX")
    assert_close(np64(gA_cmp), gA_cmp_ref, tol, "gA_cmp")
    assert_close(np64(gA_sum), gA_rec_ref + gA_cmp_ref, tol, "gA (accumulated)")
    if E is None:
        return
    # anchor-table gradients: receiver (Y = gXhat, +1) and sender (Y = gX, -1)
    gE_r = lac.mapl_anchor_grad(g["gXhat"], g["tids"], g["P"], V, 1.0, r=r)
    gE_s = lac.mapl_anchor_grad(gX, g["tids"], g["P"], V, -1.0, r=r)
    torch.cuda.synchronize()
    ra = P.shape[0]
    assert gE_r.shape == (V, ra) and gE_s.shape == (V, ra)
    zero = np.zeros((len(t), r))
    ref_r = codec.anchor_grad(zero, t, P, np.zeros_like(A), V, gXhat=np64(inp["gXhat"]), P_recv=P)
    assert_close(np64(gE_r), ref_r, F32_TOL, "gE receiver")
    ref_s_tf = codec.anchor_grad(zero, t, P, np.zeros_like(A), V, gXhat=-np64(gX), P_recv=P)
    assert_close(np64(gE_s), ref_s_tf, F32_TOL, "gE sender (teacher-forced)")
    assert_close(np64(gE_s), codec.anchor_grad(np64(gZ), t, P, A, V), tol, "gE sender (end to end)")


# (anchor kind, N, d, r, ra): ra None = the kind's own (r, 0 or d)
BF16_CASES = [
    ("none", 1000, 512, 128, None),
    ("none", 200, 128, 32, None),
    ("none", 300, 1024, 512, None),
    ("factorised", 1000, 512, 128, 64),
    ("factorised", 1000, 512, 128, 256),
    ("factorised", 777, 1024, 256, 128),
    ("factorised", 500, 1024, 512, 256),
    ("factorised", 300, 512, 64, 512),
    ("full", 1000, 512, 128, None),
    ("full", 600, 640, 256, None),
    ("full", 300, 1024, 512, None),
    ("full", 129, 128, 64, None),
]


@pytest.mark.parametrize("anchor,N,d,r,ra", BF16_CASES)
def test_bf16_anchor_variants(anchor, N, d, r, ra):
    inp = synth.codec_inputs(90 + N, N, d, r, 700, "bf16", ra=ra, anchor=anchor)
    run_and_check(inp, BF16_TOL)


FP32_CASES = [
    ("none", 37, 100, 7, None),
    ("factorised", 37, 100, 7, 5),
    ("factorised", 57, 100, 7, 12),
    ("full", 37, 100, 7, None),
    ("full", 257, 512, 96, None),
]


@pytest.mark.parametrize("anchor,N,d,r,ra", FP32_CASES)
def test_fp32_anchor_variants(anchor, N, d, r, ra):
    inp = synth.codec_inputs(95 + N, N, d, r, 50, "f32", ra=ra, anchor=anchor)
    run_and_check(inp, F32_TOL)


def test_full_anchor_matches_a_dense_identity_projector():
    """P = NULL (rows added or subtracted directly) against a dense identity P
    through the general path: the two are the same map."""
    inp = synth.codec_inputs(97, 700, 512, 128, 300, "bf16", anchor="full")
    g = to_dev(inp)
    I = torch.eye(512, dtype=torch.bfloat16, device=DEV)
    Z0 = lac.mapl_compress(g["X"], g["tids"], g["E"], None, g["A"])
    Z1 = lac.mapl_compress(g["X"], g["tids"], g["E"], I, g["A"])
    Xh0 = lac.mapl_reconstruct(Z0, g["tids"], g["E"], None, g["A"])
    Xh1 = lac.mapl_reconstruct(Z0, g["tids"], g["E"], I, g["A"])
    gE0 = lac.mapl_anchor_grad(g["gXhat"], g["tids"], None, 300, 1.0)
    gE1 = lac.mapl_anchor_grad(g["gXhat"], g["tids"], I, 300, 1.0, r=128)
    torch.cuda.synchronize()
    # compress: -(I A)^T rounds to exactly -A^T, and both sum in the same order
    assert torch.equal(Z0, Z1)
    assert_close(np64(Xh0), np64(Xh1), BF16_TOL / 10, "Xhat, identity vs dense I")
    assert_close(np64(gE0), np64(gE1), F32_TOL, "gE, identity vs dense I")


@pytest.mark.parametrize("anchor,ra", [("none", None), ("factorised", 256), ("full", None)])
def test_prepacked_variants_give_identical_bits(anchor, ra):
    inp = synth.codec_inputs(98, 500, 512, 128, 300, "bf16", ra=ra, anchor=anchor)
    g = to_dev(inp)
    pk = lac.mapl_pack(g["P"], g["A"], ra=inp["ra"])
    outs = []
    for kw in (dict(), dict(pk=pk, pk_ready=True)):
        Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"], **kw)
        Xh = lac.mapl_reconstruct(Z, g["tids"], g["E"], g["P"], g["A"], **kw)
        gZ, _ = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
        gX, gA = lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"], **kw)
        torch.cuda.synchronize()
        outs.append([Z, Xh, gX, gA])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_full_anchor_out_of_range_tids_use_a_zero_row():
    inp = synth.codec_inputs(99, 400, 512, 128, 300, "bf16", anchor="full")
    t = inp["tids"].clone()
    t[::5] = -3
    t[2::9] = 300
    inp["tids"] = t
    g = to_dev(inp)
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], None, g["A"])
    Xh = lac.mapl_reconstruct(Z, g["tids"], g["E"], None, g["A"])
    gE = lac.mapl_anchor_grad(g["gXhat"], g["tids"], None, 300, 1.0)
    torch.cuda.synchronize()
    # reading: an invalid id's anchor row is zero -> oracle with a zero row appended
    tn = t.numpy()
    keep = (tn >= 0) & (tn < 300)
    tm = np.where(keep, tn, 300)
    E_ext = np.vstack([np64(inp["E"]), np.zeros((1, 512))])
    I = np.eye(512)
    X, A = np64(inp["X"]), np64(inp["A"])
    assert_close(np64(Z), codec.compress(X, tm, E_ext, I, A), BF16_TOL, "Z")
    assert_close(np64(Xh), codec.reconstruct(np64(Z), tm, E_ext, I, A), BF16_TOL, "Xhat")
    ref = codec.anchor_grad(np.zeros((int(keep.sum()), 128)), tn[keep], I, np.zeros((512, 128)), 300,
                            gXhat=np64(inp["gXhat"])[keep], P_recv=I)
    assert_close(np64(gE), ref, F32_TOL, "gE (invalid ids dropped)")


# ------------------------------------------- full-size workloads (150M) --

@pytest.mark.parametrize("anchor,ra", [("none", None), ("full", None), ("factorised", 256)])
def test_full_size_variants(anchor, ra):
    c = synth.CONFIGS["150m"]
    inp = synth.codec_inputs(c["seed"], c["B"] * c["T"], c["d"], c["r"], c["V"], c["dtype"], ra=ra, anchor=anchor)
    run_and_check(inp, BF16_TOL)
