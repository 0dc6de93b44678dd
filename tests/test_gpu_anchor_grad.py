"""GPU parity of the anchor-table gradient gE_small (Eq. (3): E_small is
trainable; its rows enter Eq. (1) with a minus sign and Eq. (2) with a plus
sign) against the fp64 oracle, through the C ABI.

The output is fp32 whatever the input dtype.  Teacher-forced comparisons (the
oracle reads the exact Y bits the GPU read) hold to the fp32 bound 1e-5
relative L2; the sender's end-to-end chain (gZ -> bf16 gX -> gE) is judged at
the bf16 bound 1e-2.  The fixed-point accumulation makes the result bitwise
independent of token order, which is tested directly."""
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


def oracle_rows(Y, tids, P, V, alpha):
    """alpha * scatter-sum of Y P^T by tids, through the oracle's receiver
    form (gZ = 0, gXhat = alpha * Y).  Tokens whose id is outside [0, V) are
    dropped first: they have no table row."""
    t = np.asarray(tids, dtype=np.int64)
    keep = (t >= 0) & (t < V)
    Y, t = alpha * np.asarray(Y, np.float64)[keep], t[keep]
    P = np.asarray(P, np.float64)
    r = P.shape[0]
    return codec.anchor_grad(np.zeros((len(t), r)), t, P, np.zeros((P.shape[1], r)), V, gXhat=Y, P_recv=P)


def sender_chain(inp, g):
    """gZ from the receiver's backward, gX from the sender's (both on the GPU)."""
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    gZ, _ = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
    gX, _ = lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"])
    return gZ, gX


def check_both_tables(inp, tol_e2e):
    g = to_dev(inp)
    V, t, P = inp["V"], inp["tids"].numpy(), np64(inp["P"])
    # receiver's table: Y = gXhat, alpha = +1
    gE_r = lac.mapl_anchor_grad(g["gXhat"], g["tids"], g["P"], V, 1.0)
    # sender's table: Y = gX, alpha = -1; then both into one shared table
    gZ, gX = sender_chain(inp, g)
    gE_s = lac.mapl_anchor_grad(gX, g["tids"], g["P"], V, -1.0)
    gE_sum = gE_r.clone()
    lac.mapl_anchor_grad(gX, g["tids"], g["P"], V, -1.0, gE=gE_sum, accumulate=True)
    torch.cuda.synchronize()
    A = np64(inp["A"])
    ref_r = oracle_rows(np64(inp["gXhat"]), t, P, V, 1.0)
    assert_close(np64(gE_r), ref_r, F32_TOL, "gE receiver")
    ref_r_oracle = codec.anchor_grad(np.zeros((len(t), P.shape[0])), t, P, A, V, gXhat=np64(inp["gXhat"]), P_recv=P)
    assert_close(np64(gE_r), ref_r_oracle, F32_TOL, "gE receiver (oracle form)")
    # teacher-forced on the GPU's gX bits
    ref_s_tf = oracle_rows(np64(gX), t, P, V, -1.0)
    assert_close(np64(gE_s), ref_s_tf, F32_TOL, "gE sender (teacher-forced)")
    # end to end: the oracle's -gZ (P A)^T from the GPU's gZ bits
    ref_s = codec.anchor_grad(np64(gZ), t, P, A, V)
    assert_close(np64(gE_s), ref_s, tol_e2e, "gE sender (end to end)")
    # the two tables can cancel (r = d makes A A^T = I, so gX = gXhat): judge
    # the sum's error against the size of its parts
    err = np.linalg.norm(np64(gE_sum) - (ref_r + ref_s_tf)) / (np.linalg.norm(ref_r) + np.linalg.norm(ref_s_tf))
    assert err <= F32_TOL, f"gE shared table (accumulated): error {err:.3e} relative to its parts"


def test_tiny_config_fp32():
    c = synth.CONFIGS["tiny"]
    inp = synth.codec_inputs(c["seed"], c["B"] * c["T"], c["d"], c["r"], c["V"], "f32")
    check_both_tables(inp, F32_TOL)


@pytest.mark.parametrize("N,d,r,V", [(77, 96, 20, 50), (300, 160, 33, 7), (1, 64, 64, 3)])
def test_fp32_odd_shapes(N, d, r, V):
    inp = synth.codec_inputs(40 + N, N, d, r, V, "f32")
    check_both_tables(inp, F32_TOL)


@pytest.mark.parametrize("N,d,r,V", [(1000, 384, 64, 300), (257, 1024, 128, 5000), (777, 2048, 256, 40),
                                     (96, 1024, 512, 1)])
def test_bf16_small(N, d, r, V):
    inp = synth.codec_inputs(50 + N, N, d, r, V, "bf16")
    check_both_tables(inp, BF16_TOL)


@pytest.mark.parametrize("N,d,r,V", [(96, 128, 32, 1), (33, 256, 32, 9), (500, 640, 128, 64)])
def test_bf16_receiver_narrow_shapes(N, d, r, V):
    inp = synth.codec_inputs(70 + N, N, d, r, V, "bf16")
    g = to_dev(inp)
    gE = lac.mapl_anchor_grad(g["gXhat"], g["tids"], g["P"], V, 1.0)
    torch.cuda.synchronize()
    ref = oracle_rows(np64(inp["gXhat"]), inp["tids"].numpy(), np64(inp["P"]), V, 1.0)
    assert_close(np64(gE), ref, F32_TOL, "gE receiver")


def test_out_of_range_tids_contribute_nothing():
    V = 400
    inp = synth.codec_inputs(61, 700, 512, 64, V, "bf16")
    t = inp["tids"].clone()
    t[::5] = -1
    t[2::9] = V
    t[4::13] = 2 ** 31 - 1
    g = to_dev(inp)
    g["tids"] = t.to(DEV)
    gE = lac.mapl_anchor_grad(g["gXhat"], g["tids"], g["P"], V, 0.5)
    torch.cuda.synchronize()
    assert_close(np64(gE), oracle_rows(np64(inp["gXhat"]), t.numpy(), np64(inp["P"]), V, 0.5), F32_TOL, "gE")


def test_token_order_does_not_change_a_bit():
    # integer sums are associative: any permutation of the tokens gives the
    # same table, bit for bit (Zipf ids put hundreds of tokens on one row)
    inp = synth.codec_inputs(62, 4096, 1024, 128, 2000, "bf16")
    g = to_dev(inp)
    gE1 = lac.mapl_anchor_grad(g["gXhat"], g["tids"], g["P"], 2000, -1.0)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(4096)).to(DEV)
    gE2 = lac.mapl_anchor_grad(g["gXhat"][perm].contiguous(), g["tids"][perm].contiguous(), g["P"], 2000, -1.0)
    gE3 = lac.mapl_anchor_grad(g["gXhat"], g["tids"], g["P"], 2000, -1.0)
    torch.cuda.synchronize()
    assert torch.equal(gE1, gE2)
    assert torch.equal(gE1, gE3)


def test_prepacked_weights_give_identical_bits():
    inp = synth.codec_inputs(64, 3000, 1024, 128, 700, "bf16")
    g = to_dev(inp)
    pk = lac.mapl_pack(g["P"], g["A"])
    a = lac.mapl_anchor_grad(g["gXhat"], g["tids"], g["P"], 700, 1.0)
    b = lac.mapl_anchor_grad(g["gXhat"], g["tids"], g["P"], 700, 1.0, pk=pk, pk_ready=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_zero_gradient_and_empty_batch():
    inp = synth.codec_inputs(63, 128, 256, 32, 50, "bf16")
    g = to_dev(inp)
    gE = torch.full((50, 32), 9.0, device=DEV)
    lac.mapl_anchor_grad(torch.zeros_like(g["gXhat"]), g["tids"], g["P"], 50, 1.0, gE=gE)
    torch.cuda.synchronize()
    assert bool((gE == 0).all())
    gE.fill_(2.5)
    lac.mapl_anchor_grad(torch.zeros_like(g["gXhat"]), g["tids"], g["P"], 50, 1.0, gE=gE, accumulate=True)
    lac.mapl_anchor_grad(g["gXhat"][:0], g["tids"][:0], g["P"], 50, 1.0, gE=gE, accumulate=True)
    torch.cuda.synchronize()
    assert bool((gE == 2.5).all())
    lac.mapl_anchor_grad(g["gXhat"][:0], g["tids"][:0], g["P"], 50, 1.0, gE=gE)
    torch.cuda.synchronize()
    assert bool((gE == 0).all())


@pytest.mark.parametrize("dtype,r,ident", [("bf16", 128, False), ("bf16", 64, False), ("f32", 32, False),
                                           ("bf16", 256, True), ("f32", 256, True)])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_non_finite_gradient_marks_the_table(dtype, r, ident, bad):
    """A NaN or an Inf in Y has no fixed-point scale: the whole table becomes
    NaN (also when accumulating) instead of the value vanishing or saturating.
    Covers each projection path: the codec's streaming kernel (bf16 r = 128),
    the plain bf16 and fp32 kernels and the identity (full-rank anchor)."""
    N, d, V = 333, 256, 70
    inp = synth.codec_inputs(64, N, d, r, V, dtype)
    g = to_dev(inp)
    Y = g["gXhat"].clone()
    Y[17, 5] = bad
    P = None if ident else g["P"]
    ra = d if ident else r
    gE = lac.mapl_anchor_grad(Y, g["tids"], P, V, 1.0, r=r)
    gE2 = torch.ones((V, ra), dtype=torch.float32, device=DEV)
    lac.mapl_anchor_grad(Y, g["tids"], P, V, -1.0, gE=gE2, accumulate=True, r=r)
    torch.cuda.synchronize()
    assert bool(torch.isnan(gE).all()) and bool(torch.isnan(gE2).all())
    # the same call on finite data is finite again (nothing is left behind)
    gE3 = lac.mapl_anchor_grad(g["gXhat"], g["tids"], P, V, 1.0, r=r)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(gE3).all())


@pytest.mark.parametrize("name,r", [("150m", None), ("sweep", 512), ("1b", None)])
def test_full_size(name, r):
    c = synth.CONFIGS[name]
    inp = synth.codec_inputs(c["seed"], c["B"] * c["T"], c["d"], r or c["r"], c["V"], c["dtype"],
                             x_kind=c.get("x_kind", "gauss"))
    check_both_tables(inp, BF16_TOL)
