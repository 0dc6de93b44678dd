"""GPU parity of the SPEL projector update (Section 3.3, Eq. (4)-(7),
Algorithm 1 step 4) against the fp64 oracle, through the C ABI.  All outputs
are fp32 and judged within 1e-5 relative L2."""
import numpy as np
import pytest
import torch

import learned_activation_compression_amd as lac
import synth
from oracle import spel
from parity_util import F32_TOL, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(A, g, m, alpha, beta, iters, expect_status=0):
    Ad, gd, md = A.clone().to(DEV), g.clone().to(DEV), m.clone().to(DEV)
    D = torch.empty_like(Ad)
    st = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    lac.spel_step(Ad, gd, md, alpha, beta, iters, D_out=D, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == expect_status
    return Ad, md, D


def spectrum_matrix(seed, d, r, cond):
    """A d x r matrix with singular values geometrically spread over [1/cond, 1] (times 1e-3)."""
    rng = np.random.default_rng(seed)
    U = np.linalg.qr(rng.standard_normal((d, r)))[0]
    V = np.linalg.qr(rng.standard_normal((r, r)))[0]
    sv = np.geomspace(1.0 / cond, 1.0, r)
    return torch.from_numpy((1e-3 * (U * sv) @ V.T).astype(np.float32))


def check(A, g, m, alpha, beta, iters, Ad, md, D):
    An, mn, Dn, _ = spel.spel_step(np64(A), np64(g), np64(m), alpha, beta, iters)
    assert_close(np64(md), mn, F32_TOL, "m")
    assert_close(np64(D), Dn, F32_TOL, "D")
    assert_close(np64(Ad), An, F32_TOL, "A")
    r = A.shape[1]
    An64 = np64(Ad)
    orth = np.linalg.norm(An64.T @ An64 - np.eye(r)) / np.sqrt(r)
    assert orth <= 1e-5, orth


def test_spel_1b_config():
    c = synth.CONFIGS["1b"]
    s = c["spel"]
    inp = synth.spel_inputs(c["seed"], c["d"], c["r"], s["g_var"])
    Ad, md, D = run(inp["A"], inp["g"], inp["m"], s["alpha"], s["beta"], s["ns_iters"])
    check(inp["A"], inp["g"], inp["m"], s["alpha"], s["beta"], s["ns_iters"], Ad, md, D)


@pytest.mark.parametrize("d,r,alpha,beta,iters", [(256, 32, 0.05, 0.9, 8), (1024, 128, 1e-3, 0.9, 8),
                                                  (512, 64, 0.3, 0.5, 5), (96, 96, 0.1, 0.0, 8),
                                                  (2048, 512, 2e-3, 0.95, 8),
                                                  (1056, 160, 0.02, 0.9, 8), (768, 192, 0.05, 0.9, 8),
                                                  (224, 224, 0.1, 0.5, 8)])
def test_spel_shapes_with_nonzero_momentum(d, r, alpha, beta, iters):
    inp = synth.spel_inputs(100 + d + r, d, r, 1e-3)
    m0 = torch.from_numpy(synth.gaussian(synth.stream(7, d, r), (d, r), 1e-4).astype(np.float32))
    Ad, md, D = run(inp["A"], inp["g"], m0, alpha, beta, iters)
    check(inp["A"], inp["g"], m0, alpha, beta, iters, Ad, md, D)


def test_spel_two_consecutive_steps():
    inp = synth.spel_inputs(31, 1024, 128, 1e-3)
    A, g, m = inp["A"], inp["g"], inp["m"]
    Ad, gd, md = A.clone().to(DEV), g.to(DEV), m.clone().to(DEV)
    A64, m64 = np64(A), np64(m)
    for step in range(2):
        lac.spel_step(Ad, gd, md, 1e-3, 0.9, 8)
        A64, m64, _, _ = spel.spel_step(A64, np64(g), m64, 1e-3, 0.9, 8)
    torch.cuda.synchronize()
    assert_close(np64(md), m64, F32_TOL, "m after 2 steps")
    assert_close(np64(Ad), A64, F32_TOL, "A after 2 steps")


def test_spel_zero_gradient_gives_zero_direction():
    inp = synth.spel_inputs(32, 512, 64, 1e-3)
    z = torch.zeros_like(inp["g"])
    Ad, md, D = run(inp["A"], z, z, 0.1, 0.9, 8)
    assert torch.count_nonzero(md) == 0 and torch.count_nonzero(D) == 0
    assert_close(np64(Ad), np64(inp["A"]), F32_TOL, "A fixed point")


def test_spel_repeat_is_bitwise_deterministic():
    inp = synth.spel_inputs(33, 2048, 256, 1e-3)
    a = run(inp["A"], inp["g"], inp["m"], 1e-3, 0.9, 8)
    b = run(inp["A"], inp["g"], inp["m"], 1e-3, 0.9, 8)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d,r", [(1024, 128), (2048, 256)])
def test_spel_repeat_is_bitwise_deterministic_in_gram_space(d, r):
    # r <= 256 runs the r x r (Gram-space) form of the iteration, whose workgroups meet at counters
    inp = synth.spel_inputs(34, d, r, 1e-3)
    m0 = torch.from_numpy(synth.gaussian(synth.stream(8, d, r), (d, r), 1e-4).astype(np.float32))
    a = run(inp["A"], inp["g"], m0, 1e-3, 0.9, 8)
    b = run(inp["A"], inp["g"], m0, 1e-3, 0.9, 8)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d,r", [(1024, 128), (2048, 256)])
def test_spel_wait_timeout_leaves_the_state_unchanged_then_recovers(monkeypatch, d, r):
    # the r x r iteration's workgroups wait for one another with a bounded wait; a test hook
    # lowers the bound to zero, so the first wait gives up and every kernel still exits: the
    # step must then be abandoned -- A and m bit-for-bit as they were, status 1 -- and the next
    # call with the normal bound must be correct again
    inp = synth.spel_inputs(35, d, r, 1e-3)
    m0 = torch.from_numpy(synth.gaussian(synth.stream(11, d, r), (d, r), 1e-4).astype(np.float32))
    monkeypatch.setenv("MAPL_SPEL_SPIN_LIMIT", "0")
    Ad, md, D = run(inp["A"], inp["g"], m0, 1e-3, 0.9, 8, expect_status=1)
    assert torch.equal(Ad.cpu(), inp["A"]) and torch.equal(md.cpu(), m0)
    monkeypatch.delenv("MAPL_SPEL_SPIN_LIMIT")
    Ad, md, D = run(inp["A"], inp["g"], m0, 1e-3, 0.9, 8)
    check(inp["A"], inp["g"], m0, 1e-3, 0.9, 8, Ad, md, D)


@pytest.mark.parametrize("d,r", [(1024, 128), (2048, 256), (640, 96)])
def test_spel_dxr_form_below_r256(monkeypatch, d, r):
    # a device that cannot hold every workgroup of the one-launch Gram-space iteration runs
    # each Newton-Schulz step on the d x r iterate; a test hook selects that form here
    inp = synth.spel_inputs(500 + d + r, d, r, 1e-3)
    m0 = torch.from_numpy(synth.gaussian(synth.stream(13, d, r), (d, r), 1e-4).astype(np.float32))
    monkeypatch.setenv("MAPL_SPEL_GRAM_SPACE", "0")
    Ad, md, D = run(inp["A"], inp["g"], m0, 1e-3, 0.9, 8)
    monkeypatch.delenv("MAPL_SPEL_GRAM_SPACE")
    check(inp["A"], inp["g"], m0, 1e-3, 0.9, 8, Ad, md, D)


@pytest.mark.parametrize("d,r,cond", [(1024, 128, 1e2), (1024, 128, 1e4), (256, 32, 1e4), (640, 96, 1e3),
                                      (2048, 256, 1e2), (2048, 256, 1e4), (1056, 160, 1e4)])
def test_spel_ill_conditioned_momentum(d, r, cond):
    """The LMO's input spread over a wide spectrum (condition number 1e2 to
    1e4) through the r x r Gram-space iteration (every r <= 256 here).  g = 0
    leaves m = beta m0, so the prescribed spectrum reaches the polar map
    unchanged."""
    inp = synth.spel_inputs(400 + d + r, d, r, 1e-3)
    m0 = spectrum_matrix(int(cond) + d + r, d, r, cond)
    z = torch.zeros_like(inp["g"])
    Ad, md, D = run(inp["A"], z, m0, 0.05, 0.9, 8)
    check(inp["A"], z, m0, 0.05, 0.9, 8, Ad, md, D)


@pytest.mark.parametrize("d,r,cond", [(1024, 128, 1e4), (2048, 256, 1e2), (640, 96, 1e3)])
def test_spel_ill_conditioned_momentum_dxr_form(monkeypatch, d, r, cond):
    """The same spectra through the d x r iteration (selected by the test hook)."""
    inp = synth.spel_inputs(400 + d + r, d, r, 1e-3)
    m0 = spectrum_matrix(int(cond) + d + r, d, r, cond)
    z = torch.zeros_like(inp["g"])
    monkeypatch.setenv("MAPL_SPEL_GRAM_SPACE", "0")
    Ad, md, D = run(inp["A"], z, m0, 0.05, 0.9, 8)
    monkeypatch.delenv("MAPL_SPEL_GRAM_SPACE")
    check(inp["A"], z, m0, 0.05, 0.9, 8, Ad, md, D)


@pytest.mark.parametrize("d,r,cond", [(1024, 128, 1e3), (2048, 256, 1e3)])
def test_spel_ill_conditioned_gradient(d, r, cond):
    """The Euclidean gradient itself ill-conditioned, with a non-zero momentum."""
    inp = synth.spel_inputs(500 + d + r, d, r, 1e-3)
    g = spectrum_matrix(7 + d, d, r, cond) * 10.0
    m0 = spectrum_matrix(8 + d, d, r, 10.0)
    Ad, md, D = run(inp["A"], g, m0, 1e-2, 0.9, 8)
    check(inp["A"], g, m0, 1e-2, 0.9, 8, Ad, md, D)


def test_spel_fed_by_the_codecs_own_projector_gradient():
    """Algorithm 1 end to end on the 150M boundary: gA from both backward maps
    of the bf16 codec (fp32 [1024][128]) is the Euclidean gradient of one
    spel_step on the fp32 projector; judged against the oracle on the same gA."""
    c = synth.CONFIGS["150m"]
    N = c["B"] * c["T"]
    inp = synth.codec_inputs(c["seed"], N, c["d"], c["r"], c["V"], "bf16")
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    gZ, gA = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
    lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"], gA=gA, accumulate=True)
    torch.cuda.synchronize()
    sp = synth.spel_inputs(c["seed"], c["d"], c["r"], 1e-3)
    gA = gA.cpu()
    assert torch.isfinite(gA).all()
    m0 = torch.from_numpy(synth.gaussian(synth.stream(12, c["d"], c["r"]), (c["d"], c["r"]), 1.0).astype(np.float32))
    Ad, md, D = run(sp["A"], gA, m0, 1e-3, 0.9, 8)
    check(sp["A"], gA, m0, 1e-3, 0.9, 8, Ad, md, D)


@pytest.mark.parametrize("d,r", [(1024, 128), (2048, 256)])
def test_spel_state_saved_and_reloaded_continues_bit_exactly(d, r):
    """Algorithm 1 threads (A_p, m_p) from step to step: two steps in place
    equal one step, a round trip of A and m through host memory into fresh
    device buffers, and a second step -- bit for bit."""
    inp = synth.spel_inputs(600 + d, d, r, 1e-3)
    gd = inp["g"].to(DEV)
    A1, m1 = inp["A"].clone().to(DEV), inp["m"].clone().to(DEV)
    lac.spel_step(A1, gd, m1, 1e-3, 0.9, 8)
    lac.spel_step(A1, gd, m1, 1e-3, 0.9, 8)
    A2, m2 = inp["A"].clone().to(DEV), inp["m"].clone().to(DEV)
    lac.spel_step(A2, gd, m2, 1e-3, 0.9, 8)
    torch.cuda.synchronize()
    saved = (A2.cpu().numpy().copy(), m2.cpu().numpy().copy())
    del A2, m2
    A3, m3 = torch.from_numpy(saved[0]).to(DEV), torch.from_numpy(saved[1]).to(DEV)
    lac.spel_step(A3, gd, m3, 1e-3, 0.9, 8)
    torch.cuda.synchronize()
    assert torch.equal(A1, A3) and torch.equal(m1, m3)


@pytest.mark.parametrize("d,r,iters", [(1024, 128, 1), (1024, 128, 2), (256, 64, 3), (640, 96, 4), (128, 32, 6),
                                       (1024, 128, 13), (2048, 256, 1), (2048, 256, 2), (512, 160, 3),
                                       (2048, 256, 13)])
def test_spel_few_and_many_iterations(d, r, iters):
    # m, D and A against the oracle for step counts other than 8 (A is not yet orthonormal
    # after one or two steps, so only the parity is checked)
    inp = synth.spel_inputs(300 + d + r + iters, d, r, 1e-3)
    m0 = torch.from_numpy(synth.gaussian(synth.stream(10, d, r), (d, r), 1e-4).astype(np.float32))
    Ad, md, D = run(inp["A"], inp["g"], m0, 0.02, 0.9, iters)
    An, mn, Dn, _ = spel.spel_step(np64(inp["A"]), np64(inp["g"]), np64(m0), 0.02, 0.9, iters)
    assert_close(np64(md), mn, F32_TOL, "m")
    assert_close(np64(D), Dn, F32_TOL, "D")
    assert_close(np64(Ad), An, F32_TOL, "A")


# ------------------------------------------------------------ Polar Express --
# The same step with the Polar Express polar map (5 LMO / 7 retraction steps,
# the schedule from [1e-3, 1]) against the oracle's spel_step_polar_express.

def run_pe(A, g, m, alpha, beta, lmo=5, ret=7):
    Ad, gd, md = A.clone().to(DEV), g.clone().to(DEV), m.clone().to(DEV)
    D = torch.empty_like(Ad)
    lac.spel_step_polar_express(Ad, gd, md, alpha, beta, lmo, ret, D_out=D)
    torch.cuda.synchronize()
    return Ad, md, D


def check_pe(A, g, m, alpha, beta, Ad, md, D, lmo=5, ret=7):
    An, mn, Dn, _ = spel.spel_step_polar_express(np64(A), np64(g), np64(m), alpha, beta, lmo, ret)
    assert_close(np64(md), mn, F32_TOL, "m")
    assert_close(np64(D), Dn, F32_TOL, "D")
    assert_close(np64(Ad), An, F32_TOL, "A")
    r = A.shape[1]
    An64 = np64(Ad)
    orth = np.linalg.norm(An64.T @ An64 - np.eye(r)) / np.sqrt(r)
    assert orth <= 1e-5, orth


@pytest.mark.parametrize("d,r,alpha,beta", [(1024, 128, 1e-3, 0.9), (2048, 256, 2e-3, 0.95), (256, 32, 0.05, 0.9),
                                            (96, 96, 0.1, 0.0), (1056, 160, 0.02, 0.9), (2048, 512, 1e-3, 0.9)])
def test_spel_polar_express_shapes(d, r, alpha, beta):
    inp = synth.spel_inputs(200 + d + r, d, r, 1e-3)
    m0 = torch.from_numpy(synth.gaussian(synth.stream(9, d, r), (d, r), 1e-4).astype(np.float32))
    Ad, md, D = run_pe(inp["A"], inp["g"], m0, alpha, beta)
    check_pe(inp["A"], inp["g"], m0, alpha, beta, Ad, md, D)


def test_spel_polar_express_other_step_counts():
    inp = synth.spel_inputs(41, 512, 64, 1e-3)
    Ad, md, D = run_pe(inp["A"], inp["g"], inp["m"], 0.01, 0.9, lmo=3, ret=9)
    check_pe(inp["A"], inp["g"], inp["m"], 0.01, 0.9, Ad, md, D, lmo=3, ret=9)


def test_spel_polar_express_zero_gradient_and_repeat():
    inp = synth.spel_inputs(42, 1024, 128, 1e-3)
    z = torch.zeros_like(inp["g"])
    Ad, md, D = run_pe(inp["A"], z, z, 0.1, 0.9)
    assert torch.count_nonzero(md) == 0 and torch.count_nonzero(D) == 0
    assert_close(np64(Ad), np64(inp["A"]), F32_TOL, "A fixed point")
    a = run_pe(inp["A"], inp["g"], inp["m"], 1e-3, 0.9)
    b = run_pe(inp["A"], inp["g"], inp["m"], 1e-3, 0.9)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_spel_polar_express_two_consecutive_steps():
    inp = synth.spel_inputs(43, 1024, 128, 1e-3)
    A, g, m = inp["A"], inp["g"], inp["m"]
    Ad, gd, md = A.clone().to(DEV), g.to(DEV), m.clone().to(DEV)
    A64, m64 = np64(A), np64(m)
    for _ in range(2):
        lac.spel_step_polar_express(Ad, gd, md, 1e-3, 0.9)
        A64, m64, _, _ = spel.spel_step_polar_express(A64, np64(g), m64, 1e-3, 0.9)
    torch.cuda.synchronize()
    assert_close(np64(md), m64, F32_TOL, "m after 2 steps")
    assert_close(np64(Ad), A64, F32_TOL, "A after 2 steps")
