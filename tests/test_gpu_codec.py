"""GPU parity of the MAPL codec (Eq. (1)-(3)) and its backward against the
fp64 oracle, through the C ABI.

Every comparison is relative L2 over the whole tensor: fp32 outputs within
1e-5, bf16 outputs within 1e-2.  Each map is judged teacher-forced (the oracle
reads the exact bits the GPU read) and, for the forward pair, also end to end
against the oracle's own chain."""
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


def run_forward(g, pk=None, pk_ready=False):
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"], pk=pk, pk_ready=pk_ready)
    Xh = lac.mapl_reconstruct(Z, g["tids"], g["E"], g["P"], g["A"], pk=pk, pk_ready=pk_ready)
    torch.cuda.synchronize()
    return Z, Xh


def check_forward(inp, Z, Xh, tol):
    X, t, E, P, A = (np64(inp["X"]), inp["tids"].numpy(), np64(inp["E"]), np64(inp["P"]), np64(inp["A"]))
    Z_ref = codec.compress(X, t, E, P, A)
    assert_close(np64(Z), Z_ref, tol, "Z")
    # teacher-forced: reconstruct from the GPU's Z bits
    assert_close(np64(Xh), codec.reconstruct(np64(Z), t, E, P, A), tol, "Xhat (teacher-forced)")
    # end to end: the oracle's own chain
    assert_close(np64(Xh), codec.reconstruct(Z_ref, t, E, P, A), tol, "Xhat (end to end)")


def check_backward(inp, g, tol, Z):
    gXh = inp["gXhat"]
    gZ, gA_rec = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
    gX, gA_cmp = lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"])
    gA_sum = gA_rec.clone()
    lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"], gA=gA_sum, accumulate=True)
    torch.cuda.synchronize()
    A, X, t, E, P = np64(inp["A"]), np64(inp["X"]), inp["tids"].numpy(), np64(inp["E"]), np64(inp["P"])
    gZ_ref, gA_rec_ref = codec.reconstruct_bwd(np64(gXh), np64(Z), A)
    assert_close(np64(gZ), gZ_ref, tol, "gZ")
    assert_close(np64(gA_rec), gA_rec_ref, tol, "gA_rec")
    gX_ref, gA_cmp_ref = codec.compress_bwd(np64(gZ), X, t, E, P, A)
    assert_close(np64(gX), gX_ref, tol, "gX")
    assert_close(np64(gA_cmp), gA_cmp_ref, tol, "gA_cmp")
    assert_close(np64(gA_sum), gA_rec_ref + gA_cmp_ref, tol, "gA (accumulated)")


# ------------------------------------------------------------------ fp32 --

def test_tiny_config_fp32_codec_and_backward():
    c = synth.CONFIGS["tiny"]
    N = c["B"] * c["T"]
    inp = synth.codec_inputs(c["seed"], N, c["d"], c["r"], c["V"], "f32")
    g = to_dev(inp)
    Z, Xh = run_forward(g)
    check_forward(inp, Z, Xh, F32_TOL)
    check_backward(inp, g, F32_TOL, Z)


@pytest.mark.parametrize("N,d,r", [(1, 8, 3), (37, 100, 7), (257, 512, 96)])
def test_fp32_codec_odd_shapes(N, d, r):
    inp = synth.codec_inputs(11, N, d, r, 50, "f32")
    g = to_dev(inp)
    Z, Xh = run_forward(g)
    check_forward(inp, Z, Xh, F32_TOL)
    check_backward(inp, g, F32_TOL, Z)


def test_fp32_round_trip_in_span():
    """Section 3.2: with equal anchors, a residual inside span(A) round-trips."""
    inp = synth.codec_inputs(1, 128, 256, 32, 1000, "f32")
    A64, P64 = inp["A64"], inp["P64"]
    W = np.random.default_rng(3).standard_normal((128, 32))
    X = codec.anchor(inp["tids"].numpy(), np64(inp["E"]), np64(inp["P"])) + W @ np64(inp["A"]).T
    inp["X"] = torch.from_numpy(X.astype(np.float32))
    g = to_dev(inp)
    Z, Xh = run_forward(g)
    assert_close(np64(Xh), np64(inp["X"]), 1e-5, "round trip")


# ------------------------------------------------------------------ bf16 --

SMALL_BF16 = [  # (N, d, r): several tiles plus a ragged tail in tokens and channels
    (1000, 1024, 128),
    (777, 2048, 256),
    (130, 384, 64),      # d not a multiple of the 256-channel tile
    (300, 1024, 512),
    (65, 512, 32),
    (200, 640, 32),
    (1, 128, 32),
]


@pytest.mark.parametrize("N,d,r", SMALL_BF16)
def test_bf16_codec_small(N, d, r):
    inp = synth.codec_inputs(21, N, d, r, 5000, "bf16")
    g = to_dev(inp)
    Z, Xh = run_forward(g)
    check_forward(inp, Z, Xh, BF16_TOL)
    check_backward(inp, g, BF16_TOL, Z)


def test_bf16_prepacked_weights_give_identical_bits():
    inp = synth.codec_inputs(22, 500, 1024, 128, 5000, "bf16")
    g = to_dev(inp)
    Z0, Xh0 = run_forward(g)
    pk = lac.mapl_pack(g["P"], g["A"])
    Z1, Xh1 = run_forward(g, pk=pk, pk_ready=True)
    assert torch.equal(Z0, Z1) and torch.equal(Xh0, Xh1)


@pytest.mark.parametrize("N,d,r", [(1000, 1024, 128), (777, 2048, 256), (130, 384, 64)])
def test_bf16_compress_with_kernel_events(N, d, r):
    # the instrumented launch (hipExtLaunchKernelGGL with the caller's events) computes the same
    # bits, stamps a positive kernel time, and the arming lasts for one call only
    inp = synth.codec_inputs(24, N, d, r, 5000, "bf16")
    g = to_dev(inp)
    Z0 = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    lac.mapl_time_next_compress_kernel(e0, e1)
    Z1 = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 100.0, ms
    Z2 = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])  # not armed any more
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == ms
    assert torch.equal(Z0, Z1) and torch.equal(Z0, Z2)
    # an armed call that cannot be timed launches nothing and leaves Z alone
    Zf = torch.full((N, r), 7.0, device=DEV)
    lac.mapl_time_next_compress_kernel(e0, e1)
    with pytest.raises(lac.MaplError):
        lac.mapl_compress(g["X"].float(), g["tids"], g["E"].float(), g["P"].float(), g["A"].float(), Z=Zf)
    torch.cuda.synchronize()
    assert bool((Zf == 7.0).all())


def test_bf16_repeat_is_bitwise_deterministic():
    inp = synth.codec_inputs(23, 2048, 1024, 128, 32000, "bf16")
    g = to_dev(inp)
    outs = []
    for _ in range(2):
        Z, Xh = run_forward(g)
        gZ, gA1 = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
        gX, gA2 = lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"])
        torch.cuda.synchronize()
        outs.append([Z, Xh, gZ, gA1, gX, gA2])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_bf16_out_of_range_tids_use_a_zero_anchor():
    inp = synth.codec_inputs(24, 300, 1024, 128, 5000, "bf16")
    t = inp["tids"].clone()
    t[::7] = -1
    t[3::11] = 5000
    inp["tids"] = t
    g = to_dev(inp)
    bad = lac.mapl_check_tids(g["tids"], 5000)
    Z, Xh = run_forward(g)
    assert int(bad.item()) == int(((t < 0) | (t >= 5000)).sum())
    # reading: an invalid id's anchor row is zero -> oracle with a zero row appended
    E_ext = np.vstack([np64(inp["E"]), np.zeros((1, 128))])
    tm = np.where((t.numpy() >= 0) & (t.numpy() < 5000), t.numpy(), 5000)
    X, P, A = np64(inp["X"]), np64(inp["P"]), np64(inp["A"])
    assert_close(np64(Z), codec.compress(X, tm, E_ext, P, A), BF16_TOL, "Z")
    assert_close(np64(Xh), codec.reconstruct(np64(Z), tm, E_ext, P, A), BF16_TOL, "Xhat")


def test_empty_batch_leaves_outputs_alone():
    inp = synth.codec_inputs(25, 64, 1024, 128, 100, "bf16")
    g = to_dev(inp)
    Z = torch.full((0, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    out = lac.mapl_compress(g["X"][:0], g["tids"][:0], g["E"], g["P"], g["A"], Z=Z)
    assert out.shape == (0, 128)
    gA = torch.full((1024, 128), 3.0, device=DEV)
    lac.mapl_reconstruct_bwd(g["gXhat"][:0], g["X"][:0, :128].contiguous(), g["A"], gA=gA, accumulate=True)
    torch.cuda.synchronize()
    assert bool((gA == 3.0).all())


# --------------------------------------------------- full-size workloads --

def _full(name, r=None):
    c = synth.CONFIGS[name]
    N = c["B"] * c["T"]
    return synth.codec_inputs(c["seed"], N, c["d"], r or c["r"], c["V"], c["dtype"], x_kind=c.get("x_kind", "gauss"))


@pytest.mark.parametrize("name,r", [("150m", None), ("sweep", 64), ("sweep", 256), ("sweep", 512), ("1b", None)])
def test_full_size_codec_and_backward(name, r):
    inp = _full(name, r)
    g = to_dev(inp)
    pk = lac.mapl_pack(g["P"], g["A"])
    Z, Xh = run_forward(g, pk=pk, pk_ready=True)
    check_forward(inp, Z, Xh, BF16_TOL)
    check_backward(inp, g, BF16_TOL, Z)
