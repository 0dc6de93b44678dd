"""GPU parity of the residual multi-codebook VQ (Section 3.5) and the streaming
codebook sync (Appendix F) against the fp64 oracle, through the C ABI.

Codes must equal the oracle's argmin except where the oracle's top-2 distance
gap is below 1e-6 relative to the smallest distance; each round is judged
teacher-forced on the GPU's own codes of earlier rounds, and every token is
checked.  Decoding in fp32 is within 1e-5 relative L2; stream sync is
bit-exact."""
import math

import numpy as np
import pytest
import torch

import learned_activation_compression_amd as lac
import synth
from oracle import rvq
from parity_util import BF16_TOL, F32_TOL, assert_close, check_codes, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def encode_and_check(Z: torch.Tensor, C: torch.Tensor, G, K, R, what):
    R_c = C.shape[0]
    r = Z.shape[1]
    stride = 0 if R_c == 1 else r * K
    codes = lac.rvq_encode(Z, C, G, K, R, round_stride=stride)
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    ora = rvq.encode(np64(Z), np64(C), G, K, R, teacher=gc)
    n_mis = check_codes(gc, ora, what)
    return codes, ora, n_mis, stride


@pytest.mark.parametrize("R_c", [1, 2])
def test_rvq_config_full_size(R_c):
    c = synth.CONFIGS["rvq"]
    N = c["B"] * c["T"]
    inp = synth.codec_inputs(c["seed"], N, c["d"], c["r"], c["V"], "bf16", with_grad=False)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    C = synth.rvq_codebooks(c["seed"], R_c, c["G"], c["K"], c["r"] // c["G"], c["codebook_var"]).to(DEV)
    codes, ora, n_mis, stride = encode_and_check(Z, C, c["G"], c["K"], c["R"], f"rvq R_c={R_c}")
    assert n_mis <= 2, n_mis   # the kernel's codes are exact: only ties at fp64 resolution may differ
    # decode in fp32 and bf16
    Zq = lac.rvq_decode(codes, C, c["G"], c["K"], c["R"], c["r"], round_stride=stride)
    Zq16 = lac.rvq_decode(codes, C, c["G"], c["K"], c["R"], c["r"], round_stride=stride, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = rvq.decode(codes.cpu().numpy(), np64(C), c["G"], c["K"], c["R"])
    assert_close(np64(Zq), ref, F32_TOL, "decode fp32")
    assert_close(np64(Zq16), ref, BF16_TOL, "decode bf16")
    # residual energy does not grow in aggregate (progressive refinement)
    e = ora["energy"]
    assert e[1] <= e[0] and e[2] <= e[1]


@pytest.mark.parametrize("G,var", [(8, 1.0 / 32.0), (128, 1.0)])
def test_rvq_of_the_backward_gradient(G, var):
    """Section 3.5 quantizes the backward gradients too: gZ = gXhat A from the
    receiver's backward map at the RVQ workload (r = 256, K = 256, R = 2),
    grouped as configured (G = 8 x w = 32) and as in the paper's Table 1
    (G = 128 x w = 2, 2 rounds: 256 code bytes per token).  Codebooks match
    the scale of gZ (unit variance per entry for w = 2).  Every token of every
    group and round is checked."""
    step = 1
    c = synth.CONFIGS["rvq"]
    N, r, K, R = c["B"] * c["T"], c["r"], c["K"], c["R"]
    inp = synth.codec_inputs(c["seed"], N, c["d"], r, c["V"], "bf16")
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    Z = lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"])
    gZ, _ = lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"])
    C = synth.rvq_codebooks(c["seed"], 1, G, K, r // G, var, sub=1).to(DEV)
    codes = lac.rvq_encode(gZ, C, G, K, R)
    Zq = lac.rvq_decode(codes, C, G, K, R, r)
    torch.cuda.synchronize()
    assert codes.shape == (N, R, G) and codes.dtype == torch.uint8
    if G == 128:
        assert codes[0].numel() == 256  # Table 1's payload per token
    sel = np.arange(0, N, step)
    gc = codes.cpu().numpy()[sel]
    ora = rvq.encode(np64(gZ)[sel], np64(C), G, K, R, teacher=gc)
    n_mis = check_codes(gc, ora, f"gZ G={G}")
    assert n_mis <= 2, n_mis
    ref = rvq.decode(gc, np64(C), G, K, R)
    assert_close(np64(Zq)[sel], ref, F32_TOL, "decode")
    Zq16 = lac.rvq_decode(codes, C, G, K, R, r, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_close(np64(Zq16)[sel], ref, BF16_TOL, "decode bf16")
    e = ora["energy"]
    assert e[1] <= e[0] and e[2] <= e[1]


@pytest.mark.parametrize("w,K,R,R_c,N", [(2, 256, 2, 1, 1000), (4, 64, 3, 3, 333), (8, 32, 1, 1, 70),
                                         (16, 128, 2, 2, 513), (32, 256, 2, 1, 4097), (64, 32, 4, 1, 100)])
def test_rvq_shapes(w, K, R, R_c, N):
    G = 4 if w < 64 else 2
    r = G * w
    rng = np.random.default_rng(w * 1000 + K)
    Z = torch.from_numpy(rng.standard_normal((N, r)).astype(np.float32)).to(DEV)
    C = torch.from_numpy((rng.standard_normal((R_c, G, K, w)) / math.sqrt(w)).astype(np.float32)).to(DEV)
    codes, ora, n_mis, stride = encode_and_check(Z, C, G, K, R, f"w={w} K={K}")
    Zq = lac.rvq_decode(codes, C, G, K, R, r, round_stride=stride)
    torch.cuda.synchronize()
    assert_close(np64(Zq), rvq.decode(codes.cpu().numpy(), np64(C), G, K, R), F32_TOL, "decode")


@pytest.mark.parametrize("w,K", [(2, 1), (2, 5), (2, 255), (4, 17), (8, 33), (16, 100), (32, 1), (32, 47),
                                 (64, 200)])
def test_rvq_codebook_sizes_not_a_multiple_of_32(w, K):
    """1 <= K <= 256 in any size: the kernels pad the codebook to a multiple of
    32 with codewords that never win."""
    G, R, N = 4 if w < 64 else 2, 2, 700
    r = G * w
    rng = np.random.default_rng(w * 1000 + K)
    Z = torch.from_numpy(rng.standard_normal((N, r)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    C = torch.from_numpy((rng.standard_normal((R, G, K, w)) / math.sqrt(w)).astype(np.float32)).to(DEV)
    codes, ora, n_mis, stride = encode_and_check(Z, C, G, K, R, f"w={w} K={K}")
    assert n_mis <= 1
    assert int(codes.max()) < K
    Zq = lac.rvq_decode(codes, C, G, K, R, r, round_stride=stride)
    torch.cuda.synchronize()
    assert_close(np64(Zq), rvq.decode(codes.cpu().numpy(), np64(C), G, K, R), F32_TOL, "decode")


@pytest.mark.parametrize("w", [2, 4])
def test_rvq_decode_of_unaligned_codes(w):
    """Codes starting at an odd byte address take the general decode path and
    give the same values as the aligned (vector) path."""
    G, K, R, N = 16, 64, 2, 300
    r = G * w
    rng = np.random.default_rng(7 + w)
    C = torch.from_numpy(rng.standard_normal((1, G, K, w)).astype(np.float32)).to(DEV)
    codes = torch.from_numpy(rng.integers(0, K, (N, R, G)).astype(np.uint8)).to(DEV)
    buf = torch.zeros(N * R * G + 1, dtype=torch.uint8, device=DEV)
    buf[1:] = codes.reshape(-1)
    odd = buf[1:].view(N, R, G)
    a = lac.rvq_decode(codes, C, G, K, R, r)
    b = lac.rvq_decode(odd, C, G, K, R, r)
    torch.cuda.synchronize()
    assert odd.data_ptr() % 2 == 1
    assert torch.equal(a, b)
    assert_close(np64(a), rvq.decode(codes.cpu().numpy(), np64(C), G, K, R), F32_TOL, "decode")


@pytest.mark.parametrize("w,R,R_c", [(2, 6, 1), (4, 5, 5), (2, 4, 4), (8, 6, 6), (32, 5, 1)])
def test_rvq_decode_many_rounds_and_codes_out_of_range(w, R, R_c):
    """More rounds than the narrow decode reads in one batch (four), so a partial
    second batch, and codes >= K, which add nothing: the expected rows are the
    oracle's sums with each such code pointed at an appended zero codeword."""
    G, K, N = 8, 37, 611
    r = G * w
    rng = np.random.default_rng(w * 10 + R)
    C = torch.from_numpy((rng.standard_normal((R_c, G, K, w)) / math.sqrt(w)).astype(np.float32)).to(DEV)
    codes_np = rng.integers(0, K, size=(N, R, G)).astype(np.uint8)
    bad = rng.random((N, R, G)) < 0.05
    codes_np[bad] = rng.integers(K, 256, size=int(bad.sum())).astype(np.uint8)
    codes = torch.from_numpy(codes_np).to(DEV)
    stride = 0 if R_c == 1 else r * K
    Zq = lac.rvq_decode(codes, C, G, K, R, r, round_stride=stride)
    torch.cuda.synchronize()
    C_ext = np.concatenate([np64(C), np.zeros((R_c, G, 1, w))], axis=2)
    want = rvq.decode(np.minimum(codes_np, K), C_ext, G, K + 1, R)
    assert_close(np64(Zq), want, F32_TOL, "decode")


def test_rvq_codeword_inputs_come_back_exactly():
    rng = np.random.default_rng(5)
    N, G, K, w = 1000, 8, 256, 32
    C = (rng.standard_normal((1, G, K, w)) / math.sqrt(w)).astype(np.float32)
    k_true = rng.integers(0, K, size=(N, G))
    Z = np.concatenate([C[0, g][k_true[:, g]] for g in range(G)], axis=1)
    Zd, Cd = torch.from_numpy(Z).to(DEV), torch.from_numpy(C).to(DEV)
    codes = lac.rvq_encode(Zd, Cd, G, K, 1)
    Zq = lac.rvq_decode(codes, Cd, G, K, 1, G * w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes.cpu().numpy()[:, 0, :], k_true)
    assert torch.equal(Zq, Zd)


def test_rvq_duplicate_codewords_pick_the_lowest_index():
    rng = np.random.default_rng(6)
    N, G, K, w = 512, 2, 64, 16
    C = (rng.standard_normal((1, G, K, w)) / 4).astype(np.float32)
    C[0, :, 40] = C[0, :, 9]      # duplicate pair in different 32-codeword blocks
    C[0, :, 17] = C[0, :, 9]      # and one in the same block
    target = np.concatenate([C[0, g, 9] for g in range(G)])
    Z = (target[None, :] + 1e-3 * rng.standard_normal((N, G * w))).astype(np.float32)
    codes = lac.rvq_encode(torch.from_numpy(Z).to(DEV), torch.from_numpy(C).to(DEV), G, K, 1)
    torch.cuda.synchronize()
    assert np.all(codes.cpu().numpy() == 9)


@pytest.mark.parametrize("w", [8, 32])
def test_rvq_nan_group_gets_code_zero_and_others_unaffected(w):
    rng = np.random.default_rng(7)
    N, G, K = 64, 2, 32
    C = rng.standard_normal((1, G, K, w)).astype(np.float32)
    Z = rng.standard_normal((N, G * w)).astype(np.float32)
    Z[5, :w] = np.nan
    codes = lac.rvq_encode(torch.from_numpy(Z).to(DEV), torch.from_numpy(C).to(DEV), G, K, 1)
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    assert gc[5, 0, 0] == 0
    Z[5, :w] = 0
    ref = rvq.encode(Z, C, G, K, 1)["codes"]
    mask = np.ones_like(gc, dtype=bool)
    mask[5, 0, 0] = False
    assert np.array_equal(gc[mask], ref[mask])


@pytest.mark.parametrize("w", [2, 8, 32])
def test_rvq_nan_codeword_never_wins(w):
    # a codeword with a NaN scores NaN on the matrix cores and is never a candidate
    rng = np.random.default_rng(9)
    N, G, K = 700, 2, 64
    C = (rng.standard_normal((1, G, K, w)) / math.sqrt(w)).astype(np.float32)
    Z = np.concatenate([C[0, g][rng.integers(0, K, N)] for g in range(G)], axis=1)
    Z = (Z + 0.05 * rng.standard_normal(Z.shape)).astype(np.float32)
    C[0, 0, 5, w - 1] = np.nan
    codes = lac.rvq_encode(torch.from_numpy(Z).to(DEV), torch.from_numpy(C).to(DEV), G, K, 1).cpu().numpy()
    assert not np.any(codes[:, 0, 0] == 5)
    Cf = C.copy()
    Cf[0, 0, 5] = 1e6  # the oracle with that codeword out of reach
    ora = rvq.encode(Z.astype(np.float64), Cf.astype(np.float64), G, K, 1, teacher=codes)
    check_codes(codes, ora, "NaN codeword")


def test_rvq_identical_codewords_all_tie_to_index_zero():
    # every codeword equal: all K are within the bf16 bound, all are rescored, the lowest index wins
    rng = np.random.default_rng(10)
    N, G, K, w = 300, 2, 256, 32
    C = np.broadcast_to(rng.standard_normal((1, G, 1, w)).astype(np.float32), (1, G, K, w)).copy()
    Z = rng.standard_normal((N, G * w)).astype(np.float32)
    codes = lac.rvq_encode(torch.from_numpy(Z).to(DEV), torch.from_numpy(C).to(DEV), G, K, 2)
    torch.cuda.synchronize()
    assert np.all(codes.cpu().numpy() == 0)


def test_rvq_repeat_is_bitwise_deterministic():
    rng = np.random.default_rng(8)
    Z = torch.from_numpy(rng.standard_normal((4096, 256)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    C = torch.from_numpy((rng.standard_normal((2, 8, 256, 32)) / math.sqrt(32)).astype(np.float32)).to(DEV)
    a = lac.rvq_encode(Z, C, 8, 256, 2, round_stride=256 * 256)
    b = lac.rvq_encode(Z, C, 8, 256, 2, round_stride=256 * 256)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_stream_apply_is_bit_exact_and_converges_to_the_sender():
    c = synth.CONFIGS["rvq"]
    R_c, G, K, w = 2, c["G"], c["K"], c["r"] // c["G"]
    recv = synth.rvq_codebooks(c["seed"], R_c, G, K, w)
    noise = torch.from_numpy(synth.gaussian(synth.stream(c["seed"], 9), recv.shape, 1e-4).astype(np.float32))
    sender = recv + noise
    C = recv.clone().to(DEV)
    ref = recv.numpy().copy()
    for call in range(3):
        idx, vals = synth.stream_packets(c["seed"], call, sender)
        lac.rvq_stream_apply(C, idx.to(DEV), vals.to(DEV))
        ref = rvq.stream_apply(ref, idx.numpy(), vals.numpy())
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), ref)
    # a full sweep of all codewords (with a duplicate index: the later one wins)
    idx = torch.arange(R_c * G * K, dtype=torch.int32)
    idx = torch.cat([torch.tensor([5], dtype=torch.int32), idx])
    vals = torch.cat([torch.zeros(1, w), sender.reshape(-1, w)])
    lac.rvq_stream_apply(C, idx.to(DEV), vals.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), sender)


def _packet(rng, n, total, w, extra_bad=True):
    idx = rng.integers(0, total, size=n).astype(np.int32)
    if n >= 4:
        idx[1] = idx[0]                    # a duplicate: the later entry wins
        if extra_bad:
            idx[2] = total                 # out of range: skipped
            idx[3] = -7
    vals = rng.standard_normal((n, w)).astype(np.float32)
    return torch.from_numpy(idx).to(DEV), torch.from_numpy(vals).to(DEV)


@pytest.mark.parametrize("N,r,G,K,R,R_c,stride_kind,n,out", [
    (16384, 128, 4, 256, 2, 1, "shared", 4, torch.bfloat16),     # the step's receiver (one launch)
    (1000, 256, 8, 256, 2, 2, "rounds", 16, torch.float32),      # a book per round (one launch)
    (777, 64, 8, 17, 3, 3, "rounds", 64, torch.float32),         # w = 8, the largest fused packet, codes >= K
    (333, 128, 2, 256, 1, 1, "shared", 9, torch.bfloat16),       # w = 64
    (500, 64, 8, 17, 2, 2, "padded", 8, torch.float32),          # round stride not a whole codeword count
    (640, 256, 8, 256, 2, 2, "rounds", 65, torch.float32),       # packet over the fused limit: two launches
    (640, 64, 16, 256, 2, 1, "shared", 8, torch.bfloat16),       # w = 4: two launches
    (1, 128, 4, 256, 2, 1, "shared", 4, torch.float32),          # one token
])
def test_stream_decode_is_the_sync_then_the_decode(N, r, G, K, R, R_c, stride_kind, n, out):
    """rvq_stream_decode gives the bits of rvq_stream_apply followed by rvq_decode: the
    decoded rows and the updated books, duplicates, out-of-range ids and codes >= K
    included, on the single-launch path and on the fallbacks."""
    w = r // G
    rng = np.random.default_rng(N + r + n)
    stride = {"shared": 0, "rounds": G * K * w, "padded": G * K * w + 4}[stride_kind]
    # books held: R_c for a shared book, R with a book per round, one more as room for the padded stride
    nb = {"shared": R_c, "rounds": R, "padded": R + 1}[stride_kind]
    C0 = torch.from_numpy((rng.standard_normal((nb, G, K, w)) / np.sqrt(w)).astype(np.float32)).to(DEV)
    codes = torch.from_numpy(rng.integers(0, 256 if K < 256 else K, size=(N, R, G)).astype(np.uint8)).to(DEV)
    idx, vals = _packet(rng, n, nb * G * K, w)
    Ca, Cb = C0.clone(), C0.clone()
    lac.rvq_stream_apply(Cb, idx, vals)
    ref = lac.rvq_decode(codes, Cb, G, K, R, r, round_stride=stride, out_dtype=out)
    got = lac.rvq_stream_decode(Ca, idx, vals, codes, G, K, R, r, round_stride=stride, out_dtype=out)
    torch.cuda.synchronize()
    assert torch.equal(Ca, Cb)
    assert torch.equal(got, ref)


def test_stream_decode_with_unaligned_values_takes_two_launches():
    N, r, G, K, R, w = 900, 256, 8, 256, 2, 32
    rng = np.random.default_rng(5)
    C0 = torch.from_numpy((rng.standard_normal((1, G, K, w)) / 8).astype(np.float32)).to(DEV)
    codes = torch.from_numpy(rng.integers(0, K, size=(N, R, G)).astype(np.uint8)).to(DEV)
    idx, vals = _packet(rng, 12, G * K, w)
    buf = torch.empty(12 * w + 1, device=DEV)
    odd = buf[1:].view(12, w)
    odd.copy_(vals)
    Ca, Cb = C0.clone(), C0.clone()
    lac.rvq_stream_apply(Cb, idx, vals)
    ref = lac.rvq_decode(codes, Cb, G, K, R, r)
    got = lac.rvq_stream_decode(Ca, idx, odd, codes, G, K, R, r)
    torch.cuda.synchronize()
    assert torch.equal(Ca, Cb) and torch.equal(got, ref)
