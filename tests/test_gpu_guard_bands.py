"""Canary guard bands: every output of every entry point is written into the
front of a larger buffer whose tail holds a known bit pattern; after the call
the tail must be unchanged (no kernel writes past the end of its output, at
ragged token counts and at the workload shapes).  Inputs are seeded synthetic
boundaries (Section 3.2, 3.3 and 3.5 shapes)."""
import numpy as np
import pytest
import torch

import learned_activation_compression_amd as lac
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
GUARD = 4096  # elements of canary after each output


def guarded(shape, dtype):
    """(view, buffer): a contiguous view of `shape` at the front of a buffer
    with GUARD extra elements of canary after it."""
    n = int(np.prod(shape))
    esz = torch.tensor([], dtype=dtype).element_size()
    raw = torch.full(((n + GUARD) * esz,), 0xA5, dtype=torch.uint8, device=DEV)
    buf = raw.view(dtype)
    return buf[:n].view(*shape), raw


def tail_ok(raw, n_elems, dtype):
    esz = torch.tensor([], dtype=dtype).element_size()
    return bool((raw[n_elems * esz:] == 0xA5).all())


@pytest.mark.parametrize("N,d,r", [(16384, 1024, 128), (333, 512, 64), (1000, 1024, 256), (517, 1024, 512)])
def test_codec_outputs_stay_inside_their_buffers(N, d, r):
    inp = synth.codec_inputs(90 + r, N, d, r, 3000, "bf16")
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    Z, rz = guarded((N, r), torch.bfloat16)
    Xh, rx = guarded((N, d), torch.bfloat16)
    gZ, rgz = guarded((N, r), torch.bfloat16)
    gX, rgx = guarded((N, d), torch.bfloat16)
    gA, rga = guarded((d, r), torch.float32)
    pkn = lac.mapl_pack_bytes(d, r)
    pk, rpk = guarded((pkn,), torch.uint8)
    lac.mapl_pack(g["P"], g["A"], pk=pk)
    lac.mapl_compress(g["X"], g["tids"], g["E"], g["P"], g["A"], Z=Z, pk=pk, pk_ready=True)
    lac.mapl_reconstruct(Z, g["tids"], g["E"], g["P"], g["A"], Xhat=Xh, pk=pk, pk_ready=True)
    lac.mapl_reconstruct_bwd(g["gXhat"], Z, g["A"], gZ=gZ, gA=gA, pk=pk, pk_ready=True)
    lac.mapl_compress_bwd(gZ, g["X"], g["tids"], g["E"], g["P"], g["A"], gX=gX, gA=gA, accumulate=True, pk=pk,
                          pk_ready=True)
    V = inp["V"]
    gE, rge = guarded((V, r), torch.float32)
    lac.mapl_anchor_grad(gX, g["tids"], g["P"], V, -1.0, gE=gE, pk=pk, pk_ready=True, r=r)
    torch.cuda.synchronize()
    for name, raw, n, dt in (("Z", rz, N * r, torch.bfloat16), ("Xhat", rx, N * d, torch.bfloat16),
                             ("gZ", rgz, N * r, torch.bfloat16), ("gX", rgx, N * d, torch.bfloat16),
                             ("gA", rga, d * r, torch.float32), ("pack", rpk, pkn, torch.uint8),
                             ("gE", rge, V * r, torch.float32)):
        assert tail_ok(raw, n, dt), f"{name} written past its end"
    assert torch.isfinite(Xh).all() and torch.isfinite(gA).all()


@pytest.mark.parametrize("N,w,K", [(16384, 32, 256), (999, 2, 256), (700, 8, 17)])
def test_rvq_outputs_stay_inside_their_buffers(N, w, K):
    G, R = 256 // w, 2
    rng = np.random.default_rng(N + w)
    Z = torch.from_numpy(rng.standard_normal((N, 256)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    C = torch.from_numpy((rng.standard_normal((R, G, K, w)) / np.sqrt(w)).astype(np.float32)).to(DEV)
    codes, rc = guarded((N, R, G), torch.uint8)
    lac.rvq_encode(Z, C, G, K, R, round_stride=256 * K, codes=codes)
    Zq, rq = guarded((N, 256), torch.float32)
    lac.rvq_decode(codes, C, G, K, R, 256, round_stride=256 * K, Zq=Zq)
    Cs, rcs = guarded((R, G, K, w), torch.float32)
    Cs.copy_(C)
    idx = torch.tensor([0, 5, R * G * K - 1], dtype=torch.int32, device=DEV)
    lac.rvq_stream_apply(Cs, idx, torch.ones((3, w), device=DEV))
    Zf, rf = guarded((N, 256), torch.bfloat16)
    Cf, rcf = guarded((R, G, K, w), torch.float32)
    Cf.copy_(C)
    lac.rvq_stream_decode(Cf, idx, torch.ones((3, w), device=DEV), codes, G, K, R, 256, round_stride=256 * K, Zq=Zf)
    torch.cuda.synchronize()
    assert tail_ok(rc, N * R * G, torch.uint8)
    assert tail_ok(rq, N * 256, torch.float32)
    assert tail_ok(rcs, R * G * K * w, torch.float32)
    assert tail_ok(rf, N * 256, torch.bfloat16)
    assert tail_ok(rcf, R * G * K * w, torch.float32)


@pytest.mark.parametrize("d,r", [(1024, 128), (2048, 256), (96, 96)])
def test_spel_outputs_and_workspace_stay_inside_their_buffers(d, r):
    inp = synth.spel_inputs(95, d, r, 1e-3)
    A, ra = guarded((d, r), torch.float32)
    m, rm = guarded((d, r), torch.float32)
    D, rd = guarded((d, r), torch.float32)
    A.copy_(inp["A"])
    m.copy_(inp["m"])
    nws = lac.spel_workspace_bytes(d, r)
    ws, rws = guarded((nws,), torch.uint8)
    st, rst = guarded((1,), torch.int32)
    lac.spel_step(A, inp["g"].to(DEV), m, 1e-3, 0.9, 8, D_out=D, status=st, ws=ws)
    torch.cuda.synchronize()
    for name, raw, n, dt in (("A", ra, d * r, torch.float32), ("m", rm, d * r, torch.float32),
                             ("D", rd, d * r, torch.float32), ("ws", rws, nws, torch.uint8),
                             ("status", rst, 1, torch.int32)):
        assert tail_ok(raw, n, dt), f"{name} written past its end"
    assert int(st.item()) == 0
