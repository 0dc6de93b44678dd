"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/mapl.h declares, and its host validation returns the documented status
codes before anything is enqueued.  No call here reaches a kernel launch, so
these run without a GPU: calls that pass validation stop at the device set-up
(raising the kernels' LDS limits), which reports MAPL_ERR_HIP when there is no
device -- the path a refused limit takes on a GPU."""
import ctypes

import numpy as np

import pytest

import learned_activation_compression_amd as lac

OK, ENULL, ESHAPE, EDTYPE, EARG, EWS, EHIP, ETID = 0, -1, -2, -3, -4, -5, -6, -7
F32, BF16 = lac.MAPL_F32, lac.MAPL_BF16
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    return lac.load()


def test_library_exports_every_declared_symbol(lib):
    names = lac.exported_symbols()
    assert len(names) == 23, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(lac._SIGS), set(names) ^ set(lac._SIGS)


def test_status_strings_and_version(lib):
    for s in (OK, ENULL, ESHAPE, EDTYPE, EARG, EWS, EHIP, ETID):
        assert lib.mapl_status_string(s) != b"unknown status"
    assert b"token id" in lib.mapl_status_string(ETID)
    assert lib.mapl_status_string(-99) == b"unknown status"
    assert lib.mapl_version().startswith(b"mapl-gfx950")


def test_pack_and_workspace_sizes(lib):
    d, r = 1024, 128
    want = 4 * 2 * r * d + 2 * r * r
    got = lib.mapl_pack_bytes(d, r, r, BF16)
    assert want <= got <= want + 5 * 256
    # no anchor: only the two A sections
    assert 2 * 2 * r * d <= lib.mapl_pack_bytes(d, r, 0, BF16) <= 2 * 2 * r * d + 5 * 256
    # anchor rank 256 beside r = 128: P sections d x 256, Q sections r x 256
    want = 2 * 2 * r * d + 2 * 2 * 256 * d + 2 * r * 256
    assert want <= lib.mapl_pack_bytes(d, r, 256, BF16) <= want + 5 * 256
    assert lib.mapl_pack_bytes(d, r, r, F32) == 0
    assert lib.mapl_pack_bytes(d, r, 96, BF16) == 0                      # anchor rank not a multiple of 64
    assert lib.mapl_pack_bytes(d, r, d + 128, BF16) == 0                 # anchor rank above d
    assert lib.mapl_bwd_workspace_bytes(8, 2048, d, r, r, BF16) > 0
    assert lib.mapl_bwd_workspace_bytes(8, 2048, d, r, 0, BF16) < lib.mapl_bwd_workspace_bytes(8, 2048, d, r, d, BF16)
    assert lib.mapl_bwd_workspace_bytes(1, 128, 256, 32, 32, F32) == 128 * 256 * 4
    assert lib.mapl_bwd_workspace_bytes(1, 128, 1000, 32, 32, BF16) == 0     # d % 64 != 0
    assert lib.spel_workspace_bytes(2048, 256) >= 4 * 2048 * 256 * 4    # 3 iterates + the uncommitted momentum
    assert lib.spel_workspace_bytes(2048, 250) == 0                      # r % 32 != 0


def _compress(lib, **kw):
    a = dict(X=FAKE, tids=FAKE, E=FAKE, P=FAKE, A=FAKE, Z=FAKE, B=8, T=2048, d=1024, r=128, ra=128, V=32000,
             dt=BF16, pk=FAKE, pk_bytes=10 ** 7, pk_ready=1, s=None)
    a.update(kw)
    return lib.mapl_compress(a["X"], a["tids"], a["E"], a["P"], a["A"], a["Z"], a["B"], a["T"], a["d"], a["r"],
                             a["ra"], a["V"], a["dt"], a["pk"], a["pk_bytes"], a["pk_ready"], a["s"])


def test_compress_kernel_timing_arming(lib):
    # exactly one event is an error; both NULL disarm
    assert lib.mapl_time_next_compress_kernel(FAKE, None) == ENULL
    assert lib.mapl_time_next_compress_kernel(None, FAKE) == ENULL
    assert lib.mapl_time_next_compress_kernel(None, None) == OK
    # an armed call that cannot be timed fails before any validation or launch ...
    for bad in (dict(dt=F32), dict(r=512), dict(B=0)):
        assert lib.mapl_time_next_compress_kernel(FAKE, FAKE) == OK
        assert _compress(lib, **bad) == EARG
        # ... and takes the arming: the same call disarmed reaches its own validation
        assert _compress(lib, **bad, X=None) in (ENULL, OK)
    # a failing call also takes the arming: the next one validates normally
    assert lib.mapl_time_next_compress_kernel(FAKE, FAKE) == OK
    assert _compress(lib, X=None) == ENULL
    assert _compress(lib, d=1000) == ESHAPE
    # disarming before the call leaves it unaffected
    assert lib.mapl_time_next_compress_kernel(FAKE, FAKE) == OK
    assert lib.mapl_time_next_compress_kernel(None, None) == OK
    assert _compress(lib, dt=F32, X=None) == ENULL


def test_compress_validation(lib):
    assert _compress(lib, X=None) == ENULL
    assert _compress(lib, tids=None) == ENULL
    assert _compress(lib, pk=None) == ENULL
    assert _compress(lib, pk_bytes=100) == EWS
    assert _compress(lib, d=1000) == ESHAPE          # bf16 needs d % 128 == 0
    assert _compress(lib, d=320) == ESHAPE
    assert _compress(lib, r=96) == ESHAPE            # bf16 needs r a power of two
    assert _compress(lib, r=100) == ESHAPE           # bf16 needs r % 32 == 0
    assert _compress(lib, r=2048) == ESHAPE          # r > d
    assert _compress(lib, r=1024, d=1024) == ESHAPE  # bf16 r <= 512
    assert _compress(lib, V=0) == ESHAPE
    assert _compress(lib, B=-1) == ESHAPE
    assert _compress(lib, dt=7) == EDTYPE
    assert _compress(lib, pk_ready=2) == EARG
    assert _compress(lib, dt=F32, d=8192, r=64, pk=None, pk_bytes=0) == ESHAPE  # fp32 d <= 4096
    # anchor rank
    assert _compress(lib, ra=-1) == ESHAPE
    assert _compress(lib, ra=2048) == ESHAPE         # ra > d
    assert _compress(lib, ra=96) == ESHAPE           # bf16: ra != r streams in 64-wide chunks
    assert _compress(lib, r=32, ra=64) == ESHAPE     # ... and needs r % 64 == 0
    assert _compress(lib, ra=0, tids=None, E=None, P=None, V=0, B=0) == OK    # no anchor: no table needed
    assert _compress(lib, ra=0, X=None, tids=None, E=None, P=None, V=0) == ENULL
    assert _compress(lib, ra=1024, B=0) == OK        # full anchor
    assert _compress(lib, dt=F32, ra=100, pk=None, pk_bytes=0, B=0) == OK
    # P = NULL stands for the identity only with the full-rank anchor (ra == d)
    assert _compress(lib, ra=1024, P=None, B=0) == OK
    assert _compress(lib, ra=128, P=None) == ENULL
    assert _compress(lib, ra=1024, E=None, P=None) == ENULL


def test_empty_batch_is_a_no_op(lib):
    # N = 0 passes validation and returns before any launch
    assert _compress(lib, B=0) == OK
    assert lib.mapl_reconstruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2048, 1024, 128, 128, 32000, BF16, FAKE,
                                10 ** 7, 1, None) == OK
    assert lib.rvq_encode(FAKE, BF16, FAKE, 0, FAKE, 0, 256, 8, 256, 2, None) == OK
    assert lib.rvq_decode(FAKE, FAKE, 0, FAKE, F32, 0, 256, 8, 256, 2, None) == OK
    assert lib.rvq_stream_apply(FAKE, FAKE, FAKE, 0, 256, 8, 256, 1, None) == OK
    assert lib.rvq_stream_decode(FAKE, 0, 1, FAKE, FAKE, 0, FAKE, FAKE, F32, 0, 256, 8, 256, 2, None) == OK


def test_backward_validation(lib):
    ws = lib.mapl_bwd_workspace_bytes(8, 2048, 1024, 128, 0, BF16)   # the receiver's map has no anchor term
    f = lib.mapl_reconstruct_bwd
    assert f(None, FAKE, FAKE, FAKE, FAKE, 0, 8, 2048, 1024, 128, BF16, FAKE, 10 ** 7, 1, FAKE, ws, None) == ENULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 2048, 1024, 128, BF16, FAKE, 10 ** 7, 1, FAKE, ws - 4, None) == EWS
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 2048, 1024, 128, BF16, FAKE, 10 ** 7, 1, None, ws, None) == ENULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2048, 1024, 128, BF16, FAKE, 10 ** 7, 1, FAKE, ws, None) == EARG
    ws = lib.mapl_bwd_workspace_bytes(8, 2048, 1024, 128, 128, BF16)
    g = lib.mapl_compress_bwd
    pk = 10 ** 7

    def gc(gZ=FAKE, X=FAKE, tids=FAKE, E=FAKE, P=FAKE, A=FAKE, gX=FAKE, gA=FAKE, acc=0, B=8, T=2048, d=1024, r=128,
           ra=128, V=32000, dt=BF16, pk=FAKE, pkb=pk, pkr=1, w=FAKE, wb=ws):
        return g(gZ, X, tids, E, P, A, gX, gA, acc, B, T, d, r, ra, V, dt, pk, pkb, pkr, w, wb, None)

    assert gc(gA=None) == ENULL
    assert gc(wb=16) == EWS
    assert gc(pk=None) == ENULL
    assert gc(d=1000) == ESHAPE
    assert gc(tids=None) == ENULL
    assert gc(ra=256, wb=ws) == EWS                  # a wider anchor needs a larger workspace
    assert gc(ra=0, tids=None, E=None, P=None, V=0, B=0, acc=1) == OK   # empty, accumulate: nothing to do


def test_anchor_grad_validation(lib):
    ws = lib.mapl_anchor_grad_workspace_bytes(8, 2048, 128, 32000)
    N = 8 * 2048
    assert N * 128 * 4 <= ws <= N * 128 * 4 + 2 ** 17   # U rows + partial maxima
    assert lib.mapl_anchor_grad_workspace_bytes(8, 2048, 128, 0) == 0
    assert lib.mapl_anchor_grad_workspace_bytes(8, 2048, 128, 2 ** 22 + 1) == 0
    f = lib.mapl_anchor_grad

    def call(Y=FAKE, tids=FAKE, P=FAKE, gE=FAKE, alpha=1.0, acc=0, B=8, T=2048, d=1024, r=128, ra=128, V=32000,
             dt=BF16, pk=FAKE, pkb=10 ** 7, pkr=1, w=FAKE, wb=ws):
        return f(Y, tids, P, gE, alpha, acc, B, T, d, r, ra, V, dt, pk, pkb, pkr, w, wb, None)

    assert call(Y=None) == ENULL
    assert call(tids=None) == ENULL
    assert call(gE=None) == ENULL
    assert call(w=None) == ENULL
    assert call(wb=ws - 8) == EWS
    assert call(w=ctypes.c_void_p(0x1008)) == EARG              # ws not 16-B aligned
    assert call(acc=2) == EARG
    assert call(pkr=3) == EARG
    assert call(pk=None) == ENULL                               # bf16 needs the pack
    assert call(pkb=1000) == EWS
    assert call(alpha=float("inf")) == EARG
    assert call(d=1000) == ESHAPE                               # bf16 d % 128
    assert call(r=96) == ESHAPE                                 # bf16 r a power of two
    assert call(V=0) == ESHAPE
    assert call(V=2 ** 22 + 1) == ESHAPE                        # owner blocks scale with V
    assert call(B=1, T=2 ** 24) == ESHAPE                       # token indices take 24 bits
    assert call(dt=4) == EDTYPE
    assert call(ra=0) == ESHAPE                                 # no anchor, no table
    assert call(ra=2048) == ESHAPE
    assert call(ra=256) == EWS                                  # the workspace holds N x ra rows
    assert call(P=None) == ENULL                                # P = NULL only for ra == d
    wsd = lib.mapl_anchor_grad_workspace_bytes(8, 2048, 1024, 32000)
    assert call(ra=1024, P=None, pk=None, w=None, wb=wsd) == ENULL   # the identity reads no pack, but needs ws
    assert call(B=0, acc=1, Y=None, tids=None, P=None, w=None) == OK   # empty batch, accumulate: nothing to do


def test_rvq_validation(lib):
    e = lib.rvq_encode
    assert e(None, BF16, FAKE, 0, FAKE, 16384, 256, 8, 256, 2, None) == ENULL
    assert e(FAKE, BF16, FAKE, 0, FAKE, 16384, 256, 7, 256, 2, None) == ESHAPE   # r % G
    assert e(FAKE, BF16, FAKE, 0, FAKE, 16384, 256, 8, 512, 2, None) == ESHAPE   # K > 256 (uint8 codes)
    assert e(FAKE, BF16, FAKE, 0, FAKE, 16384, 256, 8, 0, 2, None) == ESHAPE     # K >= 1
    assert e(FAKE, BF16, FAKE, 0, FAKE, 16384, 384, 3, 256, 2, None) == ESHAPE   # w = 128 unsupported
    assert e(FAKE, BF16, FAKE, 0, FAKE, 16384, 256, 8, 256, 0, None) == ESHAPE   # R >= 1
    assert e(FAKE, BF16, FAKE, 100, FAKE, 16384, 256, 8, 256, 2, None) == EARG   # 0 < stride < r*K
    assert e(FAKE, 5, FAKE, 0, FAKE, 16384, 256, 8, 256, 2, None) == EDTYPE
    odd = ctypes.c_void_p(0x1004)
    assert e(odd, BF16, FAKE, 0, FAKE, 16384, 256, 8, 256, 2, None) == EARG    # Z not 16-B aligned
    assert e(FAKE, BF16, odd, 0, FAKE, 16384, 256, 8, 256, 2, None) == EARG    # C not 16-B aligned
    assert e(FAKE, BF16, FAKE, 256 * 256 + 2, FAKE, 16384, 256, 8, 256, 2, None) == EARG  # stride % 4
    assert lib.rvq_decode(FAKE, odd, 0, FAKE, F32, 16384, 256, 8, 256, 2, None) == EARG
    d = lib.rvq_decode
    assert d(FAKE, FAKE, 0, None, F32, 16384, 256, 8, 256, 2, None) == ENULL
    assert d(FAKE, FAKE, 0, FAKE, 9, 16384, 256, 8, 256, 2, None) == EDTYPE
    s = lib.rvq_stream_apply
    assert s(None, FAKE, FAKE, 8, 256, 8, 256, 1, None) == ENULL
    assert s(FAKE, FAKE, FAKE, 8, 250, 8, 256, 1, None) == ESHAPE
    sd = lib.rvq_stream_decode
    assert sd(None, 0, 1, FAKE, FAKE, 8, FAKE, FAKE, F32, 16384, 256, 8, 256, 2, None) == ENULL
    assert sd(FAKE, 0, 1, None, FAKE, 8, FAKE, FAKE, F32, 16384, 256, 8, 256, 2, None) == ENULL   # n > 0 needs idx
    assert sd(FAKE, 0, 1, FAKE, FAKE, 8, FAKE, None, F32, 16384, 256, 8, 256, 2, None) == ENULL
    assert sd(FAKE, 0, 1, FAKE, FAKE, -1, FAKE, FAKE, F32, 16384, 256, 8, 256, 2, None) == ESHAPE
    assert sd(FAKE, 0, 0, FAKE, FAKE, 8, FAKE, FAKE, F32, 16384, 256, 8, 256, 2, None) == ESHAPE   # R_c >= 1
    assert sd(FAKE, 0, 1, FAKE, FAKE, 8, FAKE, FAKE, F32, 16384, 250, 8, 256, 2, None) == ESHAPE
    assert sd(FAKE, 100, 1, FAKE, FAKE, 8, FAKE, FAKE, F32, 16384, 256, 8, 256, 2, None) == EARG  # 0 < stride < r*K
    assert sd(odd, 0, 1, FAKE, FAKE, 8, FAKE, FAKE, F32, 16384, 256, 8, 256, 2, None) == EARG
    assert sd(FAKE, 0, 1, FAKE, FAKE, 8, FAKE, FAKE, 9, 16384, 256, 8, 256, 2, None) == EDTYPE


def test_spel_validation(lib):
    ws = lib.spel_workspace_bytes(2048, 256)
    f = lib.spel_step
    assert f(FAKE, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 2048, 256, FAKE, ws - 1, None) == EWS
    assert f(FAKE, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 2048, 256, None, ws, None) == ENULL
    assert f(None, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 2048, 256, FAKE, ws, None) == ENULL
    assert f(FAKE, FAKE, FAKE, 1e-3, 1.0, 8, None, None, 2048, 256, FAKE, ws, None) == EARG     # beta < 1
    assert f(FAKE, FAKE, FAKE, 0.9, 0.9, 8, None, None, 2048, 256, FAKE, ws, None) == EARG      # alpha <= 0.7
    assert f(FAKE, FAKE, FAKE, float("nan"), 0.9, 8, None, None, 2048, 256, FAKE, ws, None) == EARG
    assert f(FAKE, FAKE, FAKE, 1e-3, 0.9, 0, None, None, 2048, 256, FAKE, ws, None) == EARG     # ns_iters >= 1
    assert f(FAKE, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 2048, 250, FAKE, ws, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 256, 512, FAKE, ws, None) == ESHAPE    # r > d
    odd = ctypes.c_void_p(0x1004)
    assert f(odd, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 2048, 256, FAKE, ws, None) == EARG      # A not 16-B aligned
    assert f(FAKE, FAKE, odd, 1e-3, 0.9, 8, None, None, 2048, 256, FAKE, ws, None) == EARG      # m not 16-B aligned
    assert f(FAKE, FAKE, FAKE, 1e-3, 0.9, 8, None, ctypes.c_void_p(0x1002), 2048, 256, FAKE, ws,
             None) == EARG                                                                     # status 4-B aligned


def test_spel_step_static_validation(lib):
    f = lib.spel_step_static
    assert f(None, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 1024, 128, None) == ENULL
    assert f(FAKE, FAKE, FAKE, 1e-3, 1.0, 8, None, None, 1024, 128, None) == EARG      # beta < 1
    assert f(FAKE, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 1024, 100, None) == ESHAPE    # r % 32
    assert f(FAKE, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 4096, 256, None) == EWS       # beyond the 16 MiB scratch
    assert f(ctypes.c_void_p(0x1004), FAKE, FAKE, 1e-3, 0.9, 8, None, None, 1024, 128, None) == EARG


def test_spel_polar_express_validation(lib):
    ws = lib.spel_workspace_bytes(1024, 128)
    f = lib.spel_step_polar_express

    def call(A=FAKE, m=FAKE, alpha=1e-3, beta=0.9, lmo=5, ret=7, ell=1e-3, d=1024, r=128, w=FAKE, wb=ws):
        return f(A, FAKE, m, alpha, beta, lmo, ret, ell, None, None, d, r, w, wb, None)

    assert call(A=None) == ENULL
    assert call(w=None) == ENULL
    assert call(wb=ws - 4) == EWS
    assert call(lmo=0) == EARG
    assert call(ret=33) == EARG
    assert call(ell=0.0) == EARG
    assert call(ell=1.0) == EARG
    assert call(ell=float("nan")) == EARG
    assert call(beta=1.0) == EARG
    assert call(r=100) == ESHAPE
    assert call(m=ctypes.c_void_p(0x1004)) == EARG
    g = lib.spel_polar_express_coefficients
    buf = (ctypes.c_double * 96)()
    assert g(1e-3, 5, None, None) == ENULL
    assert g(0.0, 5, buf, None) == EARG
    assert g(1e-3, 0, buf, None) == EARG
    assert g(1e-3, 33, buf, None) == EARG
    assert g(1e-3, 32, buf, None) == OK


def test_polar_express_schedule_host_matches_oracle():
    """The library's host-side schedule (C++ Remez) against the oracle's
    (NumPy Remez): two implementations of the same minimax steps."""
    from oracle import spel
    for ell in (1e-3, 0.05, 0.5):
        c, e = lac.spel_polar_express_coefficients(ell, 9)
        co, eo = spel.polar_express_coefficients(ell, 9)
        np.testing.assert_allclose(c, np.array(co), rtol=0, atol=1e-8)
        np.testing.assert_allclose(e, np.array(eo), rtol=1e-6, atol=1e-13)


def test_check_tids_validation(lib):
    assert lib.mapl_check_tids(FAKE, 10, 0, FAKE, None) == ESHAPE
    assert lib.mapl_check_tids(FAKE, 10, 5, None, None) == ENULL


def test_binding_rejects_host_tensors():
    import torch
    X = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(lac.MaplError):
        lac.mapl_compress(X, torch.zeros(4, dtype=torch.int32), torch.zeros(8, 32, dtype=torch.bfloat16),
                          torch.zeros(32, 64, dtype=torch.bfloat16), torch.zeros(64, 32, dtype=torch.bfloat16))


def test_valid_calls_without_a_device_stop_at_device_setup(lib):
    """A call that passes validation first prepares the device (the kernels'
    dynamic-LDS limits); with no device that fails, and the call returns
    MAPL_ERR_HIP having enqueued nothing -- the same path as a limit the
    runtime refuses.  mapl_init reports the same."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present: the set-up succeeds")
    assert lib.mapl_init() == EHIP
    assert _compress(lib) == EHIP
    ws = lib.spel_workspace_bytes(1024, 128)
    assert lib.spel_step(FAKE, FAKE, FAKE, 1e-3, 0.9, 8, None, None, 1024, 128, FAKE, ws, None) == EHIP
    assert lib.rvq_encode(FAKE, BF16, FAKE, 0, FAKE, 16384, 256, 128, 17, 2, None) == EHIP   # K = 17 is valid
    assert lib.rvq_stream_apply(FAKE, FAKE, FAKE, 8, 256, 8, 256, 1, None) == EHIP
    assert lib.rvq_stream_decode(FAKE, 0, 1, FAKE, FAKE, 8, FAKE, FAKE, F32, 16384, 256, 8, 256, 2, None) == EHIP


def test_tid_check_mode_of_the_binding(monkeypatch):
    """MAPL_CHECK=1 makes the binding count out-of-range ids before a map that
    reads them (mapl_check_tids) and raise MAPL_ERR_TID; without it no count
    is taken.  Checked here through the binding's own switch."""
    monkeypatch.setenv("MAPL_CHECK", "1")
    assert lac._checking()
    monkeypatch.setenv("MAPL_CHECK", "0")
    assert not lac._checking()
    monkeypatch.delenv("MAPL_CHECK")
    assert not lac._checking()
