"""MAPL pipeline-boundary activation codec for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libmapl.so`` (hand-written HIP, see
``include/mapl.h``).  Each function here has the name of the C entry point it
wraps and does argument marshalling only: shape/dtype checks, output
allocation through torch, device pointers and the current HIP stream.  Every
step of the computation runs in the library's kernels; there is no fallback,
and a missing library raises.

The method is that of "Learned Subspace Compression for Communication-
Efficient Pipeline Parallelism" (MAPL): Eq. (1)-(3) codec, its backward, the
residual VQ of Section 3.5 with the streaming sync of Appendix F, and the SPEL
projector update of Section 3.3.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "MaplError", "LIB_PATH", "load", "exported_symbols", "mapl_init",
    "mapl_pack_bytes", "mapl_pack", "mapl_compress", "mapl_time_next_compress_kernel", "mapl_reconstruct",
    "mapl_bwd_workspace_bytes", "mapl_reconstruct_bwd", "mapl_compress_bwd",
    "mapl_anchor_grad_workspace_bytes", "mapl_anchor_grad", "mapl_check_tids",
    "rvq_encode", "rvq_decode", "rvq_stream_apply", "rvq_stream_decode", "spel_workspace_bytes", "spel_step",
    "spel_step_static", "spel_step_polar_express", "spel_polar_express_coefficients",
    "MAPL_F32", "MAPL_BF16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmapl.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "mapl.h")

MAPL_F32, MAPL_BF16 = 0, 1
MAPL_ERR_TID = -7

_vp, _i64, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float

# (restype, argtypes) per exported symbol, in header order
_SIGS = {
    "mapl_status_string": (ctypes.c_char_p, [_i32]),
    "mapl_version": (ctypes.c_char_p, []),
    "mapl_init": (_i32, []),
    "mapl_pack_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "mapl_pack": (_i32, [_vp, _vp, _vp, _sz, _i64, _i64, _i64, _i32, _vp]),
    "mapl_time_next_compress_kernel": (_i32, [_vp, _vp]),
    "mapl_compress": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _vp, _sz, _i32,
                             _vp]),
    "mapl_reconstruct": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _vp, _sz,
                                _i32, _vp]),
    "mapl_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i32]),
    "mapl_reconstruct_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _i32, _vp, _sz, _i32,
                                    _vp, _sz, _vp]),
    "mapl_compress_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64,
                                 _i32, _vp, _sz, _i32, _vp, _sz, _vp]),
    "mapl_anchor_grad_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "mapl_anchor_grad": (_i32, [_vp, _vp, _vp, _vp, _f32, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _vp, _sz,
                                _i32, _vp, _sz, _vp]),
    "mapl_check_tids": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "rvq_encode": (_i32, [_vp, _i32, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _vp]),
    "rvq_decode": (_i32, [_vp, _vp, _i64, _vp, _i32, _i64, _i64, _i64, _i64, _i64, _vp]),
    "rvq_stream_apply": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp]),
    "rvq_stream_decode": (_i32, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _i64, _vp]),
    "spel_workspace_bytes": (_sz, [_i64, _i64]),
    "spel_step": (_i32, [_vp, _vp, _vp, _f32, _f32, _i32, _vp, _vp, _i64, _i64, _vp, _sz, _vp]),
    "spel_step_static": (_i32, [_vp, _vp, _vp, _f32, _f32, _i32, _vp, _vp, _i64, _i64, _vp]),
    "spel_step_polar_express": (_i32, [_vp, _vp, _vp, _f32, _f32, _i32, _i32, _f32, _vp, _vp, _i64, _i64, _vp, _sz,
                                       _vp]),
    "spel_polar_express_coefficients": (_i32, [ctypes.c_double, _i32, _vp, _vp]),
}

_lib = None


class MaplError(RuntimeError):
    """A libmapl entry point returned a negative status, or the binding
    rejected its arguments before the call."""

    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where}: status {status}"
        if _lib is not None and status < 0:
            msg += f" ({_lib.mapl_status_string(status).decode()})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


def load():
    """Load libmapl.so (built in-tree by learned_activation_compression_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MaplError(-100, "load", f"{LIB_PATH} is missing; build it with "
                            "`python -m learned_activation_compression_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols() -> list:
    """Names of the functions declared in include/mapl.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)


# ------------------------------------------------------------- marshalling --

def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MAPL_F32
    if t.dtype == torch.bfloat16:
        return MAPL_BF16
    raise MaplError(-3, "binding", f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise MaplError(-1, "binding", f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise MaplError(-1, "binding", f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MaplError(-2, "binding", f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MaplError(-3, "binding", f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise MaplError(status, where)


def _checking() -> bool:
    """MAPL_CHECK=1 in the environment: count out-of-range token ids on the
    device before every map that reads them, and raise MAPL_ERR_TID."""
    return os.environ.get("MAPL_CHECK", "0") not in ("", "0")


def _check_tids(tids, V: int, where: str, stream=None):
    if tids is None or not _checking():
        return
    bad = mapl_check_tids(tids, V, stream=stream)
    if stream is not None:
        stream.synchronize()
    n_bad = int(bad.item())  # a copy to the host: waits for the count
    if n_bad:
        raise MaplError(MAPL_ERR_TID, where, f"{n_bad} token id(s) outside [0, {V})")


def mapl_init() -> None:
    """Prepare the current device (raise the kernels' dynamic-LDS limits)."""
    _check(load().mapl_init(), "mapl_init")


def _tokens(t: torch.Tensor, width: int, name: str):
    if t.dim() == 3:
        B, T, w = t.shape
    elif t.dim() == 2:
        (B, w), T = t.shape, 1
    else:
        raise MaplError(-2, "binding", f"{name} must be [B, T, {width}] or [N, {width}]")
    if w != width:
        raise MaplError(-2, "binding", f"{name} last dim {w} != {width}")
    return B, T


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _opt(t, name, dtype=None):
    """Device pointer of an optional tensor (None -> NULL)."""
    return None if t is None else _dev(t, name, dtype)


def _ra(E_small) -> int:
    """Anchor rank: E_small is [V, ra]; None means no anchor (ra = 0)."""
    return 0 if E_small is None else int(E_small.shape[1])


# ---------------------------------------------------------------- packing --

def mapl_pack_bytes(d: int, r: int, dtype=torch.bfloat16, ra: int = None) -> int:
    """Pack size for projector rank r and anchor rank ra (default r; 0 = no anchor)."""
    ra = r if ra is None else ra
    return int(load().mapl_pack_bytes(d, r, ra, MAPL_BF16 if dtype == torch.bfloat16 else MAPL_F32))


def _pk(pk, d, r, ra, dt, like):
    nbytes = int(load().mapl_pack_bytes(d, r, ra, dt))
    if nbytes == 0:
        return None, 0
    if pk is None:
        pk = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    return pk, pk.numel() * pk.element_size()


def mapl_pack(P: torch.Tensor, A: torch.Tensor, pk: torch.Tensor = None, stream=None, ra: int = None) -> torch.Tensor:
    """Build the packed weights of (P [ra][d], A [d][r]) into pk (allocated if
    None).  P = None packs for no anchor, or with ra = d for the full-rank
    anchor (P = I)."""
    d, r = A.shape
    if P is not None:
        ra = int(P.shape[0])
    elif ra is None:
        ra = 0
    dt = _dt(A)
    pk, nb = _pk(pk, d, r, ra, dt, A)
    _check(load().mapl_pack(_opt(P, "P", A.dtype), _dev(A, "A"), pk.data_ptr() if pk is not None else None, nb,
                            d, r, ra, dt, _stream(stream)), "mapl_pack")
    return pk


# ------------------------------------------------------------------ codec --

def mapl_compress(X, tids, E_small, P, A, Z=None, pk=None, pk_ready=False, stream=None) -> torch.Tensor:
    """Eq. (1): Z = (X - E_small[tids] P) A.  X is [B,T,d] or [N,d]; E_small
    [V, ra] and P [ra, d] (E_small = P = None: no anchor)."""
    d, r = A.shape
    B, T = _tokens(X, d, "X")
    dt = _dt(X)
    ra = _ra(E_small)
    V = E_small.shape[0] if E_small is not None else 0
    if Z is None:
        Z = _empty((*X.shape[:-1], r), X.dtype, X)
    pk, nb = _pk(pk, d, r, ra, dt, X)
    if ra > 0:
        _check_tids(tids, V, "mapl_compress", stream)
    _check(load().mapl_compress(_dev(X, "X"), _opt(tids, "tids", torch.int32), _opt(E_small, "E_small", X.dtype),
                                _opt(P, "P", X.dtype), _dev(A, "A", X.dtype), _dev(Z, "Z", X.dtype), B, T, d, r, ra,
                                V, dt, pk.data_ptr() if pk is not None else None, nb, int(bool(pk_ready)),
                                _stream(stream)), "mapl_compress")
    return Z


def mapl_time_next_compress_kernel(start=None, stop=None) -> None:
    """Instrumentation: the compress kernel of this thread's next mapl_compress
    call is launched with the torch.cuda.Event objects `start` and `stop`
    (enable_timing=True) as its own begin and end stamps; None, None disarms.
    torch creates an event at its first record(), so each must have been
    recorded once.  The next mapl_compress call takes the arming and fails
    for calls that cannot be timed this way (fp32 data, r >= 512, no tokens)."""
    def raw(e, name):
        if e is None:
            return None
        h = int(e.cuda_event)
        if h == 0:
            raise MaplError(-1, "mapl_time_next_compress_kernel", f"{name} has no event yet (record it once first)")
        return h
    _check(load().mapl_time_next_compress_kernel(raw(start, "start"), raw(stop, "stop")),
           "mapl_time_next_compress_kernel")


def mapl_reconstruct(Z, tids, E_small, P, A, Xhat=None, pk=None, pk_ready=False, stream=None) -> torch.Tensor:
    """Eq. (2): Xhat = Z A^T + E_small[tids] P (receiver's E_small and P; None: no anchor)."""
    d, r = A.shape
    B, T = _tokens(Z, r, "Z")
    dt = _dt(Z)
    ra = _ra(E_small)
    V = E_small.shape[0] if E_small is not None else 0
    if Xhat is None:
        Xhat = _empty((*Z.shape[:-1], d), Z.dtype, Z)
    pk, nb = _pk(pk, d, r, ra, dt, Z)
    if ra > 0:
        _check_tids(tids, V, "mapl_reconstruct", stream)
    _check(load().mapl_reconstruct(_dev(Z, "Z"), _opt(tids, "tids", torch.int32),
                                   _opt(E_small, "E_small", Z.dtype), _opt(P, "P", Z.dtype), _dev(A, "A", Z.dtype),
                                   _dev(Xhat, "Xhat", Z.dtype), B, T, d, r, ra, V, dt,
                                   pk.data_ptr() if pk is not None else None, nb, int(bool(pk_ready)),
                                   _stream(stream)), "mapl_reconstruct")
    return Xhat


def mapl_bwd_workspace_bytes(B: int, T: int, d: int, r: int, dtype=torch.bfloat16, ra: int = None) -> int:
    """Workspace of both backward maps for anchor rank ra (default r)."""
    ra = r if ra is None else ra
    return int(load().mapl_bwd_workspace_bytes(B, T, d, r, ra, MAPL_BF16 if dtype == torch.bfloat16 else MAPL_F32))


def _ws(ws, nbytes, like):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    return ws, ws.numel() * ws.element_size()


def mapl_reconstruct_bwd(gXhat, Z, A, gZ=None, gA=None, accumulate=False, pk=None, pk_ready=False, ws=None,
                         stream=None):
    """gZ = gXhat A ;  gA (+)= gXhat^T Z.  Returns (gZ, gA)."""
    d, r = A.shape
    B, T = _tokens(gXhat, d, "gXhat")
    dt = _dt(gXhat)
    if gZ is None:
        gZ = _empty((*gXhat.shape[:-1], r), gXhat.dtype, gXhat)
    if gA is None:
        gA = torch.zeros((d, r), dtype=torch.float32, device=gXhat.device) if accumulate else \
            _empty((d, r), torch.float32, gXhat)
    pk, nb = _pk(pk, d, r, 0, dt, gXhat)  # the A^T section only
    ws, wb = _ws(ws, int(load().mapl_bwd_workspace_bytes(B, T, d, r, 0, dt)), gXhat)
    _check(load().mapl_reconstruct_bwd(_dev(gXhat, "gXhat"), _dev(Z, "Z", gXhat.dtype), _dev(A, "A", gXhat.dtype),
                                       _dev(gZ, "gZ", gXhat.dtype), _dev(gA, "gA", torch.float32),
                                       int(bool(accumulate)), B, T, d, r, dt,
                                       pk.data_ptr() if pk is not None else None, nb, int(bool(pk_ready)),
                                       ws.data_ptr() if ws is not None else None, wb, _stream(stream)),
           "mapl_reconstruct_bwd")
    return gZ, gA


def mapl_compress_bwd(gZ, X, tids, E_small, P, A, gX=None, gA=None, accumulate=False, pk=None, pk_ready=False,
                      ws=None, stream=None):
    """gX = gZ A^T ;  gA (+)= (X - E_small[tids] P)^T gZ.  Returns (gX, gA).
    E_small = P = None: no anchor."""
    d, r = A.shape
    B, T = _tokens(gZ, r, "gZ")
    dt = _dt(gZ)
    ra = _ra(E_small)
    V = E_small.shape[0] if E_small is not None else 0
    if gX is None:
        gX = _empty((*gZ.shape[:-1], d), gZ.dtype, gZ)
    if gA is None:
        gA = torch.zeros((d, r), dtype=torch.float32, device=gZ.device) if accumulate else \
            _empty((d, r), torch.float32, gZ)
    pk, nb = _pk(pk, d, r, ra, dt, gZ)
    ws, wb = _ws(ws, int(load().mapl_bwd_workspace_bytes(B, T, d, r, ra, dt)), gZ)
    if ra > 0:
        _check_tids(tids, V, "mapl_compress_bwd", stream)
    _check(load().mapl_compress_bwd(_dev(gZ, "gZ"), _dev(X, "X", gZ.dtype), _opt(tids, "tids", torch.int32),
                                    _opt(E_small, "E_small", gZ.dtype), _opt(P, "P", gZ.dtype),
                                    _dev(A, "A", gZ.dtype), _dev(gX, "gX", gZ.dtype), _dev(gA, "gA", torch.float32),
                                    int(bool(accumulate)), B, T, d, r, ra, V, dt,
                                    pk.data_ptr() if pk is not None else None, nb, int(bool(pk_ready)),
                                    ws.data_ptr() if ws is not None else None, wb, _stream(stream)),
           "mapl_compress_bwd")
    return gX, gA


def mapl_anchor_grad_workspace_bytes(B: int, T: int, ra: int, V: int) -> int:
    return int(load().mapl_anchor_grad_workspace_bytes(B, T, ra, V))


def mapl_anchor_grad(Y, tids, P, V: int, alpha: float = 1.0, gE=None, accumulate=False, pk=None, pk_ready=False,
                     r: int = None, ws=None, stream=None):
    """gE [V, ra] fp32 (+)= alpha * scatter-sum over tids of Y P^T (P [ra, d]).

    Receiver's anchor table: Y = gXhat, alpha = +1.  Sender's: Y = gX (the
    gX output of mapl_compress_bwd), alpha = -1.  r is the projector's rank,
    on which the pack layout depends (default ra).  P = None is the full-rank
    anchor (P = I, ra = d; no pack)."""
    d = Y.shape[-1]
    ra = d if P is None else int(P.shape[0])
    if P is not None and P.shape[1] != d:
        raise MaplError(-2, "binding", f"P is {tuple(P.shape)}, Y rows have {d} values")
    r = ra if r is None else r
    B, T = _tokens(Y, d, "Y")
    dt = _dt(Y)
    if gE is None:
        gE = torch.zeros((V, ra), dtype=torch.float32, device=Y.device) if accumulate else \
            _empty((V, ra), torch.float32, Y)
    pk, nb = _pk(pk, d, r, ra, dt, Y) if P is not None else (None, 0)
    ws, wb = _ws(ws, int(load().mapl_anchor_grad_workspace_bytes(B, T, ra, V)), Y)
    _check_tids(tids, V, "mapl_anchor_grad", stream)
    _check(load().mapl_anchor_grad(_dev(Y, "Y"), _dev(tids, "tids", torch.int32), _opt(P, "P", Y.dtype),
                                   _dev(gE, "gE", torch.float32), float(alpha), int(bool(accumulate)), B, T, d, r, ra,
                                   V, dt, pk.data_ptr() if pk is not None else None, nb, int(bool(pk_ready)),
                                   ws.data_ptr() if ws is not None else None, wb, _stream(stream)),
           "mapl_anchor_grad")
    return gE


def mapl_check_tids(tids, V: int, bad=None, stream=None) -> torch.Tensor:
    """Device int32 count of token ids outside [0, V)."""
    if bad is None:
        bad = _empty((1,), torch.int32, tids)
    _check(load().mapl_check_tids(_dev(tids, "tids", torch.int32), tids.numel(), V, _dev(bad, "bad", torch.int32),
                                  _stream(stream)), "mapl_check_tids")
    return bad


# -------------------------------------------------------------------- rvq --

def _check_books(C, r, K, R, round_stride, where):
    need = r * K + (R - 1) * round_stride
    if C.numel() < need:
        raise MaplError(-4, where, f"codebook tensor has {C.numel()} values, {need} needed for R={R} "
                        f"with round stride {round_stride}")


def rvq_encode(Z, C, G: int, K: int, R: int, round_stride: int = 0, codes=None, stream=None) -> torch.Tensor:
    """Residual VQ encode of Z [N][r] -> uint8 codes [N][R][G]."""
    N, r = Z.shape
    _check_books(C, r, K, R, round_stride, "rvq_encode")
    if codes is None:
        codes = _empty((N, R, G), torch.uint8, Z)
    _check(load().rvq_encode(_dev(Z, "Z"), _dt(Z), _dev(C, "C", torch.float32), round_stride,
                             _dev(codes, "codes", torch.uint8), N, r, G, K, R, _stream(stream)), "rvq_encode")
    return codes


def rvq_decode(codes, C, G: int, K: int, R: int, r: int, round_stride: int = 0, out_dtype=torch.float32, Zq=None,
               stream=None) -> torch.Tensor:
    """Residual VQ decode of codes [N][R][G] -> Zq [N][r]."""
    N = codes.shape[0]
    _check_books(C, r, K, R, round_stride, "rvq_decode")
    if Zq is None:
        Zq = _empty((N, r), out_dtype, codes)
    _check(load().rvq_decode(_dev(codes, "codes", torch.uint8), _dev(C, "C", torch.float32), round_stride,
                             _dev(Zq, "Zq"), _dt(Zq), N, r, G, K, R, _stream(stream)), "rvq_decode")
    return Zq


def rvq_stream_apply(C, idx, vals, stream=None) -> torch.Tensor:
    """Overwrite whole codewords of C [R_c][G][K][w] in place; returns C."""
    R_c, G, K, w = C.shape
    n = idx.numel()
    _check(load().rvq_stream_apply(_dev(C, "C", torch.float32), _dev(idx, "idx", torch.int32),
                                   _dev(vals, "vals", torch.float32), n, G * w, G, K, R_c, _stream(stream)),
           "rvq_stream_apply")
    return C


def rvq_stream_decode(C, idx, vals, codes, G: int, K: int, R: int, r: int, round_stride: int = 0,
                      out_dtype=torch.float32, Zq=None, stream=None) -> torch.Tensor:
    """rvq_stream_apply(C, idx, vals) then rvq_decode(codes, C, ...) in one launch for small packets:
    C [R_c][G][K][w] is updated in place and the codes [N][R][G] are decoded with the updated books."""
    N = codes.shape[0]
    R_c = C.shape[0]
    _check_books(C, r, K, R, round_stride, "rvq_stream_decode")
    if Zq is None:
        Zq = _empty((N, r), out_dtype, codes)
    n = idx.numel()
    _check(load().rvq_stream_decode(_dev(C, "C", torch.float32), round_stride, R_c, _dev(idx, "idx", torch.int32),
                                    _dev(vals, "vals", torch.float32), n, _dev(codes, "codes", torch.uint8),
                                    _dev(Zq, "Zq"), _dt(Zq), N, r, G, K, R, _stream(stream)), "rvq_stream_decode")
    return Zq


# ------------------------------------------------------------------- spel --

def spel_workspace_bytes(d: int, r: int) -> int:
    return int(load().spel_workspace_bytes(d, r))


def spel_step(A, g, m, alpha: float, beta: float, ns_iters: int = 8, D_out=None, status=None, ws=None,
              stream=None):
    """One SPEL step on fp32 A [d][r] and momentum m (both in place).
    Returns D_out (the LMO direction) if given, else None.  status: optional
    device int32 [1], set to 0 when the step was applied and to 1 when a wait
    between workgroups timed out (A and m then keep their values)."""
    d, r = A.shape
    ws, wb = _ws(ws, spel_workspace_bytes(d, r), A)
    _check(load().spel_step(_dev(A, "A", torch.float32), _dev(g, "g", torch.float32), _dev(m, "m", torch.float32),
                            float(alpha), float(beta), int(ns_iters),
                            _dev(D_out, "D_out", torch.float32) if D_out is not None else None,
                            _opt(status, "status", torch.int32), d, r,
                            ws.data_ptr() if ws is not None else None, wb, _stream(stream)), "spel_step")
    return D_out


def spel_step_static(A, g, m, alpha: float, beta: float, ns_iters: int = 8, D_out=None, status=None, stream=None):
    """spel_step with its workspace in the library's static device array
    (nothing is allocated: usable under graph capture).  Calls that overlap
    in time on one GPU race; see include/mapl.h."""
    d, r = A.shape
    _check(load().spel_step_static(_dev(A, "A", torch.float32), _dev(g, "g", torch.float32),
                                   _dev(m, "m", torch.float32), float(alpha), float(beta), int(ns_iters),
                                   _dev(D_out, "D_out", torch.float32) if D_out is not None else None,
                                   _opt(status, "status", torch.int32), d, r, _stream(stream)), "spel_step_static")
    return D_out


def spel_step_polar_express(A, g, m, alpha: float, beta: float, lmo_steps: int = 5, ret_steps: int = 7,
                            ell: float = 1e-3, D_out=None, status=None, ws=None, stream=None):
    """One SPEL step with the Polar Express polar map (5 LMO / 7 retraction
    steps by default) on fp32 A [d][r] and m (both in place).  Returns D_out
    if given, else None."""
    d, r = A.shape
    ws, wb = _ws(ws, spel_workspace_bytes(d, r), A)
    _check(load().spel_step_polar_express(_dev(A, "A", torch.float32), _dev(g, "g", torch.float32),
                                          _dev(m, "m", torch.float32), float(alpha), float(beta), int(lmo_steps),
                                          int(ret_steps), float(ell),
                                          _dev(D_out, "D_out", torch.float32) if D_out is not None else None,
                                          _opt(status, "status", torch.int32), d, r,
                                          ws.data_ptr() if ws is not None else None, wb, _stream(stream)),
           "spel_step_polar_express")
    return D_out


def spel_polar_express_coefficients(ell: float, steps: int):
    """The host-side Polar Express schedule: (coef [steps][3] float64, err [steps])."""
    import numpy as np
    coef = np.zeros((int(steps), 3), dtype=np.float64)
    err = np.zeros(int(steps), dtype=np.float64)
    _check(load().spel_polar_express_coefficients(float(ell), int(steps), coef.ctypes.data, err.ctypes.data),
           "spel_polar_express_coefficients")
    return coef, err
