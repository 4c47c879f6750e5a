"""Python binding of libqlora_nf4 (argument marshalling only).

Every function here forwards torch device tensors (as raw pointers) and the
current HIP stream to the C ABI declared in ``include/qlora_nf4.h``; all
arithmetic runs in the library's gfx950 kernels. There is no fallback: if the
shared library is missing or fails to load, the first call raises.

bf16 tensors are ``torch.bfloat16`` (passed as their uint16 bit patterns).
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")
#: measurement build of the same sources with per-launch HIP events
#: (include/qlora_nf4_timing.h); loaded only inside ``timing_build()``
TIMING_LIB_PATH = os.path.join(_HERE, "libqlora_nf4_timing.so")

QLORA_OK, QLORA_ERR_INVALID_ARG, QLORA_ERR_UNSUPPORTED, QLORA_ERR_WORKSPACE, QLORA_ERR_HIP = (
    0, -1, -2, -3, -4)
OP_QUANTIZE, OP_FWD, OP_BWD, OP_FWD_MULTI, OP_QUANTIZE_RESIDUAL, OP_LOFTQ = 0, 1, 2, 3, 4, 5


class QLoRAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class NF4WeightC(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int64), ("k", ctypes.c_int64),
        ("blocksize", ctypes.c_int32), ("double_quant", ctypes.c_int32),
        ("dq_blocksize", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
        ("absmax_q", ctypes.c_void_p), ("absmax_scale", ctypes.c_void_p),
        ("absmax_offset", ctypes.c_void_p),
    ]


_lib = None
_timing_lib = None
_use_timing = False
_vp, _i64, _i32, _f32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                              ctypes.c_float, ctypes.c_size_t)
_PW = ctypes.POINTER(NF4WeightC)

#: exported symbol -> (restype, argtypes); mirrors include/qlora_nf4.h
SIGNATURES = {
    "qlora_nf4_quantize": (ctypes.c_int, [_vp, _PW, _vp, _sz, _vp]),
    "qlora_nf4_dequantize": (ctypes.c_int, [_PW, _vp, _vp]),
    "qlora_linear_fwd": (ctypes.c_int, [_PW, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp,
                                        _vp, _sz, _vp]),
    "qlora_linear_bwd": (ctypes.c_int, [_PW, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _sz, _vp]),
    "qlora_linear_fwd_ex": (ctypes.c_int, [_PW, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp,
                                           _vp, _sz, _vp]),
    "qlora_linear_bwd_ex": (ctypes.c_int, [_PW, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _sz, _vp]),
    "qlora_linear_fwd_multi": (ctypes.c_int, [_vp, _i32, _vp, _i64, _vp, _vp, _i32, _f32, _vp,
                                              _vp, _vp, _sz, _vp]),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_PW, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp,
                                                _vp]),
    "qlora_merge": (ctypes.c_int, [_PW, _vp, _vp, _i32, _f32, _vp, _vp]),
    "qlora_nf4_quantize_residual": (ctypes.c_int, [_vp, _vp, _vp, _i32, _f32, _PW, _vp, _sz,
                                                   _vp]),
    "qlora_loftq_init": (ctypes.c_int, [_vp, _vp, _i32, _f32, _i32, _i32, _PW, _vp, _vp, _vp,
                                        _vp, _sz, _vp]),
    "qlora_nf4_storage_bytes": (_sz, [_i64, _i64, _i32]),
    "qlora_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64, _i32, _i32]),
    "qlora_nf4_codebook": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_float)]),
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_adamw_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "qlora_adamw_page_out": (ctypes.c_int, [_vp, _vp, _i32, _i64, _vp]),
    "qlora_adamw_page_in": (ctypes.c_int, [_vp, _vp, _i32, _i64, _vp]),
}

#: the timing build's extra symbols; mirrors include/qlora_nf4_timing.h
TIMING_SIGNATURES = {
    "qlora_profile_begin": (ctypes.c_int, [_i32, ctypes.c_uint32]),
    "qlora_profile_end": (ctypes.c_int, []),
    "qlora_profile_query": (ctypes.c_int, [_i32, ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_double)]),
    "qlora_profile_release": (ctypes.c_int, []),
}

#: kernel ids of the timing hooks (QLORA_K_* in include/qlora_nf4_timing.h);
#: ids 8 and 10 are reserved and never recorded
KERNELS = ["quantize", "double_quant", "dequantize", "gemm_fwd", "gemm_dx", "gemv",
           "gemv_epilogue", "lora_down", "lora_reduce", "lora_colacc", "lora_colacc_reduce",
           "merge", "layout", "adamw", "loftq_product", "loftq_small", "residual"]


def _load(path: str, signatures: dict) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with "
                          "`python -m bit_nf4_quantized_19_amd.build`")
    L = ctypes.CDLL(path)
    for name, (res, args) in signatures.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib() -> ctypes.CDLL:
    """The library every call goes through: the product build, or the timing
    build inside ``timing_build()``. Loaded once; raises if it is not built."""
    global _lib
    if _use_timing:
        return timing_lib()
    if _lib is None:
        _lib = _load(LIB_PATH, SIGNATURES)
    return _lib


def timing_lib() -> ctypes.CDLL:
    """The timing build (same kernels and entry points plus qlora_profile_*)."""
    global _timing_lib
    if _timing_lib is None:
        _timing_lib = _load(TIMING_LIB_PATH, {**SIGNATURES, **TIMING_SIGNATURES})
    return _timing_lib


@contextlib.contextmanager
def timing_build():
    """Route every call of this module to the timing build while inside."""
    global _use_timing
    prev = _use_timing
    _use_timing = True
    try:
        yield timing_lib()
    finally:
        _use_timing = prev


def status_string(status: int) -> str:
    return lib().qlora_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != QLORA_OK:
        raise QLoRAError(status, what)


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dev_bf16(t: torch.Tensor, name: str):
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor")


# ---------------------------------------------------------------------------
@dataclass
class NF4Weight:
    """Quantised weight: packed codes plus absmax or its double-quantised form."""
    d: int
    k: int
    double_quant: bool
    codes: torch.Tensor                      # uint8 [d*k/2]
    absmax: torch.Tensor | None = None       # float32 [nb]
    absmax_q: torch.Tensor | None = None     # int8 [nb]
    absmax_scale: torch.Tensor | None = None  # float32 [ceil(nb/256)]
    absmax_offset: torch.Tensor | None = None  # float32 [1]

    def c_struct(self) -> NF4WeightC:
        return NF4WeightC(self.d, self.k, 64, int(self.double_quant), 256, 0,
                          _ptr(self.codes), _ptr(self.absmax), _ptr(self.absmax_q),
                          _ptr(self.absmax_scale), _ptr(self.absmax_offset))

    @staticmethod
    def empty(d: int, k: int, double_quant: bool, device="cuda") -> "NF4Weight":
        n = d * k
        nb = n // 64
        w = NF4Weight(d, k, double_quant, torch.empty(n // 2, dtype=torch.uint8, device=device))
        if double_quant:
            w.absmax_q = torch.empty(nb, dtype=torch.int8, device=device)
            w.absmax_scale = torch.empty(-(-nb // 256), dtype=torch.float32, device=device)
            w.absmax_offset = torch.empty(1, dtype=torch.float32, device=device)
        else:
            w.absmax = torch.empty(nb, dtype=torch.float32, device=device)
        return w


def storage_bytes(d: int, k: int, double_quant: bool) -> int:
    return int(lib().qlora_nf4_storage_bytes(d, k, int(double_quant)))


def workspace_bytes(op: int, d: int, k: int, M: int = 0, r: int = 0,
                    double_quant: bool = True) -> int:
    n = lib().qlora_workspace_bytes(op, d, k, M, r, int(double_quant))
    if n == ctypes.c_size_t(-1).value:
        raise QLoRAError(QLORA_ERR_UNSUPPORTED, "workspace_bytes")
    return int(n)


def codebook():
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _check(lib().qlora_nf4_codebook(lv, th), "codebook")
    return list(lv), list(th)


def _workspace(nbytes: int, device, ws: torch.Tensor | None):
    if nbytes == 0:
        return None, 0
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    t = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + nbytes], nbytes


def quantize(W0: torch.Tensor, double_quant: bool = True, out: NF4Weight | None = None,
             ws: torch.Tensor | None = None, stream=None) -> NF4Weight:
    _dev_bf16(W0, "W0")
    d, k = W0.shape
    w = out if out is not None else NF4Weight.empty(d, k, double_quant, W0.device)
    wsb = workspace_bytes(OP_QUANTIZE, d, k, 0, 0, double_quant)
    wst, wsn = _workspace(wsb, W0.device, ws)
    cw = w.c_struct()
    _check(lib().qlora_nf4_quantize(W0.data_ptr(), ctypes.byref(cw), _ptr(wst), wsn,
                                    _stream(stream)), "qlora_nf4_quantize")
    return w


def quantize_residual(W: torch.Tensor, A: torch.Tensor, B: torch.Tensor, lora_alpha: float,
                      double_quant: bool = True, out: NF4Weight | None = None,
                      ws: torch.Tensor | None = None, stream=None) -> NF4Weight:
    """NF4 (+DQ) of bf16(W - (alpha/r) B A): the base of one LoftQ step."""
    for t, nm in ((W, "W"), (A, "A"), (B, "B")):
        _dev_bf16(t, nm)
    d, k = W.shape
    r = A.shape[0]
    w = out if out is not None else NF4Weight.empty(d, k, double_quant, W.device)
    wsb = workspace_bytes(OP_QUANTIZE_RESIDUAL, d, k, 0, r, double_quant)
    wst, wsn = _workspace(wsb, W.device, ws)
    cw = w.c_struct()
    _check(lib().qlora_nf4_quantize_residual(W.data_ptr(), A.data_ptr(), B.data_ptr(), r,
                                             float(lora_alpha), ctypes.byref(cw), _ptr(wst), wsn,
                                             _stream(stream)), "qlora_nf4_quantize_residual")
    return w


def loftq_init(W: torch.Tensor, omega: torch.Tensor, lora_alpha: float, iters: int = 1,
               power_iters: int = 4, double_quant: bool = True, ws: torch.Tensor | None = None,
               stream=None):
    """LoftQ: returns (NF4Weight, A (r x k bf16), B (d x r bf16), sigma (r fp32)).
    ``omega`` is the k x r float32 Gaussian test matrix (its column count is r)."""
    _dev_bf16(W, "W")
    if omega.dtype != torch.float32 or not omega.is_cuda or not omega.is_contiguous():
        raise ValueError("omega must be a contiguous float32 CUDA tensor")
    d, k = W.shape
    if omega.dim() != 2 or omega.shape[0] != k:
        raise ValueError("omega must be k x r")
    r = omega.shape[1]
    w = NF4Weight.empty(d, k, double_quant, W.device)
    A = torch.empty(r, k, dtype=torch.bfloat16, device=W.device)
    B = torch.empty(d, r, dtype=torch.bfloat16, device=W.device)
    sigma = torch.empty(r, dtype=torch.float32, device=W.device)
    wsb = workspace_bytes(OP_LOFTQ, d, k, 0, r, double_quant)
    wst, wsn = _workspace(wsb, W.device, ws)
    cw = w.c_struct()
    _check(lib().qlora_loftq_init(W.data_ptr(), omega.data_ptr(), r, float(lora_alpha), int(iters),
                                  int(power_iters), ctypes.byref(cw), A.data_ptr(), B.data_ptr(),
                                  sigma.data_ptr(), _ptr(wst), wsn, _stream(stream)),
           "qlora_loftq_init")
    return w, A, B, sigma


def dequantize(w: NF4Weight, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    Y = out if out is not None else torch.empty(w.d, w.k, dtype=torch.bfloat16,
                                                device=w.codes.device)
    cw = w.c_struct()
    _check(lib().qlora_nf4_dequantize(ctypes.byref(cw), Y.data_ptr(), _stream(stream)),
           "qlora_nf4_dequantize")
    return Y


class LoraDropoutC(ctypes.Structure):
    _fields_ = [("p", ctypes.c_float), ("reserved", ctypes.c_uint32), ("seed", ctypes.c_uint64),
                ("mask", ctypes.c_void_p)]


def dropout_mask(M: int, k: int, device="cuda") -> torch.Tensor:
    """Buffer for the keep bits a forward stores for its backward (M*k/4 bytes)."""
    return torch.empty(M * k // 4, dtype=torch.uint8, device=device)


def _check_mask(mask, M: int, k: int):
    if mask is None:
        return
    if (mask.dtype != torch.uint8 or not mask.is_cuda or not mask.is_contiguous()
            or mask.numel() < M * k // 4):
        raise ValueError(f"mask: contiguous uint8 device tensor of at least {M * k // 4} "
                         "bytes (M*k/4) expected")


def linear_fwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
               lora_alpha: float, save_h: bool = True, Y: torch.Tensor | None = None,
               H: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None,
               dropout: float = 0.0, seed: int = 0, mask: torch.Tensor | None = None):
    """Y = X W'^T + (alpha/r) (X~ A^T) B^T with X~ the adapter input after
    dropout at rate `dropout` (keep bits from `seed`; 0 = none); with more than
    16 tokens the bits are also stored in `mask` (M*k/4 bytes, see
    dropout_mask) when given. Returns (Y, H or None)."""
    for t, nm in ((X, "X"), (A, "A"), (B, "B")):
        _dev_bf16(t, nm)
    M = X.shape[0]
    r = A.shape[0]
    if Y is None:
        Y = torch.empty(M, w.d, dtype=torch.bfloat16, device=X.device)
    if save_h and H is None:
        H = torch.empty(M, r, dtype=torch.float32, device=X.device)
    wsb = workspace_bytes(OP_FWD, w.d, w.k, M, r, w.double_quant)
    wst, wsn = _workspace(wsb, X.device, ws)
    cw = w.c_struct()
    if dropout:
        _check_mask(mask, M, w.k)
        dr = LoraDropoutC(float(dropout), 0, int(seed), _ptr(mask))
        _check(lib().qlora_linear_fwd_ex(ctypes.byref(cw), X.data_ptr(), M, A.data_ptr(),
                                         B.data_ptr(), r, float(lora_alpha), ctypes.addressof(dr),
                                         Y.data_ptr(), _ptr(H) if save_h else None, _ptr(wst),
                                         wsn, _stream(stream)), "qlora_linear_fwd_ex")
    else:
        _check(lib().qlora_linear_fwd(ctypes.byref(cw), X.data_ptr(), M, A.data_ptr(),
                                      B.data_ptr(), r, float(lora_alpha), Y.data_ptr(),
                                      _ptr(H) if save_h else None, _ptr(wst), wsn,
                                      _stream(stream)), "qlora_linear_fwd")
    return Y, (H if save_h else None)


NOALLOC_SCRATCH_BYTES = 16 << 20


def linear_fwd_noalloc(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                       lora_alpha: float, Y: torch.Tensor, H: torch.Tensor | None = None,
                       stream=None):
    """qlora_linear_fwd_noalloc: the forward into caller-given Y (and H)
    with the library's own 16 MiB device scratch instead of a workspace
    (nothing is allocated by the library or here)."""
    for t, nm in ((X, "X"), (A, "A"), (B, "B"), (Y, "Y")):
        _dev_bf16(t, nm)
    cw = w.c_struct()
    _check(lib().qlora_linear_fwd_noalloc(ctypes.byref(cw), X.data_ptr(), X.shape[0],
                                          A.data_ptr(), B.data_ptr(), A.shape[0],
                                          float(lora_alpha), Y.data_ptr(), _ptr(H),
                                          _stream(stream)), "qlora_linear_fwd_noalloc")
    return Y, H


def linear_fwd_multi(ws_: list, X: torch.Tensor, As: list, Bs: list, lora_alpha: float,
                     save_h: bool = True, Ys: list | None = None, ws: torch.Tensor | None = None,
                     stream=None, Hs: list | None = None):
    """Sibling projections: Y_i = X W_i'^T + (alpha/r) (X A_i^T) B_i^T for up
    to four weights reading the same X, in one call. Returns (Ys, Hs)."""
    nw = len(ws_)
    if not (1 <= nw <= 4) or len(As) != nw or len(Bs) != nw:
        raise ValueError("one to four weights, each with its A and B")
    _dev_bf16(X, "X")
    for i in range(nw):
        _dev_bf16(As[i], f"A[{i}]")
        _dev_bf16(Bs[i], f"B[{i}]")
    M, r = X.shape[0], As[0].shape[0]
    if Ys is None:
        Ys = [torch.empty(M, w.d, dtype=torch.bfloat16, device=X.device) for w in ws_]
    if save_h and Hs is None:
        Hs = [torch.empty(M, r, dtype=torch.float32, device=X.device) for _ in range(nw)]
    if not save_h:
        Hs = None
    dtot = sum(w.d for w in ws_)
    wsb = workspace_bytes(OP_FWD_MULTI, dtot, ws_[0].k, M, r, ws_[0].double_quant)
    wst, wsn = _workspace(wsb, X.device, ws)
    cws = [w.c_struct() for w in ws_]
    wp = (ctypes.c_void_p * nw)(*[ctypes.addressof(c) for c in cws])
    ap = (ctypes.c_void_p * nw)(*[a.data_ptr() for a in As])
    bp = (ctypes.c_void_p * nw)(*[b.data_ptr() for b in Bs])
    yp = (ctypes.c_void_p * nw)(*[y.data_ptr() for y in Ys])
    hp = (ctypes.c_void_p * nw)(*[h.data_ptr() for h in Hs]) if save_h else None
    _check(lib().qlora_linear_fwd_multi(wp, nw, X.data_ptr(), M, ap, bp, r, float(lora_alpha), yp,
                                        hp, _ptr(wst), wsn, _stream(stream)),
           "qlora_linear_fwd_multi")
    return Ys, Hs


def linear_bwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
               lora_alpha: float, dY: torch.Tensor, H: torch.Tensor | None = None,
               need_dx: bool = True, dX=None, dA=None, dB=None,
               ws: torch.Tensor | None = None, stream=None, dropout: float = 0.0, seed: int = 0,
               mask: torch.Tensor | None = None):
    """Returns (dX or None, dA, dB); `dropout`, `seed` and `mask` as given to the
    forward (with more than 16 tokens the forward stored the keep bits in
    `mask`, which the backward then reads instead of drawing them again)."""
    for t, nm in ((X, "X"), (A, "A"), (B, "B"), (dY, "dY")):
        _dev_bf16(t, nm)
    M = X.shape[0]
    r = A.shape[0]
    dev = X.device
    if need_dx and dX is None:
        dX = torch.empty(M, w.k, dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty(r, w.k, dtype=torch.bfloat16, device=dev)
    if dB is None:
        dB = torch.empty(w.d, r, dtype=torch.bfloat16, device=dev)
    wsb = workspace_bytes(OP_BWD, w.d, w.k, M, r, w.double_quant)
    wst, wsn = _workspace(wsb, dev, ws)
    cw = w.c_struct()
    if dropout:
        _check_mask(mask, M, w.k)
        dr = LoraDropoutC(float(dropout), 0, int(seed), _ptr(mask))
        _check(lib().qlora_linear_bwd_ex(ctypes.byref(cw), X.data_ptr(), M, A.data_ptr(),
                                         B.data_ptr(), r, float(lora_alpha), ctypes.addressof(dr),
                                         dY.data_ptr(), _ptr(H), _ptr(dX) if need_dx else None,
                                         dA.data_ptr(), dB.data_ptr(), _ptr(wst), wsn,
                                         _stream(stream)), "qlora_linear_bwd_ex")
    else:
        _check(lib().qlora_linear_bwd(ctypes.byref(cw), X.data_ptr(), M, A.data_ptr(),
                                      B.data_ptr(), r, float(lora_alpha), dY.data_ptr(), _ptr(H),
                                      _ptr(dX) if need_dx else None, dA.data_ptr(), dB.data_ptr(),
                                      _ptr(wst), wsn, _stream(stream)), "qlora_linear_bwd")
    return (dX if need_dx else None), dA, dB


def merge(w: NF4Weight, A: torch.Tensor, B: torch.Tensor, lora_alpha: float,
          out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _dev_bf16(A, "A")
    _dev_bf16(B, "B")
    r = A.shape[0]
    Wm = out if out is not None else torch.empty(w.d, w.k, dtype=torch.bfloat16,
                                                 device=A.device)
    cw = w.c_struct()
    _check(lib().qlora_merge(ctypes.byref(cw), A.data_ptr(), B.data_ptr(), r,
                             float(lora_alpha), Wm.data_ptr(), _stream(stream)), "qlora_merge")
    return Wm


class AdamWHParamsC(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


def adamw_step(param: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
               grad: torch.Tensor, param_bf16: torch.Tensor, step: int, lr: float = 2e-4,
               beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
               weight_decay: float = 0.0, stream=None):
    """One AdamW step in place on (param, exp_avg, exp_avg_sq) (float32) with
    the bf16 gradient, writing the bf16 copy of the updated parameter.

    The float32 state may be CUDA tensors or page-locked host tensors
    (``pin_memory=True``; the paged-out state), which the kernel reads and
    writes in place over the host link."""
    n = param.numel()
    for t, name in ((param, "param"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a CUDA tensor or page-locked host memory")
    for t, name in ((grad, "grad"), (param_bf16, "param_bf16")):
        _dev_bf16(t, name)
        if t.numel() != n:
            raise ValueError(f"{name} must have {n} elements")
    hp = AdamWHParamsC(lr, beta1, beta2, eps, weight_decay)
    _check(lib().qlora_adamw_step(_ptr(param), _ptr(exp_avg), _ptr(exp_avg_sq), _ptr(grad),
                                  _ptr(param_bf16), n, ctypes.addressof(hp), int(step),
                                  _stream(stream)), "qlora_adamw_step")


def _page(fn: str, dst, src, stream):
    if len(dst) != len(src) or not 1 <= len(dst) <= 3:
        raise ValueError("dst and src must list the same 1 to 3 buffers")
    n = dst[0].numel()
    for t in list(dst) + list(src):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"every buffer must be a contiguous float32 tensor of {n} elements")
    arr = ctypes.c_void_p * len(dst)
    d = arr(*[t.data_ptr() for t in dst])
    s = arr(*[t.data_ptr() for t in src])
    _check(getattr(lib(), fn)(d, s, len(dst), n, _stream(stream)), fn)


def adamw_page_out(host, dev, stream=None):
    """Enqueue copies of the optimiser state ``dev`` (CUDA float32 tensors:
    param, exp_avg, exp_avg_sq or a subset) into the page-locked host
    tensors ``host`` on the stream."""
    _page("qlora_adamw_page_out", host, dev, stream)


def adamw_page_in(dev, host, stream=None):
    """Enqueue copies of the paged-out state ``host`` (page-locked float32
    tensors) back into the CUDA tensors ``dev`` on the stream."""
    _page("qlora_adamw_page_in", dev, host, stream)


def profile_begin(cap: int = 4096, kernels=None):
    """Start bracketing kernel launches of the timing build with HIP events
    (include/qlora_nf4_timing.h); only calls made inside ``timing_build()``
    are seen;
    ``kernels`` (names from KERNELS) limits the bracketing to those kernels."""
    mask = 0
    for name in kernels or ():
        mask |= 1 << KERNELS.index(name)
    _check(timing_lib().qlora_profile_begin(int(cap), mask), "qlora_profile_begin")


def profile_end():
    _check(timing_lib().qlora_profile_end(), "qlora_profile_end")


def profile_query(kernel: str):
    """(launch count, total milliseconds) of a kernel since profile_begin."""
    cnt = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    _check(timing_lib().qlora_profile_query(KERNELS.index(kernel), ctypes.byref(cnt),
                                     ctypes.byref(ms)), "qlora_profile_query")
    return int(cnt.value), float(ms.value)


__all__ = ["NF4Weight", "QLoRAError", "quantize", "dequantize", "linear_fwd", "linear_bwd",
           "merge", "storage_bytes", "workspace_bytes", "codebook", "lib",
           "OP_QUANTIZE", "OP_FWD", "OP_BWD", "SIGNATURES", "LIB_PATH", "KERNELS",
           "profile_begin", "profile_end", "profile_query", "timing_build", "timing_lib",
           "TIMING_LIB_PATH"]
