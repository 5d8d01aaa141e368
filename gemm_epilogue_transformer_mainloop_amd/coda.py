"""Thin ctypes binding of libcoda.so (include/coda.h), one function per C entry point.

The functions marshal torch tensors into pointers, sizes and the current HIP
stream and call the C library; every step of the computation runs in the HIP
kernels.  Torch is used only to allocate device memory for outputs that the
caller did not pass.  If the library is missing, every call raises: there is
no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcoda.so")
# The same kernels with the tile timeline compiled in (coda_timeline_set).
TIMELINE_LIB_PATH = os.path.join(_HERE, "libcoda_timeline.so")
INCLUDE_DIR = os.path.join(os.path.dirname(_HERE), "include")
HEADER_PATHS = [os.path.join(INCLUDE_DIR, h) for h in ("coda.h", "coda_unfused.h", "coda_probe.h")]

_lib = None

P = ctypes.c_void_p
I = ctypes.c_int
F = ctypes.c_float
SZ = ctypes.c_size_t

# name -> (restype, argtypes), following include/coda.h
_SIGS = {
    "coda_status_str": (ctypes.c_char_p, [I]),
    "coda_version": (ctypes.c_char_p, []),
    "coda_debug_extent": (I, [P, SZ]),
    "coda_nparts": (I, [I]),
    "coda_mparts": (I, [I]),
    "coda_tile_split": (I, [I, I, I]),
    "coda_tile_split_tokens": (I, [I, I, I]),
    "coda_swiglu_bwd_units": (I, [I, I, I, I]),
    "coda_lmhead_ce_workspace": (SZ, [I, I]),
    "coda_lmhead_ce_bwd_workspace": (SZ, [I, I, I]),
    "coda_gemm": (I, [P, I, P, I, P, I, I, I, I, P]),
    "coda_gemm_res_sumsq": (I, [P, I, P, I, P, I, P, P, I, P, I, P, I, I, I, P]),
    "coda_row_rms": (I, [P, I, I, I, F, P, P]),
    "coda_gemm_rowscale": (I, [P, I, P, I, P, P, I, I, I, I, P]),
    "coda_gemm_rope": (I, [P, I, P, I, P, P, F, I, I, P, I, I, I, I, P]),
    "coda_gemm_rope_bwd": (I, [P, I, P, I, P, P, F, I, I, P, I, I, I, I, P]),
    "coda_gemm_swiglu": (I, [P, I, P, I, P, P, I, P, I, I, I, I, P]),
    "coda_lmhead_ce": (I, [P, I, P, I, P, P, P, P, P, SZ, I, I, I, P]),
    "coda_gemm_swiglu_bwd": (I, [P, I, P, I, P, I, P, I, P, I, I, I, P]),
    "coda_gemm_swiglu_bwd_overlap": (I, [P, I, P, I, P, I, P, I, P, I, I, I, P]),
    "coda_row_rms_bwd": (I, [P, I, I, I, P, P]),
    "coda_gemm_rowscale_bwd": (I, [P, I, P, I, P, I, P, P, P, P, I, P, I, P, I, P, I, I, I, P]),
    "coda_col_reduce": (I, [P, I, I, P, P]),
    "coda_gemm_res_sumsq_bwd": (I, [P, I, P, I, P, I, P, I, P, I, P, I, I, I, I, P]),
    "coda_gemm_wgrad": (I, [P, I, P, I, P, I, I, I, I, I, P]),
    "coda_lmhead_ce_bwd": (I, [P, I, P, I, P, P, F, P, I, P, I, P, SZ, I, I, I, P]),
    "coda_lmhead_ce_logits": (I, [P, I, P, I, P, P, P, P, P, I, P, SZ, I, I, I, P]),
    "coda_lmhead_ce_noalloc": (I, [P, I, P, I, P, P, P, P, I, I, I, P]),
    "coda_lmhead_ce_bwd_vchunk_workspace": (SZ, [I, I, I, I]),
    "coda_lmhead_ce_bwd_vchunk": (I, [P, I, P, I, P, P, F, P, I, P, I, P, SZ, I, I, I, I, P]),
    "coda_lmhead_ce_noalloc_max_bytes": (SZ, []),
    "coda_lmhead_ce_bwd_logits": (I, [P, I, P, I, P, P, F, P, I, P, I, P, I, I, I, I, P]),
    # LayerNorm variant
    "coda_gemm_res_lnstats": (I, [P, I, P, I, P, I, P, P, I, P, I, P, P, I, I, I, P]),
    "coda_row_ln": (I, [P, P, I, I, I, F, P, P, P]),
    "coda_ln_colvec": (I, [P, I, P, P, I, I, P, P, P]),
    "coda_gemm_ln_rowscale": (I, [P, I, P, I, P, P, P, P, P, I, I, I, I, P]),
    "coda_gemm_ln_swiglu": (I, [P, I, P, I, P, P, P, P, P, I, P, I, I, I, I, P]),
    "coda_gemm_swiglu_bwd_ln": (I, [P, I, P, I, P, I, P, I, P, P, P, P, I, I, I, P]),
    "coda_row_ln_bwd": (I, [P, P, I, I, I, P, P, P]),
    "coda_gemm_ln_bwd": (I, [P, I, P, I, P, I, P, P, P, P, P, P, P, I, P, I, P, I, P, P, I, I, I, P]),
    # include/coda_unfused.h
    "coda_unfused_add": (I, [P, I, P, I, P, I, I, I, P]),
    "coda_unfused_add_rmsnorm": (I, [P, I, P, I, P, F, P, I, P, I, P, I, I, P]),
    "coda_unfused_rope": (I, [P, I, P, F, I, I, I, I, I, P]),
    "coda_unfused_swiglu": (I, [P, I, P, I, I, I, P]),
    "coda_unfused_swiglu_bwd": (I, [P, I, P, I, P, I, I, I, P]),
    "coda_unfused_rmsnorm_bwd_parts": (I, [I]),
    "coda_unfused_rmsnorm_bwd": (I, [P, I, P, I, P, P, P, I, P, I, P, I, I, P]),
    "coda_unfused_cross_entropy": (I, [P, I, P, P, P, P, I, I, P]),
    "coda_unfused_cross_entropy_bwd": (I, [P, I, P, P, F, P, I, I, I, P]),
    # include/coda_probe.h
    "coda_probe_mfma": (I, [I, I, P, P]),
    "coda_timeline_set": (I, [P, I]),
    "coda_timeline_words": (I, []),
}

STATUS = {0: "CODA_OK", 1: "CODA_ERR_NULL", 2: "CODA_ERR_SHAPE", 3: "CODA_ERR_ALIGN",
          4: "CODA_ERR_UNSUPPORTED", 5: "CODA_ERR_HIP", 6: "CODA_ERR_WORKSPACE", 7: "CODA_ERR_BOUNDS"}


class CodaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_str(status)})")


def use_library(path: str) -> None:
    """Load `path` (e.g. TIMELINE_LIB_PATH) instead of libcoda.so; only before the first call."""
    global LIB_PATH
    if _lib is not None and path != LIB_PATH:
        raise RuntimeError(f"{LIB_PATH} is already loaded")
    LIB_PATH = path


def lib():
    """Load libcoda.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run gemm_epilogue_transformer_mainloop_amd/build.py")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def header_functions():
    """Names of the functions the public headers (coda.h, coda_unfused.h, coda_probe.h) declare."""
    names = set()
    for path in HEADER_PATHS:
        with open(path) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names.update(re.findall(r"\b(coda_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def status_str(s: int) -> str:
    return lib().coda_status_str(s).decode()


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise CodaError(name, st)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else int(t.stride(0))


def _mat(t, dtype=torch.bfloat16, name="tensor"):
    if t is None:
        return None
    if t.dtype != dtype or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: need a row-major 2-D {dtype} tensor, got {t.dtype} {tuple(t.shape)} {t.stride()}")
    return t


def _dense(t, name):
    """Partials and vectors have no leading dimension in the ABI: they must be dense."""
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (the C ABI takes no leading dimension for it)")
    return t


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ----------------------------------------------------------------------------
# queries
# ----------------------------------------------------------------------------


def coda_nparts(N: int) -> int:
    return int(lib().coda_nparts(N))


def coda_mparts(M: int) -> int:
    return int(lib().coda_mparts(M))


def coda_tile_split(F: int, T: int, cus: int) -> int:
    return int(lib().coda_tile_split(F, T, cus))


def coda_tile_split_tokens(F: int, T: int, cus: int) -> int:
    return int(lib().coda_tile_split_tokens(F, T, cus))


def coda_swiglu_bwd_units(M: int, F: int, N: int, cus: int) -> int:
    return int(lib().coda_swiglu_bwd_units(M, F, N, cus))


def coda_lmhead_ce_workspace(M: int, V: int) -> int:
    return int(lib().coda_lmhead_ce_workspace(M, V))


def coda_lmhead_ce_bwd_workspace(M: int, V: int, d: int) -> int:
    return int(lib().coda_lmhead_ce_bwd_workspace(M, V, d))


def coda_debug_extent(p: int, nbytes: int) -> int:
    """CODA_DEBUG's extent check of [p, p + nbytes) (returns the status code)."""
    return int(lib().coda_debug_extent(ctypes.c_void_p(p), nbytes))


# ----------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------


def coda_gemm(X, W, Y=None):
    _mat(X, name="X"), _mat(W, name="W")
    M, K = X.shape
    N = W.shape[1]
    if Y is None:
        Y = _empty((M, N), torch.bfloat16, X)
    _call("coda_gemm", _ptr(X), _ld(X), _ptr(W), _ld(W), _ptr(Y), _ld(Y), M, N, K, _stream())
    return Y


def coda_gemm_res_sumsq(X, W, Z=None, gamma=None, U=None, H2=None, part=None, want_h2=True, want_part=True):
    M, K = X.shape
    N = W.shape[1]
    if U is None:
        U = _empty((M, N), torch.bfloat16, X)
    if H2 is None and want_h2 and gamma is not None:
        H2 = _empty((M, N), torch.bfloat16, X)
    if part is None and want_part:
        part = _empty((M, coda_nparts(N)), torch.float32, X)
    _dense(part, "part")
    _call("coda_gemm_res_sumsq", _ptr(X), _ld(X), _ptr(W), _ld(W), _ptr(Z), _ld(Z), _ptr(gamma),
          _ptr(U), _ld(U), _ptr(H2), _ld(H2), _ptr(part), M, N, K, _stream())
    return U, H2, part


def coda_row_rms(part, d: int, eps: float, r=None):
    _dense(part, "part")
    M, np_ = part.shape
    if r is None:
        r = _empty((M,), torch.float32, part)
    _call("coda_row_rms", _ptr(part), np_, M, d, ctypes.c_float(eps), _ptr(r), _stream())
    return r


def coda_gemm_rowscale(A, W, r, Y=None):
    M, K = A.shape
    N = W.shape[1]
    if Y is None:
        Y = _empty((M, N), torch.bfloat16, A)
    _call("coda_gemm_rowscale", _ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(r), _ptr(Y), _ld(Y), M, N, K, _stream())
    return Y


def _rope(name, A, W, r, pos, theta, head_dim, n_rope, Y):
    M, K = A.shape
    N = W.shape[1]
    if Y is None:
        Y = _empty((M, N), torch.bfloat16, A)
    _call(name, _ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(r), _ptr(pos), ctypes.c_float(theta), head_dim,
          n_rope, _ptr(Y), _ld(Y), M, N, K, _stream())
    return Y


def coda_gemm_rope(A, W, r, pos, theta: float, head_dim: int, n_rope: int, Y=None):
    return _rope("coda_gemm_rope", A, W, r, pos, theta, head_dim, n_rope, Y)


def coda_gemm_rope_bwd(A, W, r, pos, theta: float, head_dim: int, n_rope: int, Y=None):
    return _rope("coda_gemm_rope_bwd", A, W, r, pos, theta, head_dim, n_rope, Y)


def coda_gemm_swiglu(A, Wgu, r=None, Act=None, Pre=None, want_pre=True):
    M, K = A.shape
    F = Wgu.shape[1] // 2
    if Act is None:
        Act = _empty((M, F), torch.bfloat16, A)
    if Pre is None and want_pre:
        Pre = _empty((M, 2 * F), torch.bfloat16, A)
    _call("coda_gemm_swiglu", _ptr(A), _ld(A), _ptr(Wgu), _ld(Wgu), _ptr(r), _ptr(Act), _ld(Act), _ptr(Pre),
          _ld(Pre), M, F, K, _stream())
    return Act, Pre


def coda_lmhead_ce(H, W, labels, lse=None, loss_row=None, loss_mean=None, ws=None):
    M, d = H.shape
    V = W.shape[1]
    if lse is None:
        lse = _empty((M,), torch.float32, H)
    if loss_row is None:
        loss_row = _empty((M,), torch.float32, H)
    if loss_mean is None:
        loss_mean = _empty((1,), torch.float32, H)
    if ws is None:
        ws = _empty((max(coda_lmhead_ce_workspace(M, V), 16),), torch.uint8, H)
    _call("coda_lmhead_ce", _ptr(H), _ld(H), _ptr(W), _ld(W), _ptr(labels), _ptr(lse), _ptr(loss_row),
          _ptr(loss_mean), _ptr(ws), ws.numel() * ws.element_size(), M, V, d, _stream())
    return lse, loss_row, loss_mean


def coda_lmhead_ce_noalloc(H, W, labels, lse, loss_row=None, loss_mean=None):
    """coda_lmhead_ce with its workspace in the library's own device array;
    the caller passes the outputs (loss_row / loss_mean may be None)."""
    M, d = H.shape
    V = W.shape[1]
    _call("coda_lmhead_ce_noalloc", _ptr(H), _ld(H), _ptr(W), _ld(W), _ptr(labels), _ptr(lse), _ptr(loss_row),
          _ptr(loss_mean), M, V, d, _stream())
    return lse, loss_row, loss_mean


def coda_lmhead_ce_logits(H, W, labels, lse=None, loss_row=None, loss_mean=None, logits=None, ws=None):
    M, d = H.shape
    V = W.shape[1]
    if lse is None:
        lse = _empty((M,), torch.float32, H)
    if loss_row is None:
        loss_row = _empty((M,), torch.float32, H)
    if loss_mean is None:
        loss_mean = _empty((1,), torch.float32, H)
    if logits is None:
        logits = _empty((M, V), torch.bfloat16, H)
    if ws is None:
        ws = _empty((max(coda_lmhead_ce_workspace(M, V), 16),), torch.uint8, H)
    _call("coda_lmhead_ce_logits", _ptr(H), _ld(H), _ptr(W), _ld(W), _ptr(labels), _ptr(lse), _ptr(loss_row),
          _ptr(loss_mean), _ptr(logits), _ld(logits), _ptr(ws), ws.numel() * ws.element_size(), M, V, d,
          _stream())
    return lse, loss_row, loss_mean, logits


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------


def _swiglu_bwd(name, dOut, Wd, Pre, dPre, spart, want_spart):
    M, N = dOut.shape
    F = Wd.shape[0]
    if dPre is None:
        dPre = _empty((M, 2 * F), torch.bfloat16, dOut)
    if spart is None and want_spart:
        spart = _empty((M, coda_nparts(F)), torch.float32, dOut)
    _dense(spart, "spart")
    _call(name, _ptr(dOut), _ld(dOut), _ptr(Wd), _ld(Wd), _ptr(Pre), _ld(Pre), _ptr(dPre), _ld(dPre), _ptr(spart),
          M, F, N, _stream())
    return dPre, spart


def coda_gemm_swiglu_bwd(dOut, Wd, Pre, dPre=None, spart=None, want_spart=True):
    return _swiglu_bwd("coda_gemm_swiglu_bwd", dOut, Wd, Pre, dPre, spart, want_spart)


def coda_gemm_swiglu_bwd_overlap(dOut, Wd, Pre, dPre=None, spart=None, want_spart=True):
    return _swiglu_bwd("coda_gemm_swiglu_bwd_overlap", dOut, Wd, Pre, dPre, spart, want_spart)


def coda_row_rms_bwd(spart, d: int, s=None):
    _dense(spart, "spart")
    M, np_ = spart.shape
    if s is None:
        s = _empty((M,), torch.float32, spart)
    _call("coda_row_rms_bwd", _ptr(spart), np_, M, d, _ptr(s), _stream())
    return s


def coda_gemm_rowscale_bwd(dY, W1, U, gamma, r, s, dRes=None, dU=None, N2=None, gpart=None, want_n2=True,
                           want_gpart=True):
    M, N = dY.shape
    d = W1.shape[0]
    if dU is None:
        dU = _empty((M, d), torch.bfloat16, dY)
    if N2 is None and want_n2:
        N2 = _empty((M, d), torch.bfloat16, dY)
    if gpart is None and want_gpart:
        gpart = _empty((coda_mparts(M), d), torch.float32, dY)
    _dense(gpart, "gpart")
    _call("coda_gemm_rowscale_bwd", _ptr(dY), _ld(dY), _ptr(W1), _ld(W1), _ptr(U), _ld(U), _ptr(gamma), _ptr(r),
          _ptr(s), _ptr(dRes), _ld(dRes), _ptr(dU), _ld(dU), _ptr(N2), _ld(N2), _ptr(gpart), M, d, N, _stream())
    return dU, N2, gpart


def coda_col_reduce(gpart, dgamma=None):
    _dense(gpart, "gpart")
    mp, d = gpart.shape
    if dgamma is None:
        dgamma = _empty((d,), torch.float32, gpart)
    _call("coda_col_reduce", _ptr(gpart), mp, d, _ptr(dgamma), _stream())
    return dgamma


def coda_gemm_res_sumsq_bwd(dU, W, X=None, dRes=None, dX=None, dW=None, want_dw=True):
    M, N = dU.shape
    K = W.shape[0]
    if dX is None:
        dX = _empty((M, K), torch.bfloat16, dU)
    if dW is None and want_dw and X is not None:
        dW = _empty((K, N), torch.float32, dU)
    _call("coda_gemm_res_sumsq_bwd", _ptr(dU), _ld(dU), _ptr(W), _ld(W), _ptr(X), _ld(X), _ptr(dRes), _ld(dRes),
          _ptr(dX), _ld(dX), _ptr(dW), _ld(dW), M, N, K, _stream())
    return dX, dW


def coda_gemm_wgrad(X, dY, dW=None, accumulate=False):
    M, K = X.shape
    N = dY.shape[1]
    if dW is None:
        dW = _empty((K, N), torch.float32, X)
    _call("coda_gemm_wgrad", _ptr(X), _ld(X), _ptr(dY), _ld(dY), _ptr(dW), _ld(dW), M, K, N, int(bool(accumulate)),
          _stream())
    return dW


def coda_lmhead_ce_bwd(H, W, labels, lse, grad_scale: float, dH=None, dW=None, ws=None, ws_rows=None):
    M, d = H.shape
    V = W.shape[1]
    if dH is None:
        dH = _empty((M, d), torch.bfloat16, H)
    if dW is None:
        dW = _empty((d, V), torch.float32, H)
    if ws is None:
        rows = M if ws_rows is None else ws_rows
        ws = _empty((max(rows * V * 2, coda_lmhead_ce_bwd_workspace(M, V, d), 16),), torch.uint8, H)
    _call("coda_lmhead_ce_bwd", _ptr(H), _ld(H), _ptr(W), _ld(W), _ptr(labels), _ptr(lse),
          ctypes.c_float(grad_scale), _ptr(dH), _ld(dH), _ptr(dW), _ld(dW), _ptr(ws), ws.numel() * ws.element_size(),
          M, V, d, _stream())
    return dH, dW


def coda_lmhead_ce_bwd_vchunk_workspace(M: int, V: int, d: int, vchunk: int) -> int:
    return int(lib().coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, vchunk))


def coda_lmhead_ce_bwd_vchunk(H, W, labels, lse, grad_scale: float, vchunk: int = 8192, dH=None, dW=None, ws=None):
    M, d = H.shape
    V = W.shape[1]
    if dH is None:
        dH = _empty((M, d), torch.bfloat16, H)
    if dW is None:
        dW = _empty((d, V), torch.float32, H)
    if ws is None:
        ws = _empty((max(coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, vchunk), 256),), torch.uint8, H)
    _call("coda_lmhead_ce_bwd_vchunk", _ptr(H), _ld(H), _ptr(W), _ld(W), _ptr(labels), _ptr(lse),
          ctypes.c_float(grad_scale), _ptr(dH), _ld(dH), _ptr(dW), _ld(dW), _ptr(ws), ws.numel() * ws.element_size(),
          M, V, d, vchunk, _stream())
    return dH, dW


def coda_lmhead_ce_bwd_logits(H, W, labels, lse, grad_scale: float, logits, dH=None, dW=None):
    """logits (kept by coda_lmhead_ce_logits) is overwritten with the dlogits."""
    M, d = H.shape
    V = W.shape[1]
    if dH is None:
        dH = _empty((M, d), torch.bfloat16, H)
    if dW is None:
        dW = _empty((d, V), torch.float32, H)
    _call("coda_lmhead_ce_bwd_logits", _ptr(H), _ld(H), _ptr(W), _ld(W), _ptr(labels), _ptr(lse),
          ctypes.c_float(grad_scale), _ptr(logits), _ld(logits), _ptr(dH), _ld(dH), _ptr(dW), _ld(dW),
          M, V, d, _stream())
    return dH, dW


# ----------------------------------------------------------------------------
# LayerNorm variant
# ----------------------------------------------------------------------------


def coda_gemm_res_lnstats(X, W, Z=None, gamma=None, U=None, H2=None, pmean=None, pm2=None, want_h2=True):
    M, K = X.shape
    N = W.shape[1]
    if U is None:
        U = _empty((M, N), torch.bfloat16, X)
    if H2 is None and want_h2 and gamma is not None:
        H2 = _empty((M, N), torch.bfloat16, X)
    if pmean is None:
        pmean = _empty((M, coda_nparts(N)), torch.float32, X)
    if pm2 is None:
        pm2 = _empty((M, coda_nparts(N)), torch.float32, X)
    _dense(pmean, "pmean"), _dense(pm2, "pm2")
    _call("coda_gemm_res_lnstats", _ptr(X), _ld(X), _ptr(W), _ld(W), _ptr(Z), _ld(Z), _ptr(gamma), _ptr(U), _ld(U),
          _ptr(H2), _ld(H2), _ptr(pmean), _ptr(pm2), M, N, K, _stream())
    return U, H2, pmean, pm2


def coda_row_ln(pmean, pm2, d: int, eps: float, mu=None, r=None):
    _dense(pmean, "pmean"), _dense(pm2, "pm2")
    M, np_ = pmean.shape
    if mu is None:
        mu = _empty((M,), torch.float32, pmean)
    if r is None:
        r = _empty((M,), torch.float32, pmean)
    _call("coda_row_ln", _ptr(pmean), _ptr(pm2), np_, M, d, ctypes.c_float(eps), _ptr(mu), _ptr(r), _stream())
    return mu, r


def coda_ln_colvec(W, gamma, beta=None, cvec=None, bvec=None):
    K, N = W.shape
    if cvec is None:
        cvec = _empty((N,), torch.float32, W)
    if bvec is None and beta is not None:
        bvec = _empty((N,), torch.float32, W)
    _call("coda_ln_colvec", _ptr(W), _ld(W), _ptr(gamma), _ptr(beta), K, N, _ptr(cvec), _ptr(bvec), _stream())
    return cvec, bvec


def coda_gemm_ln_rowscale(A, W, r, mu, cvec, bvec=None, Y=None):
    M, K = A.shape
    N = W.shape[1]
    if Y is None:
        Y = _empty((M, N), torch.bfloat16, A)
    _call("coda_gemm_ln_rowscale", _ptr(A), _ld(A), _ptr(W), _ld(W), _ptr(r), _ptr(mu), _ptr(cvec), _ptr(bvec),
          _ptr(Y), _ld(Y), M, N, K, _stream())
    return Y


def coda_gemm_ln_swiglu(A, Wgu, r, mu, cvec, bvec=None, Act=None, Pre=None, want_pre=True):
    M, K = A.shape
    F = Wgu.shape[1] // 2
    if Act is None:
        Act = _empty((M, F), torch.bfloat16, A)
    if Pre is None and want_pre:
        Pre = _empty((M, 2 * F), torch.bfloat16, A)
    _call("coda_gemm_ln_swiglu", _ptr(A), _ld(A), _ptr(Wgu), _ld(Wgu), _ptr(r), _ptr(mu), _ptr(cvec), _ptr(bvec),
          _ptr(Act), _ld(Act), _ptr(Pre), _ld(Pre), M, F, K, _stream())
    return Act, Pre


def coda_gemm_swiglu_bwd_ln(dOut, Wd, Pre, cvec, bvec=None, dPre=None, spart=None, apart=None):
    M, N = dOut.shape
    F = Wd.shape[0]
    if dPre is None:
        dPre = _empty((M, 2 * F), torch.bfloat16, dOut)
    if spart is None:
        spart = _empty((M, coda_nparts(F)), torch.float32, dOut)
    if apart is None:
        apart = _empty((M, coda_nparts(F)), torch.float32, dOut)
    _dense(spart, "spart"), _dense(apart, "apart")
    _call("coda_gemm_swiglu_bwd_ln", _ptr(dOut), _ld(dOut), _ptr(Wd), _ld(Wd), _ptr(Pre), _ld(Pre), _ptr(dPre),
          _ld(dPre), _ptr(cvec), _ptr(bvec), _ptr(spart), _ptr(apart), M, F, N, _stream())
    return dPre, spart, apart


def coda_row_ln_bwd(spart, apart, d: int, s=None, a=None):
    _dense(spart, "spart"), _dense(apart, "apart")
    M, np_ = spart.shape
    if s is None:
        s = _empty((M,), torch.float32, spart)
    if a is None:
        a = _empty((M,), torch.float32, spart)
    _call("coda_row_ln_bwd", _ptr(spart), _ptr(apart), np_, M, d, _ptr(s), _ptr(a), _stream())
    return s, a


def coda_gemm_ln_bwd(dY, W1, U, gamma, beta, r, mu, s, a, dRes=None, dU=None, N2=None, gpart=None, bgpart=None,
                     want_n2=True):
    M, N = dY.shape
    d = W1.shape[0]
    if dU is None:
        dU = _empty((M, d), torch.bfloat16, dY)
    if N2 is None and want_n2:
        N2 = _empty((M, d), torch.bfloat16, dY)
    if gpart is None:
        gpart = _empty((coda_mparts(M), d), torch.float32, dY)
    if bgpart is None:
        bgpart = _empty((coda_mparts(M), d), torch.float32, dY)
    _dense(gpart, "gpart"), _dense(bgpart, "bgpart")
    _call("coda_gemm_ln_bwd", _ptr(dY), _ld(dY), _ptr(W1), _ld(W1), _ptr(U), _ld(U), _ptr(gamma), _ptr(beta),
          _ptr(r), _ptr(mu), _ptr(s), _ptr(a), _ptr(dRes), _ld(dRes), _ptr(dU), _ld(dU), _ptr(N2), _ld(N2),
          _ptr(gpart), _ptr(bgpart), M, d, N, _stream())
    return dU, N2, gpart, bgpart


# ----------------------------------------------------------------------------
# unfused baseline (include/coda_unfused.h)
# ----------------------------------------------------------------------------


def coda_unfused_add(A, B, C=None):
    M, N = A.shape
    if C is None:
        C = _empty((M, N), torch.bfloat16, A)
    _call("coda_unfused_add", _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C), _ld(C), M, N, _stream())
    return C


def coda_unfused_add_rmsnorm(Y, Z, gamma, eps: float, U=None, N2=None, r=None):
    M, d = Y.shape
    if U is None:
        U = _empty((M, d), torch.bfloat16, Y)
    if N2 is None:
        N2 = _empty((M, d), torch.bfloat16, Y)
    if r is None:
        r = _empty((M,), torch.float32, Y)
    _call("coda_unfused_add_rmsnorm", _ptr(Y), _ld(Y), _ptr(Z), _ld(Z), _ptr(gamma), ctypes.c_float(eps), _ptr(U),
          _ld(U), _ptr(N2), _ld(N2), _ptr(r), M, d, _stream())
    return U, N2, r


def coda_unfused_rope(Y, pos, theta: float, head_dim: int, n_rope: int, inverse: bool = False):
    M, N = Y.shape
    _call("coda_unfused_rope", _ptr(Y), _ld(Y), _ptr(pos), ctypes.c_float(theta), head_dim, n_rope, int(inverse),
          M, N, _stream())
    return Y


def coda_unfused_swiglu(Pre, Act=None):
    M, F2 = Pre.shape
    F = F2 // 2
    if Act is None:
        Act = _empty((M, F), torch.bfloat16, Pre)
    _call("coda_unfused_swiglu", _ptr(Pre), _ld(Pre), _ptr(Act), _ld(Act), M, F, _stream())
    return Act


def coda_unfused_swiglu_bwd(dA, Pre, dPre=None):
    M, F = dA.shape
    if dPre is None:
        dPre = _empty((M, 2 * F), torch.bfloat16, dA)
    _call("coda_unfused_swiglu_bwd", _ptr(dA), _ld(dA), _ptr(Pre), _ld(Pre), _ptr(dPre), _ld(dPre), M, F, _stream())
    return dPre


def coda_unfused_rmsnorm_bwd_parts(M: int) -> int:
    return int(lib().coda_unfused_rmsnorm_bwd_parts(M))


def coda_unfused_rmsnorm_bwd(G, U, gamma, r, dRes=None, dU=None, gpart=None, want_gpart=True):
    M, d = G.shape
    if dU is None:
        dU = _empty((M, d), torch.bfloat16, G)
    if gpart is None and want_gpart:
        gpart = _empty((coda_unfused_rmsnorm_bwd_parts(M), d), torch.float32, G)
    _dense(gpart, "gpart")
    _call("coda_unfused_rmsnorm_bwd", _ptr(G), _ld(G), _ptr(U), _ld(U), _ptr(gamma), _ptr(r), _ptr(dRes), _ld(dRes),
          _ptr(dU), _ld(dU), _ptr(gpart), M, d, _stream())
    return dU, gpart


def coda_unfused_cross_entropy(L, labels, lse=None, loss_row=None, loss_mean=None):
    M, V = L.shape
    if lse is None:
        lse = _empty((M,), torch.float32, L)
    if loss_row is None:
        loss_row = _empty((M,), torch.float32, L)
    if loss_mean is None:
        loss_mean = _empty((1,), torch.float32, L)
    _call("coda_unfused_cross_entropy", _ptr(L), _ld(L), _ptr(labels), _ptr(lse), _ptr(loss_row), _ptr(loss_mean),
          M, V, _stream())
    return lse, loss_row, loss_mean


def coda_unfused_cross_entropy_bwd(L, labels, lse, grad_scale: float, D=None):
    M, V = L.shape
    if D is None:
        D = _empty((M, V), torch.bfloat16, L)
    _call("coda_unfused_cross_entropy_bwd", _ptr(L), _ld(L), _ptr(labels), _ptr(lse), ctypes.c_float(grad_scale),
          _ptr(D), _ld(D), M, V, _stream())
    return D


# ----------------------------------------------------------------------------
# measurement support (include/coda_probe.h)
# ----------------------------------------------------------------------------


def coda_probe_mfma(blocks: int, iters: int, out=None):
    """Matrix-core clock probe; returns the int64 device tensor [blocks, 2] of
    (shader-clock ticks, reference-clock ticks) per workgroup."""
    if out is None:
        out = torch.zeros((blocks, 2), dtype=torch.int64, device="cuda")
    _call("coda_probe_mfma", blocks, iters, _ptr(out), _stream())
    return out


def coda_timeline_words() -> int:
    return lib().coda_timeline_words()


def coda_timeline_set(buf=None):
    """Install the int64 device tensor `buf` [waves, coda_timeline_words()] as
    the tile-timeline buffer of later GEMM launches (timeline build only);
    None uninstalls."""
    if buf is None:
        _call("coda_timeline_set", None, 0)
        return
    assert buf.is_cuda and buf.dtype == torch.int64 and buf.is_contiguous()
    assert buf.dim() == 2 and buf.shape[1] == coda_timeline_words()
    _call("coda_timeline_set", _ptr(buf), buf.shape[0])
