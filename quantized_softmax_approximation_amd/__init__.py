"""Quantized-softmax attention forward (and backward) for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libqsa.so (C ABI in include/qsa.h).  Every step of
the computation runs in the library's HIP kernels; this module only checks
tensors, marshals pointers and the current HIP stream, and raises on a
non-zero status.  PyTorch provides device memory and streams.

    import quantized_softmax_approximation_amd as qsa
    o = qsa.attn_fwd(q, k, v, causal=True, kind="pot", levels=8)
    dq, dk, dv = qsa.attn_bwd(q, k, v, do, causal=True, kind="kint", levels=4, grad="ste_pre")
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["attn_fwd", "attn_fwd_ex", "attn_bwd", "attn_validate", "GRADS", "variant_code", "status_string", "last_error",
           "version", "lib", "lib_path", "QSAError", "EXACT", "KINT", "POT", "EXACT_ANCHORED", "TRUNC", "UNIFORM",
           "POT_RUNNING", "F_INTERP",
           "F_WINDOW", "F_FLUSH", "DT_F32", "DT_BF16", "DT_FP8_E4M3", "IDX_FLUSHED", "IDX_MASKED"]

# ABI constants (include/qsa.h)
OK, ERR_NULL_PTR, ERR_SHAPE, ERR_PARAM, ERR_UNSUPPORTED, ERR_HIP = range(6)
DT_F32, DT_BF16, DT_FP8_E4M3 = 0, 1, 2
EXACT, KINT, POT, EXACT_ANCHORED, TRUNC, UNIFORM, POT_RUNNING = 0, 1, 2, 3, 4, 5, 6
F_INTERP, F_WINDOW, F_FLUSH = 1 << 4, 1 << 5, 1 << 6
IDX_FLUSHED, IDX_MASKED = 254, 255
GRAD_STE_POST, GRAD_EXACT, GRAD_EXACT_DETACHED, GRAD_STE_PRE, GRAD_STE_PRE_DETACHED = range(5)
GRADS = {"ste_post": GRAD_STE_POST, "exact": GRAD_EXACT, "exact_detached": GRAD_EXACT_DETACHED,
         "ste_pre": GRAD_STE_PRE, "ste_pre_detached": GRAD_STE_PRE_DETACHED}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None


class QSAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


class _Opts(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("q_descale", ctypes.c_float), ("k_descale", ctypes.c_float),
                ("v_descale", ctypes.c_float), ("row_max", ctypes.c_void_p), ("row_lo", ctypes.c_void_p),
                ("row_sum", ctypes.c_void_p), ("grid_idx", ctypes.c_void_p), ("idx_row0", ctypes.c_int),
                ("idx_rows", ctypes.c_int)]


def lib_path() -> str:
    return os.environ.get("QSA_LIB", os.path.join(_HERE, "libqsa.so"))


def lib() -> ctypes.CDLL:
    """Load libqsa.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m quantized_softmax_approximation_amd.build`")
        L = ctypes.CDLL(path)
        i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        L.qsa_attn_fwd.argtypes = [p, p, p, p, i, i, i, i, i, i, i, i, f, i, p]
        L.qsa_attn_fwd.restype = i
        L.qsa_attn_fwd_ex.argtypes = [p, p, p, p, i, i, i, i, i, i, i, i, f, i, ctypes.POINTER(_Opts), p]
        L.qsa_attn_fwd_ex.restype = i
        L.qsa_attn_bwd.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, i, f, p]
        L.qsa_attn_bwd.restype = i
        L.qsa_attn_validate.argtypes = [i, i, i, i, i, i, i, i, f, i]
        L.qsa_attn_validate.restype = i
        L.qsa_status_string.argtypes = [i]
        L.qsa_status_string.restype = ctypes.c_char_p
        L.qsa_last_error.argtypes = []
        L.qsa_last_error.restype = ctypes.c_char_p
        L.qsa_version.argtypes = []
        L.qsa_version.restype = i
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().qsa_status_string(status).decode()


def last_error() -> str:
    return lib().qsa_last_error().decode()


def version() -> int:
    return lib().qsa_version()


def variant_code(kind: str = "exact", *, interp: bool = False, window: Optional[float] = None,
                 flush: bool = False) -> int:
    """Variant bits for kind in {"exact", "exact_anchored", "kint", "pot", "pot_running", "trunc",
    "uniform"} plus flags.  For "trunc" and "uniform" the window is the support width W, not a flag."""
    base = {"exact": EXACT, "kint": KINT, "pot": POT, "exact_anchored": EXACT_ANCHORED, "trunc": TRUNC,
            "uniform": UNIFORM, "pot_running": POT_RUNNING}[kind]
    if base in (TRUNC, UNIFORM):
        return base | (F_INTERP if interp else 0) | (F_FLUSH if flush else 0)
    return base | (F_INTERP if interp else 0) | (F_WINDOW if window is not None else 0) | (F_FLUSH if flush else 0)


_DT = {torch.float32: DT_F32, torch.bfloat16: DT_BF16, torch.float8_e4m3fn: DT_FP8_E4M3}


def attn_validate(B, H, Hkv, N, d, causal, variant, k_levels, window, dtype) -> int:
    return lib().qsa_attn_validate(B, H, Hkv, N, d, int(bool(causal)), variant, k_levels, float(window), dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_out(t, shape, dtype, dev, name):
    if t is None:
        return
    if t.device != dev or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {dev}")


def _check_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    """Shapes, dtype, device and layout of the inputs; every kernel sizes its reads of K and V
    from q's N and d, so a shorter k or v must be refused here, before any launch."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H(kv), N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError(f"k and v must be [B, Hkv, N, d] = {(B, Hkv, N, d)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise ValueError("q, k, v must share one dtype among float32, bfloat16, float8_e4m3fn")
    dev = q.device
    if dev.type != "cuda" or k.device != dev or v.device != dev:
        raise ValueError("q, k, v must be on the same GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    return B, H, N, d, Hkv, dev


def attn_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False, kind: str = "exact",
                levels: int = 0, window: Optional[float] = None, interp: bool = False, flush: bool = False,
                scale: float = 0.0, q_descale: float = 0.0, k_descale: float = 0.0, v_descale: float = 0.0,
                out: Optional[torch.Tensor] = None, row_max: Optional[torch.Tensor] = None,
                row_lo: Optional[torch.Tensor] = None, row_sum: Optional[torch.Tensor] = None,
                grid_idx: Optional[torch.Tensor] = None, idx_row0: int = 0,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Attention forward through qsa_attn_fwd_ex; returns O.

    q: [B,H,N,d]; k, v: [B,Hkv,N,d]; all on one GPU, contiguous, one dtype
    (float32, bfloat16 or float8_e4m3fn).  O is float32 for float32 inputs,
    else bfloat16.  Optional outputs (row_max/row_lo/row_sum [B,H,N] float32,
    grid_idx [B,H,R,N] uint8 for query rows idx_row0..idx_row0+R-1) are
    written when given.  The call is asynchronous on `stream` (default: the
    current stream).
    """
    B, H, N, d, Hkv, dev = _check_qkv(q, k, v)
    dt = _DT[q.dtype]
    odt = torch.float32 if dt == DT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, H, N, d), dtype=odt, device=dev)
    _check_out(out, (B, H, N, d), odt, dev, "out")
    for name, t in (("row_max", row_max), ("row_lo", row_lo), ("row_sum", row_sum)):
        _check_out(t, (B, H, N), torch.float32, dev, name)
    rows = 0
    if grid_idx is not None:
        rows = grid_idx.shape[2] if grid_idx.dim() == 4 else -1
        _check_out(grid_idx, (B, H, rows, N), torch.uint8, dev, "grid_idx")
    variant = variant_code(kind, interp=interp, window=window, flush=flush)
    opts = _Opts(scale, q_descale, k_descale, v_descale, _ptr(row_max), _ptr(row_lo), _ptr(row_sum),
                 _ptr(grid_idx), idx_row0, rows)
    st = (stream or torch.cuda.current_stream(dev)).cuda_stream
    with torch.cuda.device(dev):
        status = lib().qsa_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d, int(bool(causal)),
                                       variant, int(levels), float(window or 0.0), dt, ctypes.byref(opts),
                                       ctypes.c_void_p(st))
    if status != OK:
        raise QSAError(status, last_error())
    return out


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False, kind: str = "exact",
             levels: int = 0, window: Optional[float] = None, interp: bool = False, flush: bool = False,
             out: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Attention forward through qsa_attn_fwd (scale 1/sqrt(d), descales 1).  Tensors as for
    attn_fwd_ex (float32 or bfloat16; fp8 needs the descales of attn_fwd_ex)."""
    if q.dtype == torch.float8_e4m3fn:
        raise ValueError("fp8 inputs need per-tensor descales: use attn_fwd_ex")
    B, H, N, d, Hkv, dev = _check_qkv(q, k, v)
    dt = _DT[q.dtype]
    odt = torch.float32 if dt == DT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, H, N, d), dtype=odt, device=dev)
    _check_out(out, (B, H, N, d), odt, dev, "out")
    variant = variant_code(kind, interp=interp, window=window, flush=flush)
    st = (stream or torch.cuda.current_stream(dev)).cuda_stream
    with torch.cuda.device(dev):
        status = lib().qsa_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d, int(bool(causal)),
                                    variant, int(levels), float(window or 0.0), dt, ctypes.c_void_p(st))
    if status != OK:
        raise QSAError(status, last_error())
    return out


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, do: torch.Tensor, *, causal: bool = False,
             kind: str = "exact", levels: int = 0, window: Optional[float] = None, interp: bool = False,
             flush: bool = False, grad: str = "ste_post", scale: float = 0.0,
             stream: Optional[torch.cuda.Stream] = None):
    """Gradients (dq, dk, dv) of sum(do * O) through qsa_attn_bwd, O being attn_fwd of the
    same arguments.  q, do: [B,H,N,d]; k, v: [B,Hkv,N,d]; one dtype, float32 or bfloat16,
    contiguous, on one GPU.  The gradients are float32 (dk, dv summed over each KV head's
    query heads).  grad: one of GRADS.  Asynchronous on `stream` (default: the current one).
    """
    if grad not in GRADS:
        raise ValueError(f"grad must be one of {sorted(GRADS)}")
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d) or tuple(do.shape) != (B, H, N, d):
        raise ValueError("k, v must be [B, Hkv, N, d] and do [B, H, N, d]")
    if not (q.dtype == k.dtype == v.dtype == do.dtype) or q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("q, k, v, do must share one dtype, float32 or bfloat16")
    dev = q.device
    if k.device != dev or v.device != dev or do.device != dev:
        raise ValueError("q, k, v, do must be on the same GPU")
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev)
    dv = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev)
    variant = variant_code(kind, interp=interp, window=window, flush=flush)
    st = (stream or torch.cuda.current_stream(dev)).cuda_stream
    with torch.cuda.device(dev):
        status = lib().qsa_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv,
                                    N, d, int(bool(causal)), variant, int(levels), float(window or 0.0), _DT[q.dtype],
                                    GRADS[grad], float(scale), ctypes.c_void_p(st))
    if status != OK:
        raise QSAError(status, last_error())
    return dq, dk, dv
