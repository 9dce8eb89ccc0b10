"""ctypes binding of liblinattn.so (C ABI in ``include/linattn.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch provides device memory (outputs and the
workspace are torch allocations) and the stream (the current torch stream).
There is no fallback: if the library is missing or cannot be loaded, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblinattn.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_HIP = range(5)
LA_BF16, LA_FP32 = 0, 1

EXPORTS = ("la_version", "la_status_str", "la_last_error", "la_fwd_workspace_bytes",
           "la_chunk_fwd", "la_state_scan", "la_bwd_workspace_bytes", "la_chunk_bwd",
           "la_fwd_gated_workspace_bytes", "la_chunk_fwd_gated", "la_state_scan_gated",
           "la_bwd_gated_workspace_bytes", "la_chunk_bwd_gated",
           "la_decay_grad_workspace_bytes", "la_decay_grad", "la_step", "la_chunk_bwd_from_fwd",
           "la_chunk_bwd_gated_from_fwd", "la_step_gated", "la_chunk_fwd_noalloc")


class LinAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class la_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("L", ctypes.c_int64),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("nseg", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("split", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m long_sequence_causal_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    sp = ctypes.POINTER(la_shape)
    L.la_version.restype = ctypes.c_int
    L.la_version.argtypes = []
    L.la_status_str.restype = ctypes.c_char_p
    L.la_status_str.argtypes = [ctypes.c_int]
    L.la_last_error.restype = ctypes.c_char_p
    L.la_last_error.argtypes = []
    L.la_fwd_workspace_bytes.restype = sz
    L.la_fwd_workspace_bytes.argtypes = [sp]
    L.la_bwd_workspace_bytes.restype = sz
    L.la_bwd_workspace_bytes.argtypes = [sp]
    L.la_chunk_fwd.restype = ctypes.c_int
    L.la_chunk_fwd.argtypes = [sp] + [vp] * 8 + [sz, vp]
    L.la_state_scan.restype = ctypes.c_int
    L.la_state_scan.argtypes = [i64, i64, i32, i32, i32, vp, vp, i64, vp, vp, vp, i32, vp]
    L.la_chunk_bwd.restype = ctypes.c_int
    L.la_chunk_bwd.argtypes = [sp] + [vp] * 12 + [sz, vp]
    L.la_fwd_gated_workspace_bytes.restype = sz
    L.la_fwd_gated_workspace_bytes.argtypes = [sp]
    L.la_chunk_fwd_gated.restype = ctypes.c_int
    L.la_chunk_fwd_gated.argtypes = [sp] + [vp] * 8 + [sz, vp]
    L.la_bwd_gated_workspace_bytes.restype = sz
    L.la_bwd_gated_workspace_bytes.argtypes = [sp]
    L.la_chunk_bwd_gated.restype = ctypes.c_int
    L.la_chunk_bwd_gated.argtypes = [sp] + [vp] * 13 + [sz, vp]
    L.la_chunk_bwd_gated_from_fwd.restype = ctypes.c_int
    L.la_chunk_bwd_gated_from_fwd.argtypes = [sp] + [vp] * 14 + [sz, vp]
    L.la_state_scan_gated.restype = ctypes.c_int
    L.la_state_scan_gated.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp]
    L.la_chunk_bwd_from_fwd.restype = ctypes.c_int
    L.la_chunk_bwd_from_fwd.argtypes = [sp] + [vp] * 13 + [sz, vp]
    L.la_step.restype = ctypes.c_int
    L.la_step.argtypes = [i64, i64, i32, i32, i32] + [vp] * 7 + [vp]
    L.la_step_gated.restype = ctypes.c_int
    L.la_step_gated.argtypes = [i64, i64, i32, i32, i32] + [vp] * 7 + [vp]
    L.la_decay_grad_workspace_bytes.restype = sz
    L.la_decay_grad_workspace_bytes.argtypes = [sp]
    L.la_decay_grad.restype = ctypes.c_int
    L.la_decay_grad.argtypes = [sp] + [vp] * 9 + [sz, vp]
    L.la_chunk_fwd_noalloc.restype = ctypes.c_int
    L.la_chunk_fwd_noalloc.argtypes = [sp] + [vp] * 8
    _lib = L
    return L


def _check(status: int):
    if status != LA_OK:
        L = lib()
        msg = L.la_last_error().decode()
        raise LinAttnError(status, msg or L.la_status_str(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return LA_BF16
    if dt == torch.float32:
        return LA_FP32
    raise TypeError(f"unsupported token dtype {dt}")


def _need(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _expect_all(device, *specs):
    """Each (tensor, name, shape, dtype) with a tensor given must have exactly
    `shape` -- the kernels index every buffer by the sizes passed through the C
    ABI, which cannot see tensor extents -- and be a contiguous `dtype` tensor
    on `device`.  Every shape is checked before any dtype or device."""
    for t, name, shape, _ in specs:
        if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    for t, name, _, dtype in specs:
        if t is None:
            continue
        _need(t, name, dtype)
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _out_specs(out, names, shapes, dtypes):
    """_expect_all specs of a tuple of preallocated outputs (none if out is None)."""
    if out is None:
        return ()
    if len(out) != len(names):
        raise ValueError(f"out must hold {len(names)} tensors ({', '.join(names)})")
    return tuple(zip(out, names, shapes, dtypes))


def make_shape(B, H, L, dk, dv, nseg=1, dtype=LA_BF16, split=0) -> la_shape:
    return la_shape(int(B), int(H), int(L), int(dk), int(dv), int(nseg), int(dtype),
                    int(split), 0)


def la_fwd_workspace_bytes(shape: la_shape) -> int:
    return int(lib().la_fwd_workspace_bytes(ctypes.byref(shape)))


def la_bwd_workspace_bytes(shape: la_shape) -> int:
    return int(lib().la_bwd_workspace_bytes(ctypes.byref(shape)))


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def la_chunk_fwd(q, k, v, lam, S0=None, nseg: int = 1, need_O: bool = True,
                 need_S_end: bool = True, split: int = 0, out=None, S_end_out=None,
                 workspace=None):
    """Forward pass.  q, k [B,H,L,dk], v [B,H,L,dv] (bf16 or fp32), lam [H] fp32,
    S0 [B,H,nseg,dk,dv] fp32 or None.  Returns (O or None, S_end or None)."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    dev = q.device
    _expect_all(
        dev,
        (q, "q", (B, H, L, dk), q.dtype),
        (k, "k", (B, H, L, dk), q.dtype),
        (v, "v", (B, H, L, dv), q.dtype),
        (lam, "lam", (H,), torch.float32),
        (S0, "S0", (B, H, nseg, dk, dv), torch.float32),
        (out, "out", (B, H, L, dv), q.dtype),
        (S_end_out, "S_end_out", (B, H, nseg, dk, dv), torch.float32))
    shape = make_shape(B, H, L, dk, dv, nseg, dt, split)
    O = None
    if need_O:
        O = out if out is not None else torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    S_end = None
    if need_S_end:
        S_end = S_end_out if S_end_out is not None else torch.empty(
            (B, H, nseg, dk, dv), dtype=torch.float32, device=q.device)
    nbytes = la_fwd_workspace_bytes(shape)
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    _check(lib().la_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                              _ptr(S0), _ptr(O), _ptr(S_end), _ptr(ws),
                              ws.numel() if ws is not None else 0, _stream()))
    return O, S_end


def la_chunk_fwd_noalloc(q, k, v, lam, O, S_end, S0=None, nseg: int = 1, split: int = 0):
    """la_chunk_fwd into preallocated O and/or S_end (either may be None, not
    both) with the library's fixed scratch array instead of a workspace: no
    device memory is allocated by this call."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    _expect_all(
        q.device,
        (q, "q", (B, H, L, dk), q.dtype),
        (k, "k", (B, H, L, dk), q.dtype),
        (v, "v", (B, H, L, dv), q.dtype),
        (lam, "lam", (H,), torch.float32),
        (S0, "S0", (B, H, nseg, dk, dv), torch.float32),
        (O, "O", (B, H, L, dv), q.dtype),
        (S_end, "S_end", (B, H, nseg, dk, dv), torch.float32))
    shape = make_shape(B, H, L, dk, dv, nseg, dt, split)
    _check(lib().la_chunk_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                                      _ptr(S0), _ptr(O), _ptr(S_end), _stream()))
    return O, S_end


def la_fwd_gated_workspace_bytes(shape: la_shape) -> int:
    return int(lib().la_fwd_gated_workspace_bytes(ctypes.byref(shape)))


def la_chunk_fwd_gated(q, k, v, log_alpha, S0=None, nseg: int = 1, need_O: bool = True,
                       need_S_end: bool = True, split: int = 0, out=None, S_end_out=None,
                       workspace=None):
    """Gated forward pass.  As la_chunk_fwd with log_alpha [B,H,L] fp32 (the
    log of the per-token gates) in place of lam.  Returns (O or None, S_end or None)."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    dev = q.device
    _expect_all(
        dev,
        (q, "q", (B, H, L, dk), q.dtype),
        (k, "k", (B, H, L, dk), q.dtype),
        (v, "v", (B, H, L, dv), q.dtype),
        (log_alpha, "log_alpha", (B, H, L), torch.float32),
        (S0, "S0", (B, H, nseg, dk, dv), torch.float32),
        (out, "out", (B, H, L, dv), q.dtype),
        (S_end_out, "S_end_out", (B, H, nseg, dk, dv), torch.float32))
    shape = make_shape(B, H, L, dk, dv, nseg, dt, split)
    O = None
    if need_O:
        O = out if out is not None else torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    S_end = None
    if need_S_end:
        S_end = S_end_out if S_end_out is not None else torch.empty(
            (B, H, nseg, dk, dv), dtype=torch.float32, device=q.device)
    nbytes = la_fwd_gated_workspace_bytes(shape)
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    _check(lib().la_chunk_fwd_gated(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(log_alpha), _ptr(S0), _ptr(O), _ptr(S_end), _ptr(ws),
                                    ws.numel() if ws is not None else 0, _stream()))
    return O, S_end


def la_state_scan_gated(dS, log_decay, S0=None, reverse: bool = False, out=None,
                        need_S_end: bool = True, S_end_out=None):
    """Gated segment combine.  dS [B,H,P,dk,dv] fp32, log_decay [B,H,P] fp32,
    S0 [B,H,dk,dv] or None.  Returns (S_start, S_end or None)."""
    B, H, P, dk, dv = dS.shape
    dev = dS.device
    _expect_all(
        dev,
        (dS, "dS", (B, H, P, dk, dv), torch.float32),
        (log_decay, "log_decay", (B, H, P), torch.float32),
        (S0, "S0", (B, H, dk, dv), torch.float32),
        (out, "out", (B, H, P, dk, dv), torch.float32),
        (S_end_out, "S_end_out", (B, H, dk, dv), torch.float32))
    S_start = out if out is not None else torch.empty_like(dS)
    if S_end_out is not None:
        S_end = S_end_out
    else:
        S_end = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dS.device) if need_S_end else None
    _check(lib().la_state_scan_gated(B, H, P, dk, dv, _ptr(dS), _ptr(log_decay), _ptr(S0),
                                     _ptr(S_start), _ptr(S_end), int(bool(reverse)), _stream()))
    return S_start, S_end


def la_state_scan(dS, lam, seg_len: int, S0=None, reverse: bool = False, out=None,
                  need_S_end: bool = True, S_end_out=None):
    """Segment scan.  dS [B,H,P,dk,dv] fp32, lam [H], S0 [B,H,dk,dv] or None.
    Returns (S_start [B,H,P,dk,dv], S_end [B,H,dk,dv] or None); ``out`` may be dS."""
    B, H, P, dk, dv = dS.shape
    dev = dS.device
    _expect_all(
        dev,
        (dS, "dS", (B, H, P, dk, dv), torch.float32),
        (lam, "lam", (H,), torch.float32),
        (S0, "S0", (B, H, dk, dv), torch.float32),
        (out, "out", (B, H, P, dk, dv), torch.float32),
        (S_end_out, "S_end_out", (B, H, dk, dv), torch.float32))
    S_start = out if out is not None else torch.empty_like(dS)
    if S_end_out is not None:
        S_end = S_end_out
    else:
        S_end = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dS.device) if need_S_end else None
    _check(lib().la_state_scan(B, H, P, dk, dv, _ptr(dS), _ptr(lam), int(seg_len), _ptr(S0),
                               _ptr(S_start), _ptr(S_end), int(bool(reverse)), _stream()))
    return S_start, S_end


def la_chunk_bwd(q, k, v, lam, dO, S0=None, dS_end=None, nseg: int = 1,
                 need_dS0: bool = True, split: int = 0, workspace=None, out=None,
                 fwd_workspace=None):
    """Backward pass.  Returns (dQ, dK, dV, dS0 or None).  `out`, if given, is
    a (dQ, dK, dV, dS0-or-None) tuple of preallocated outputs.  With
    `fwd_workspace` (the workspace tensor a la_chunk_fwd call with the same
    shape and inputs just used) the call goes to la_chunk_bwd_from_fwd, which
    reuses that call's sub-segment start states."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    dev = q.device
    _expect_all(
        dev,
        (q, "q", (B, H, L, dk), q.dtype),
        (k, "k", (B, H, L, dk), q.dtype),
        (v, "v", (B, H, L, dv), q.dtype),
        (dO, "dO", (B, H, L, dv), q.dtype),
        (lam, "lam", (H,), torch.float32),
        (S0, "S0", (B, H, nseg, dk, dv), torch.float32),
        (dS_end, "dS_end", (B, H, nseg, dk, dv), torch.float32),
        *_out_specs(out, ("dQ", "dK", "dV", "dS0"),
                    ((B, H, L, dk), (B, H, L, dk), (B, H, L, dv), (B, H, nseg, dk, dv)),
                    (q.dtype, q.dtype, q.dtype, torch.float32)))
    shape = make_shape(B, H, L, dk, dv, nseg, dt, split)
    if out is not None:
        dQ, dK, dV, dS0 = out
    else:
        dQ = torch.empty_like(q)
        dK = torch.empty_like(k)
        dV = torch.empty_like(v)
        dS0 = torch.empty((B, H, nseg, dk, dv), dtype=torch.float32, device=q.device) if need_dS0 else None
    nbytes = la_bwd_workspace_bytes(shape)
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    nws = ws.numel() if ws is not None else 0
    if fwd_workspace is not None:
        need = la_fwd_workspace_bytes(shape)
        if fwd_workspace.numel() * fwd_workspace.element_size() < need:
            raise ValueError(f"fwd_workspace holds fewer than the {need} bytes of this shape's plan")
        _need(fwd_workspace, "fwd_workspace")
        _check(lib().la_chunk_bwd_from_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(lam), _ptr(S0), _ptr(dO), _ptr(dS_end),
                                           _ptr(fwd_workspace), _ptr(dQ), _ptr(dK), _ptr(dV),
                                           _ptr(dS0), _ptr(ws), nws, _stream()))
    else:
        _check(lib().la_chunk_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
                                  _ptr(S0), _ptr(dO), _ptr(dS_end), _ptr(dQ), _ptr(dK), _ptr(dV),
                                  _ptr(dS0), _ptr(ws), nws, _stream()))
    return dQ, dK, dV, dS0


def la_bwd_gated_workspace_bytes(shape: la_shape) -> int:
    return int(lib().la_bwd_gated_workspace_bytes(ctypes.byref(shape)))


def la_chunk_bwd_gated(q, k, v, log_alpha, dO, S0=None, dS_end=None, nseg: int = 1,
                       need_dS0: bool = True, need_dlog_alpha: bool = True, split: int = 0,
                       workspace=None, out=None, fwd_workspace=None):
    """Backward of the gated forward.  Returns (dQ, dK, dV, dS0 or None,
    dlog_alpha or None); `out` may give all five preallocated (None entries
    are not returned).  With `fwd_workspace` (the workspace tensor a
    la_chunk_fwd_gated call with the same shape and inputs just used) the call
    goes to la_chunk_bwd_gated_from_fwd."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    dev = q.device
    _expect_all(
        dev,
        (q, "q", (B, H, L, dk), q.dtype),
        (k, "k", (B, H, L, dk), q.dtype),
        (v, "v", (B, H, L, dv), q.dtype),
        (dO, "dO", (B, H, L, dv), q.dtype),
        (log_alpha, "log_alpha", (B, H, L), torch.float32),
        (S0, "S0", (B, H, nseg, dk, dv), torch.float32),
        (dS_end, "dS_end", (B, H, nseg, dk, dv), torch.float32),
        *_out_specs(out, ("dQ", "dK", "dV", "dS0", "dlog_alpha"),
                    ((B, H, L, dk), (B, H, L, dk), (B, H, L, dv), (B, H, nseg, dk, dv), (B, H, L)),
                    (q.dtype, q.dtype, q.dtype, torch.float32, torch.float32)))
    shape = make_shape(B, H, L, dk, dv, nseg, dt, split)
    if out is not None:
        dQ, dK, dV, dS0, dG = out
    else:
        dQ, dK, dV = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dS0 = torch.empty((B, H, nseg, dk, dv), dtype=torch.float32, device=q.device) if need_dS0 else None
        dG = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if need_dlog_alpha else None
    nbytes = la_bwd_gated_workspace_bytes(shape)
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    nws = ws.numel() if ws is not None else 0
    if fwd_workspace is not None:
        need = la_fwd_gated_workspace_bytes(shape)
        if fwd_workspace.numel() * fwd_workspace.element_size() < need:
            raise ValueError(f"fwd_workspace holds fewer than the {need} bytes of this shape's plan")
        _need(fwd_workspace, "fwd_workspace")
        _check(lib().la_chunk_bwd_gated_from_fwd(
            ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(S0), _ptr(dO),
            _ptr(dS_end), _ptr(fwd_workspace), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dS0), _ptr(dG),
            _ptr(ws), nws, _stream()))
    else:
        _check(lib().la_chunk_bwd_gated(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(log_alpha), _ptr(S0), _ptr(dO), _ptr(dS_end),
                                        _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dS0), _ptr(dG),
                                        _ptr(ws), nws, _stream()))
    return dQ, dK, dV, dS0, dG


def la_decay_grad_workspace_bytes(shape: la_shape) -> int:
    return int(lib().la_decay_grad_workspace_bytes(ctypes.byref(shape)))


def la_decay_grad(q, k, v, lam, dO, S0=None, dS_end=None, nseg: int = 1, split: int = 0,
                  workspace=None, out=None):
    """Gradient [H] fp32 of l = sum_t <dO_t, o_t> + <dS_end, S_end> with
    respect to the per-head decays lam, summed over the batch and segments."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    dev = q.device
    _expect_all(
        dev,
        (q, "q", (B, H, L, dk), q.dtype),
        (k, "k", (B, H, L, dk), q.dtype),
        (v, "v", (B, H, L, dv), q.dtype),
        (dO, "dO", (B, H, L, dv), q.dtype),
        (lam, "lam", (H,), torch.float32),
        (S0, "S0", (B, H, nseg, dk, dv), torch.float32),
        (dS_end, "dS_end", (B, H, nseg, dk, dv), torch.float32),
        (out, "out", (H,), torch.float32))
    shape = make_shape(B, H, L, dk, dv, nseg, dt, split)
    dlam = out if out is not None else torch.empty((H,), dtype=torch.float32, device=q.device)
    nbytes = la_decay_grad_workspace_bytes(shape)
    ws = workspace if workspace is not None else _workspace(nbytes, q.device)
    _check(lib().la_decay_grad(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S0),
                               _ptr(dO), _ptr(dS_end), _ptr(dlam), _ptr(ws),
                               ws.numel() if ws is not None else 0, _stream()))
    return dlam


def la_step(q, k, v, lam, S=None, out=None, S_out=None, need_o: bool = True):
    """One decode step: S' = lam_h S + k v^T, o = q^T S' for q, k [B,H,dk],
    v [B,H,dv] and S [B,H,dk,dv] fp32 (None = zero).  S_out may be S (in
    place).  Returns (o or None, S')."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    dev = q.device
    _expect_all(
        dev,
        (q, "q", (B, H, dk), q.dtype),
        (k, "k", (B, H, dk), q.dtype),
        (v, "v", (B, H, dv), q.dtype),
        (lam, "lam", (H,), torch.float32),
        (S, "S", (B, H, dk, dv), torch.float32),
        (S_out, "S_out", (B, H, dk, dv), torch.float32),
        (out, "out", (B, H, dv), q.dtype))
    if S_out is None:
        S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    o = out if out is not None else (
        torch.empty((B, H, dv), dtype=q.dtype, device=q.device) if need_o else None)
    _check(lib().la_step(B, H, dk, dv, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(S),
                         _ptr(S_out), _ptr(o), _stream()))
    return o, S_out


def la_step_gated(q, k, v, log_alpha, S=None, out=None, S_out=None, need_o: bool = True):
    """One gated decode step: S' = exp(log_alpha) S + k v^T, o = q^T S' for
    q, k [B,H,dk], v [B,H,dv], log_alpha [B,H] fp32 (the token's log-gate per
    sequence and head) and S [B,H,dk,dv] fp32 (None = zero).  S_out may be S
    (in place).  Returns (o or None, S')."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    dev = q.device
    _expect_all(
        dev,
        (q, "q", (B, H, dk), q.dtype),
        (k, "k", (B, H, dk), q.dtype),
        (v, "v", (B, H, dv), q.dtype),
        (log_alpha, "log_alpha", (B, H), torch.float32),
        (S, "S", (B, H, dk, dv), torch.float32),
        (S_out, "S_out", (B, H, dk, dv), torch.float32),
        (out, "out", (B, H, dv), q.dtype))
    if S_out is None:
        S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    o = out if out is not None else (
        torch.empty((B, H, dv), dtype=q.dtype, device=q.device) if need_o else None)
    _check(lib().la_step_gated(B, H, dk, dv, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                               _ptr(S), _ptr(S_out), _ptr(o), _stream()))
    return o, S_out
