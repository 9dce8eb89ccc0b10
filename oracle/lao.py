"""Python front of the CPU oracle (``lao.c``), fp64 numpy in and out.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library.  It imports
nothing from the product package.

Every function here is the plain token recurrence of decayed causal linear
attention (see the header of ``lao.c`` for the definition and the pages it
follows); this module only marshals arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lao.c")
# LAO_LIB names another build of lao.c to load instead (e.g. one made with
# the host sanitizers by the tests); build() never writes over it
_LIB = os.environ.get("LAO_LIB") or os.path.join(_HERE, "liblao.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math)."""
    if os.environ.get("LAO_LIB"):
        return _LIB
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def bind(lib):
    """Declare the C signatures on an opened oracle library and return it."""
    i64, dp, lp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.lao_fwd.argtypes = [i64] * 6 + [dp] * 7
    lib.lao_fwd.restype = ctypes.c_int
    lib.lao_fwd_rows.argtypes = [i64] * 6 + [dp] * 5 + [i64, lp, lp, dp]
    lib.lao_fwd_rows.restype = ctypes.c_int
    lib.lao_bwd.argtypes = [i64] * 6 + [dp] * 11
    lib.lao_bwd.restype = ctypes.c_int
    lib.lao_scan.argtypes = [i64] * 5 + [dp, dp, i64, dp, dp, dp, ctypes.c_int]
    lib.lao_scan.restype = ctypes.c_int
    lib.lao_fwd_gated.argtypes = [i64] * 6 + [dp] * 7
    lib.lao_fwd_gated.restype = ctypes.c_int
    lib.lao_scan_gated.argtypes = [i64] * 5 + [dp] * 5 + [ctypes.c_int]
    lib.lao_scan_gated.restype = ctypes.c_int
    lib.lao_bwd_gated.argtypes = [i64] * 6 + [dp] * 12
    lib.lao_bwd_gated.restype = ctypes.c_int
    lib.lao_threads.restype = ctypes.c_int
    lib.lao_threads.argtypes = []
    lib.lao_set_threads.restype = ctypes.c_int
    lib.lao_set_threads.argtypes = [ctypes.c_int]
    return lib


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().lao_threads())


def set_threads(n: int) -> int:
    """Run later oracle calls on n threads; returns the count in force."""
    return int(_load().lao_set_threads(int(n)))


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.ctypes.data)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with code {rc}")


def fwd(Q, K, V, lam, S0=None, nseg: int = 1, need_O: bool = True):
    """Token recurrence forward.

    Q, K: [B,H,L,dk]; V: [B,H,L,dv]; lam: [H]; S0: [B,H,nseg,dk,dv] or None.
    Returns (O [B,H,L,dv] or None, S_end [B,H,nseg,dk,dv]).
    """
    Q, K, V, lam, S0 = map(_f64, (Q, K, V, lam, S0))
    B, H, L, dk = Q.shape
    dv = V.shape[-1]
    O = np.empty((B, H, L, dv)) if need_O else None
    S_end = np.empty((B, H, nseg, dk, dv))
    rc = _load().lao_fwd(B, H, L, dk, dv, nseg, _ptr(Q), _ptr(K), _ptr(V),
                         _ptr(lam), _ptr(S0), _ptr(O), _ptr(S_end))
    _check(rc, "fwd")
    return O, S_end


def fwd_rows(Q, K, V, lam, seq, rows, S0=None, nseg: int = 1):
    """Selected output rows by direct summation (cost O(t*d) per row).

    seq, rows: int arrays of equal length; seq indexes the flattened
    [B*H*nseg] segment axis and rows the 0-based token inside that segment.
    Returns [len(rows), dv].
    """
    Q, K, V, lam, S0 = map(_f64, (Q, K, V, lam, S0))
    B, H, L, dk = Q.shape
    dv = V.shape[-1]
    seq = np.ascontiguousarray(np.asarray(seq, dtype=np.int64))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((rows.shape[0], dv))
    rc = _load().lao_fwd_rows(B, H, L, dk, dv, nseg, _ptr(Q), _ptr(K), _ptr(V),
                              _ptr(lam), _ptr(S0), rows.shape[0], _ptr(seq),
                              _ptr(rows), _ptr(out))
    _check(rc, "fwd_rows")
    return out


def bwd(Q, K, V, lam, dO, S0=None, dS_end=None, nseg: int = 1):
    """Backward of the recurrence; returns (dQ, dK, dV, dS0)."""
    Q, K, V, lam, dO, S0, dS_end = map(_f64, (Q, K, V, lam, dO, S0, dS_end))
    B, H, L, dk = Q.shape
    dv = V.shape[-1]
    dQ = np.empty((B, H, L, dk))
    dK = np.empty((B, H, L, dk))
    dV = np.empty((B, H, L, dv))
    dS0 = np.empty((B, H, nseg, dk, dv))
    rc = _load().lao_bwd(B, H, L, dk, dv, nseg, _ptr(Q), _ptr(K), _ptr(V),
                         _ptr(lam), _ptr(S0), _ptr(dO), _ptr(dS_end),
                         _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dS0))
    _check(rc, "bwd")
    return dQ, dK, dV, dS0


def scan(dS, lam, seg_len: int, S0=None, reverse: bool = False):
    """Segment state-combine scan.

    dS: [B,H,P,dk,dv]; lam: [H]; S0: [B,H,dk,dv] or None.
    Returns (S_start [B,H,P,dk,dv], S_end [B,H,dk,dv]).
    """
    dS, lam, S0 = map(_f64, (dS, lam, S0))
    B, H, P, dk, dv = dS.shape
    S_start = np.empty_like(dS)
    S_end = np.empty((B, H, dk, dv))
    rc = _load().lao_scan(B, H, P, dk, dv, _ptr(dS), _ptr(lam), int(seg_len),
                          _ptr(S0), _ptr(S_start), _ptr(S_end), int(bool(reverse)))
    _check(rc, "scan")
    return S_start, S_end


def fwd_gated(Q, K, V, G, S0=None, nseg: int = 1, need_O: bool = True):
    """Gated token recurrence forward: S_t = exp(g_t) S_{t-1} + k_t v_t^T.

    Q, K: [B,H,L,dk]; V: [B,H,L,dv]; G = log alpha: [B,H,L];
    S0: [B,H,nseg,dk,dv] or None.  Returns (O or None, S_end [B,H,nseg,dk,dv]).
    """
    Q, K, V, G, S0 = map(_f64, (Q, K, V, G, S0))
    B, H, L, dk = Q.shape
    dv = V.shape[-1]
    O = np.empty((B, H, L, dv)) if need_O else None
    S_end = np.empty((B, H, nseg, dk, dv))
    rc = _load().lao_fwd_gated(B, H, L, dk, dv, nseg, _ptr(Q), _ptr(K), _ptr(V),
                               _ptr(G), _ptr(S0), _ptr(O), _ptr(S_end))
    _check(rc, "fwd_gated")
    return O, S_end


def scan_gated(dS, LD, S0=None, reverse: bool = False):
    """Segment combine with per-segment log decays LD [B,H,P].

    dS: [B,H,P,dk,dv]; S0: [B,H,dk,dv] or None.
    Returns (S_start [B,H,P,dk,dv], S_end [B,H,dk,dv]).
    """
    dS, LD, S0 = map(_f64, (dS, LD, S0))
    B, H, P, dk, dv = dS.shape
    S_start = np.empty_like(dS)
    S_end = np.empty((B, H, dk, dv))
    rc = _load().lao_scan_gated(B, H, P, dk, dv, _ptr(dS), _ptr(LD), _ptr(S0),
                                _ptr(S_start), _ptr(S_end), int(bool(reverse)))
    _check(rc, "scan_gated")
    return S_start, S_end


def bwd_gated(Q, K, V, G, dO, S0=None, dS_end=None, nseg: int = 1):
    """Backward of the gated recurrence; returns (dQ, dK, dV, dS0, dG) with
    dG = d loss / d log(alpha) [B,H,L]."""
    Q, K, V, G, dO, S0, dS_end = map(_f64, (Q, K, V, G, dO, S0, dS_end))
    B, H, L, dk = Q.shape
    dv = V.shape[-1]
    dQ = np.empty((B, H, L, dk))
    dK = np.empty((B, H, L, dk))
    dV = np.empty((B, H, L, dv))
    dS0 = np.empty((B, H, nseg, dk, dv))
    dG = np.empty((B, H, L))
    rc = _load().lao_bwd_gated(B, H, L, dk, dv, nseg, _ptr(Q), _ptr(K), _ptr(V), _ptr(G),
                               _ptr(S0), _ptr(dO), _ptr(dS_end), _ptr(dQ), _ptr(dK), _ptr(dV),
                               _ptr(dS0), _ptr(dG))
    _check(rc, "bwd_gated")
    return dQ, dK, dV, dS0, dG


def dlambda(Q, K, V, lam, dO, S0=None, dS_end=None, nseg: int = 1):
    """Gradient of the loss sum_t <do_t, o_t> + <dS_end, S_end> with respect
    to the per-head decay lambda [H]: every token's gate is lambda_h, so by
    the chain rule dl/dlambda_h = sum over the head's tokens of
    d l / d log(alpha_t) divided by lambda_h (the gated backward with
    constant gates)."""
    Q = _f64(Q)
    B, H, L, _ = Q.shape
    lam = _f64(lam)
    G = np.broadcast_to(np.log(lam)[None, :, None], (B, H, L)).copy()
    dG = bwd_gated(Q, K, V, G, dO, S0=S0, dS_end=dS_end, nseg=nseg)[4]
    return dG.sum(axis=(0, 2)) / lam


def step(q, k, v, lam, S=None):
    """One token of the recurrence for every (b, h): S' = lambda_h S + k v^T,
    o = q^T S' (the recurrent, constant-memory form of the LASP-2 page's
    abstract; the same update as the token loop of ``lao.c``).  q, k [B,H,dk],
    v [B,H,dv], lam [H], S [B,H,dk,dv] (None = zero).  Returns (o, S')."""
    q, k, v, lam = _f64(q), _f64(k), _f64(v), _f64(lam)
    B, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S is None else _f64(S)
    S1 = np.empty((B, H, dk, dv))
    o = np.empty((B, H, dv))
    for b in range(B):
        for h in range(H):
            S1[b, h] = lam[h] * S[b, h] + np.outer(k[b, h], v[b, h])
            o[b, h] = q[b, h] @ S1[b, h]
    return o, S1
