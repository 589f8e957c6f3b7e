"""fp64 CPU oracle for exact attention (forward and backward).

TEST INFRASTRUCTURE ONLY: the parity oracle of the GPU library. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it. It shares no code with the
GPU library (its arithmetic lives in ``oracle.c``; this module only marshals numpy arrays).

The oracle is the standard definition of scaled dot-product attention, which the pages give
as the exact result FlashAttention-2 reproduces ("Flash Attention spiegata: una guida
completa", section "Attention standard vs Flash attention"). See ``oracle.c`` for the
formulas. Inputs are float64 arrays (the bf16 inputs of a test are widened exactly before
they get here); outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def compile_library(src: str, out: str) -> str:
    """gcc a copy of the oracle source into a shared library. No fast-math: sums keep index order."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src,
                           "-lm", "-lpthread"])
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile liboracle.so in-tree."""
    return compile_library(_SRC, _LIB_PATH)


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, p, dbl, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
    lib.oracle_forward.restype = cint
    lib.oracle_forward.argtypes = [p, p, p, i64, i64, i64, i64, i64, cint, i64, dbl, p, i64, p, p, cint]
    lib.oracle_row_stats.restype = cint
    lib.oracle_row_stats.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, cint, i64, dbl, p, i64, p, p, p,
                                     cint]
    lib.oracle_backward_dq.restype = cint
    lib.oracle_backward_dq.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, cint, i64, dbl, p, p, i64, p,
                                       cint]
    lib.oracle_backward_dkdv.restype = cint
    lib.oracle_backward_dkdv.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, cint, i64, dbl, p, p, p, p,
                                         i64, p, p, cint]
    lib.oracle_decode.restype = cint
    lib.oracle_decode.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, cint, dbl, p, p]
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _shapes(q, k):
    if q.ndim != 4 or k.ndim != 4:
        raise ValueError("q, k, v must be [B,H,N,d]")
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or Hkv < 1 or Hq % Hkv:
        raise ValueError("inconsistent shapes q %s k %s" % (q.shape, k.shape))
    return B, Hq, Hkv, N, d


def _rows(rows, nslices, N):
    if rows is None:
        r = np.tile(np.arange(N, dtype=np.int32), (nslices, 1))
    else:
        r = np.asarray(rows, dtype=np.int32)
        if r.ndim == 1:
            r = np.tile(r, (nslices, 1))
        if r.shape[0] != nslices:
            raise ValueError("rows must be [slices, k] or [k]")
    return np.ascontiguousarray(r)


class Oracle:
    """The oracle bound to one compiled copy of ``oracle.c``."""

    def __init__(self, lib_path: str):
        self.lib = _bind(lib_path)

    def forward(self, q, k, v, causal: bool, scale: float, rows=None, threads: int | None = None,
                window: int = -1):
        """O [B,Hq,R,d] and LSE [B,Hq,R] (natural log) for query rows ``rows`` (all if None).

        ``rows`` is [R] (same rows in every (b,hq) slice) or [B*Hq, R]. ``window`` >= 0 (with
        ``causal``) restricts row i to keys i - window .. i.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, N, d = _shapes(q, k)
        r = _rows(rows, B * Hq, N)
        R = r.shape[1]
        o = np.empty((B, Hq, R, d), dtype=np.float64)
        lse = np.empty((B, Hq, R), dtype=np.float64)
        rc = self.lib.oracle_forward(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, Hq, Hkv, N, d,
                                    int(bool(causal)), int(window), float(scale), r.ctypes.data, R,
                                    o.ctypes.data, lse.ctypes.data, threads or default_threads())
        if rc:
            raise RuntimeError("oracle_forward failed (%d)" % rc)
        return o, lse

    def row_stats(self, q, k, v, dO, causal: bool, scale: float, threads: int | None = None,
                  window: int = -1, rows=None):
        """(m, l, D), each [B,Hq,R]: row max, softmax denominator, and sum_j P_ij dP_ij of the
        query rows ``rows`` (all N rows if None; same forms as in :func:`forward`)."""
        q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
        B, Hq, Hkv, N, d = _shapes(q, k)
        r = _rows(rows, B * Hq, N)
        R = r.shape[1]
        m = np.empty((B, Hq, R)); l = np.empty((B, Hq, R)); D = np.empty((B, Hq, R))
        rc = self.lib.oracle_row_stats(q.ctypes.data, k.ctypes.data, v.ctypes.data, dO.ctypes.data,
                                      B, Hq, Hkv, N, d, int(bool(causal)), int(window), float(scale),
                                      r.ctypes.data, R, m.ctypes.data, l.ctypes.data, D.ctypes.data,
                                      threads or default_threads())
        if rc:
            raise RuntimeError("oracle_row_stats failed (%d)" % rc)
        return m, l, D

    def backward(self, q, k, v, dO, causal: bool, scale: float, qrows=None, krows=None,
                 threads: int | None = None, stats=None, window: int = -1):
        """dQ [B,Hq,Rq,d] for query rows ``qrows``; dK, dV [B,Hkv,Rk,d] for key rows ``krows``.

        Row arguments take the same forms as in :func:`forward` (slices are (b,hq) for qrows and
        (b,hkv) for krows). Returns (dq, dk, dv, (m, l, D)).
        """
        q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
        B, Hq, Hkv, N, d = _shapes(q, k)
        nt = threads or default_threads()
        if stats is None:
            stats = self.row_stats(q, k, v, dO, causal, scale, threads=nt, window=window)
        m, l, D = (np.ascontiguousarray(x, dtype=np.float64) for x in stats)
        rq = _rows(qrows, B * Hq, N)
        rk = _rows(krows, B * Hkv, N)
        dq = np.empty((B, Hq, rq.shape[1], d))
        dk = np.empty((B, Hkv, rk.shape[1], d))
        dv = np.empty((B, Hkv, rk.shape[1], d))
        lib = self.lib
        rc = lib.oracle_backward_dq(q.ctypes.data, k.ctypes.data, v.ctypes.data, dO.ctypes.data,
                                    B, Hq, Hkv, N, d, int(bool(causal)), int(window), float(scale),
                                    D.ctypes.data,
                                    rq.ctypes.data, rq.shape[1], dq.ctypes.data, nt)
        if rc:
            raise RuntimeError("oracle_backward_dq failed (%d)" % rc)
        rc = lib.oracle_backward_dkdv(q.ctypes.data, k.ctypes.data, v.ctypes.data, dO.ctypes.data,
                                      B, Hq, Hkv, N, d, int(bool(causal)), int(window), float(scale),
                                      m.ctypes.data, l.ctypes.data, D.ctypes.data,
                                      rk.ctypes.data, rk.shape[1], dk.ctypes.data, dv.ctypes.data, nt)
        if rc:
            raise RuntimeError("oracle_backward_dkdv failed (%d)" % rc)
        return dq, dk, dv, (m, l, D)


    def decode(self, q, k, v, causal: bool, scale: float):
        """O [B,Hq,Nq,d] and LSE [B,Hq,Nq] of Nq query rows against Nk cached keys; causal rows
        are aligned to the end of the cache (row i sees keys j <= Nk - Nq + i)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
            raise ValueError("q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d]")
        B, Hq, Nq, d = q.shape
        Bk, Hkv, Nk, dk = k.shape
        if (Bk, dk) != (B, d) or Hq % Hkv:
            raise ValueError("inconsistent shapes q %s k %s" % (q.shape, k.shape))
        o = np.empty((B, Hq, Nq, d))
        lse = np.empty((B, Hq, Nq))
        rc = self.lib.oracle_decode(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, Hq, Hkv, Nq, Nk, d,
                                    int(bool(causal)), float(scale), o.ctypes.data, lse.ctypes.data)
        if rc:
            raise RuntimeError("oracle_decode failed (%d)" % rc)
        return o, lse


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def forward(q, k, v, causal: bool, scale: float, rows=None, threads: int | None = None, window: int = -1):
    return default().forward(q, k, v, causal, scale, rows=rows, threads=threads, window=window)


def row_stats(q, k, v, dO, causal: bool, scale: float, threads: int | None = None, window: int = -1,
              rows=None):
    return default().row_stats(q, k, v, dO, causal, scale, threads=threads, window=window, rows=rows)


def backward(q, k, v, dO, causal: bool, scale: float, qrows=None, krows=None,
             threads: int | None = None, stats=None, window: int = -1):
    return default().backward(q, k, v, dO, causal, scale, qrows=qrows, krows=krows,
                              threads=threads, stats=stats, window=window)


def decode(q, k, v, causal: bool, scale: float):
    return default().decode(q, k, v, causal, scale)


def forward_flops(B: int, Hq: int, N: int, d: int, causal: bool, nrows: int | None = None) -> float:
    """Counted FLOPs of a forward over ``nrows`` rows per slice (4*N*d per full row, halved if causal)."""
    rows = N if nrows is None else nrows
    f = 4.0 * B * Hq * rows * N * d
    return f / 2 if causal else f
