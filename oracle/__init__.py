"""CPU oracle for the MoDA forward (fp64, plain C + OpenMP).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and the HIP library never calls it.

What it computes is the plain definition of Mixture-of-Depths Attention
(hyper.ai page on arXiv 2603.15619, section "Mixture-of-Depths Attention
(MoDA)"; chatpaper.ai abstract): for every query row (b, h, t) one softmax,
scaled by 1/sqrt(d), over the causal sequence keys 0..t of KV head h // G and
the L depth keys of token t, followed by the weighted sum of the matching
values.  ``moda_oracle.c`` writes the steps out; this module builds it with
gcc and marshals arrays through ctypes.  ``depth_forward`` is depth attention
alone (same page, section "Depth stream mechanism"): each query row over its
own token's L depth entries only.

Every function here has pins in ``tests/test_oracle_pins.py``; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moda_oracle.c")
_LIB = os.path.join(_HERE, "libmoda_oracle.so")

F32, BF16, F64 = 0, 1, 2

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load (building first if needed) and declare the C entry points."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if path is None and (not os.path.exists(p) or
                         os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(p)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_moda_fwd.argtypes = [i64] * 6 + [ctypes.c_int] + [vp] * 5 + [dp, dp]
    lib.oracle_moda_fwd.restype = ctypes.c_int
    lib.oracle_moda_rows.argtypes = [i64, vp] + [i64] * 6 + [ctypes.c_int] + [vp] * 5 + [dp, dp]
    lib.oracle_moda_rows.restype = ctypes.c_int
    lib.oracle_moda_row_weights.argtypes = ([i64] * 6 + [ctypes.c_int] + [i64] * 3 +
                                            [vp] * 5 + [dp, dp])
    lib.oracle_moda_row_weights.restype = ctypes.c_int
    lib.oracle_depth_fwd.argtypes = [i64] * 6 + [ctypes.c_int] + [vp] * 3 + [dp, dp]
    lib.oracle_depth_fwd.restype = ctypes.c_int
    lib.oracle_moda_bwd.argtypes = [i64] * 6 + [ctypes.c_int] + [vp] * 6 + [dp] * 5
    lib.oracle_moda_bwd.restype = ctypes.c_int
    lib.oracle_moda_bwd_rows.argtypes = ([i64, vp] + [i64] * 6 + [ctypes.c_int] + [vp] * 6 +
                                         [dp] * 3)
    lib.oracle_moda_bwd_rows.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _as_input(a: np.ndarray, dtype_code: int) -> np.ndarray:
    want = {F32: np.float32, BF16: np.uint16, F64: np.float64}[dtype_code]
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"oracle input has dtype {a.dtype}, expected {np.dtype(want)}")
    return a


def _code_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.uint16:  # raw bf16 bit patterns
        return BF16
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def moda_forward(q, k, v, kd=None, vd=None, *, lib=None):
    """Full fp64 MoDA forward.

    q [B,Hq,T,d]; k, v [B,Hkv,T,d]; kd, vd [B,Hkv,T,L,d] (None for L = 0).
    Arrays are float32, float64, or uint16 holding bf16 bit patterns (all five
    the same).  Returns (out [B,Hq,T,d] float64, lse [B,Hq,T] float64).
    """
    lib = lib or load()
    code = _code_of(q)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    L = 0 if kd is None else kd.shape[3]
    q, k, v = (_as_input(x, code) for x in (q, k, v))
    if L:
        kd, vd = _as_input(kd, code), _as_input(vd, code)
        assert kd.shape == (B, Hkv, T, L, d) and vd.shape == kd.shape
    else:
        kd = vd = None
    assert k.shape == (B, Hkv, T, d) and v.shape == k.shape
    out = np.empty((B, Hq, T, d), np.float64)
    lse = np.empty((B, Hq, T), np.float64)
    rc = lib.oracle_moda_fwd(B, Hq, Hkv, T, L, d, code, _ptr(q), _ptr(k), _ptr(v),
                             _ptr(kd), _ptr(vd), _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_moda_fwd failed with code {rc}")
    return out, lse


def moda_rows(rows, shape, q_rows, k, v, kd_rows=None, vd_rows=None, *, lib=None):
    """fp64 MoDA forward for selected rows only.

    rows [R,3] int64 (b, h, t); shape = (B, Hq, Hkv, T, L, d);
    q_rows [R,d]; k, v [B,Hkv,T,d]; kd_rows, vd_rows [R,L,d] (token t's depth
    rows of each selected row).  Returns (out [R,d], lse [R]) in float64.
    """
    lib = lib or load()
    B, Hq, Hkv, T, L, d = (int(x) for x in shape)
    code = _code_of(q_rows)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.shape[0]
    q_rows, k, v = (_as_input(x, code) for x in (q_rows, k, v))
    if L:
        kd_rows, vd_rows = _as_input(kd_rows, code), _as_input(vd_rows, code)
        assert kd_rows.shape == (R, L, d) and vd_rows.shape == (R, L, d)
    else:
        kd_rows = vd_rows = None
    out = np.empty((R, d), np.float64)
    lse = np.empty((R,), np.float64)
    rc = lib.oracle_moda_rows(R, _ptr(rows), B, Hq, Hkv, T, L, d, code, _ptr(q_rows),
                              _ptr(k), _ptr(v), _ptr(kd_rows), _ptr(vd_rows),
                              _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_moda_rows failed with code {rc}")
    return out, lse


def moda_row_weights(q, k, v, kd, vd, b, h, t, *, lib=None):
    """Explicit normalised weights of row (b, h, t): t+1 sequence then L depth.

    Returns (weights [t+1+L] float64, out_row [d] float64).
    """
    lib = lib or load()
    code = _code_of(q)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    L = 0 if kd is None else kd.shape[3]
    q, k, v = (_as_input(x, code) for x in (q, k, v))
    if L:
        kd, vd = _as_input(kd, code), _as_input(vd, code)
    else:
        kd = vd = None
    p = np.empty((t + 1 + L,), np.float64)
    o = np.empty((d,), np.float64)
    rc = lib.oracle_moda_row_weights(B, Hq, Hkv, T, L, d, code, b, h, t, _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(kd), _ptr(vd), _ptr(o), _ptr(p))
    if rc:
        raise ValueError(f"oracle_moda_row_weights failed with code {rc}")
    return p, o


def depth_forward(q, kd, vd, *, lib=None):
    """fp64 depth attention alone: each query row over its own token's L depth
    entries, one softmax scaled by 1/sqrt(d) (no sequence keys).

    q [B,Hq,T,d]; kd, vd [B,Hkv,T,L,d] with L >= 1, same element type as q.
    Returns (out [B,Hq,T,d] float64, lse [B,Hq,T] float64).
    """
    lib = lib or load()
    code = _code_of(q)
    B, Hq, T, d = q.shape
    Hkv, L = kd.shape[1], kd.shape[3]
    q, kd, vd = (_as_input(x, code) for x in (q, kd, vd))
    assert kd.shape == (B, Hkv, T, L, d) and vd.shape == kd.shape
    out = np.empty((B, Hq, T, d), np.float64)
    lse = np.empty((B, Hq, T), np.float64)
    rc = lib.oracle_depth_fwd(B, Hq, Hkv, T, L, d, code, _ptr(q), _ptr(kd), _ptr(vd),
                              _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_depth_fwd failed with code {rc}")
    return out, lse


def moda_backward(q, k, v, kd, vd, dout, *, lib=None):
    """fp64 MoDA backward: gradients of a loss whose gradient with respect to
    the MoDA output is ``dout`` [B,Hq,T,d] (same element type as q).

    Returns (dq [B,Hq,T,d], dk, dv [B,Hkv,T,d], dkd, dvd [B,Hkv,T,L,d] or None
    when L = 0), all float64.
    """
    lib = lib or load()
    code = _code_of(q)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    L = 0 if kd is None else kd.shape[3]
    q, k, v, dout = (_as_input(x, code) for x in (q, k, v, dout))
    if L:
        kd, vd = _as_input(kd, code), _as_input(vd, code)
    else:
        kd = vd = None
    dq = np.empty((B, Hq, T, d), np.float64)
    dk = np.empty((B, Hkv, T, d), np.float64)
    dv = np.empty((B, Hkv, T, d), np.float64)
    dkd = np.empty((B, Hkv, T, L, d), np.float64) if L else None
    dvd = np.empty((B, Hkv, T, L, d), np.float64) if L else None
    rc = lib.oracle_moda_bwd(B, Hq, Hkv, T, L, d, code, _ptr(q), _ptr(k), _ptr(v), _ptr(kd),
                             _ptr(vd), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkd),
                             _ptr(dvd))
    if rc:
        raise ValueError(f"oracle_moda_bwd failed with code {rc}")
    return dq, dk, dv, dkd, dvd


def moda_backward_rows(rows, shape, q_rows, dout_rows, k, v, kd_rows=None, vd_rows=None, *,
                       lib=None):
    """fp64 MoDA backward for selected rows only (the backward's per-row steps).

    rows [R,3] int64 (b, h, t); shape = (B, Hq, Hkv, T, L, d); q_rows, dout_rows
    [R,d]; k, v [B,Hkv,T,d]; kd_rows, vd_rows [R,L,d] (token t's depth rows of
    each selected row).  Returns (dq [R,d], p [R,T+L], ds [R,T+L]) in float64:
    the row's dQ, and its weight and softmax gradient for each entry it reads
    (sequence keys 0..t, then depth entries at t+1+i; zero elsewhere).  dK_j is
    then s * sum over the rows that read key j of ds[row, j] * q_row, and dV_j
    the sum of p[row, j] * dout_row (likewise for the depth entries).
    """
    lib = lib or load()
    B, Hq, Hkv, T, L, d = (int(x) for x in shape)
    code = _code_of(q_rows)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.shape[0]
    q_rows, dout_rows, k, v = (_as_input(x, code) for x in (q_rows, dout_rows, k, v))
    if L:
        kd_rows, vd_rows = _as_input(kd_rows, code), _as_input(vd_rows, code)
        assert kd_rows.shape == (R, L, d) and vd_rows.shape == (R, L, d)
    else:
        kd_rows = vd_rows = None
    dq = np.empty((R, d), np.float64)
    p = np.empty((R, T + L), np.float64)
    ds = np.empty((R, T + L), np.float64)
    rc = lib.oracle_moda_bwd_rows(R, _ptr(rows), B, Hq, Hkv, T, L, d, code, _ptr(q_rows),
                                  _ptr(dout_rows), _ptr(k), _ptr(v), _ptr(kd_rows),
                                  _ptr(vd_rows), _ptr(dq), _ptr(p), _ptr(ds))
    if rc:
        raise ValueError(f"oracle_moda_bwd_rows failed with code {rc}")
    return dq, p, ds


def num_threads(*, lib=None) -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS or all cores)."""
    return int((lib or load()).oracle_num_threads())
