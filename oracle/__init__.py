"""fp64 CPU oracle for the selective scan (S6) and its one-token decode step.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports, links or runs
anything here, and this package imports nothing from the HIP library.

The arithmetic lives in ``oracle.c`` (plain C, IEEE fp64, sequential in time, OpenMP
over independent rows); this module builds it with gcc, converts inputs to exact
float64 copies and calls it through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

_d = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            lib.oracle_selective_scan.restype = ctypes.c_int
            lib.oracle_selective_scan.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _i64p,
                _d, _d, _d, _d, _d, _d, _d, _d, ctypes.c_int, _d, _i64p, _d, _d, ctypes.c_int]
            lib.oracle_selective_scan_bwd.restype = ctypes.c_int
            lib.oracle_selective_scan_bwd.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _i64p,
                _d, _d, _d, _d, _d, _d, _d, _d, ctypes.c_int, _d, _i64p, _d, _d,
                _d, _d, _d, _d, _d, _d, _d, _d, _d, ctypes.c_int, ctypes.c_int]
            lib.oracle_causal_conv1d.restype = ctypes.c_int
            lib.oracle_causal_conv1d.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _d, _d, _d, _d, ctypes.c_int,
                _d, _d, ctypes.c_int]
            lib.oracle_state_update.restype = ctypes.c_int
            lib.oracle_state_update.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _i64p,
                _d, _d, _d, _d, _d, _d, _d, _d, _d, _d, ctypes.c_int]
            lib.oracle_ssd_scan.restype = ctypes.c_int
            lib.oracle_ssd_scan.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                _d, _d, _d, _d, _d, _d, _d, _d, ctypes.c_int, _d, _i64p, ctypes.c_int64, _d, _d, ctypes.c_int,
                ctypes.c_int]
            lib.oracle_softplus.restype = None
            lib.oracle_softplus.argtypes = [_d, _d, ctypes.c_int64]
            lib.oracle_silu.restype = None
            lib.oracle_silu.argtypes = [_d, _d, ctypes.c_int64]
            lib.oracle_max_threads.restype = ctypes.c_int
            lib.oracle_max_threads.argtypes = []
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.cast(None, _d)
    return a.ctypes.data_as(_d)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def softplus(x) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_softplus(_ptr(x), _ptr(y), x.size)
    return y


def silu(x) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_silu(_ptr(x), _ptr(y), x.size)
    return y


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus_flag=True,
                   rows=None, nthreads: int = 0, h0=None, seq_lens=None):
    """Run the fp64 scan.

    u, delta, z: (batch, d_inner, L); A: (d_inner, d_state); B, C: (batch, d_state, L);
    D, delta_bias: (d_inner,).  Any float dtype; values are taken exactly as float64.
    h0: optional starting state (batch, d_inner, d_state) (default zeros).
    seq_lens: optional (batch,) lengths (clamped to [0, L]): steps stop there, outputs past the
    end are 0 and last_state is the state after the batch's own last step.
    rows: optional flat row indices r = b * d_inner + d to compute (default: all rows).
    Returns (out, last_state): (batch, d_inner, L) and (batch, d_inner, d_state) when rows
    is None, else (len(rows), L) and (len(rows), d_state).
    """
    u = np.asarray(u)
    Bt, Dn, L = u.shape
    N = np.asarray(A).shape[1]
    if rows is None:
        sel = np.arange(Bt * Dn, dtype=np.int64)
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    ch = sel % Dn
    rb = np.ascontiguousarray(sel // Dn)

    def rows_of(a):
        return None if a is None else _f64(np.asarray(a).reshape(Bt * Dn, L)[sel])

    u_r, dl_r, z_r = rows_of(u), rows_of(delta), rows_of(z)
    A_r = _f64(np.asarray(A)[ch])
    D_r = None if D is None else _f64(np.asarray(D)[ch])
    b_r = None if delta_bias is None else _f64(np.asarray(delta_bias)[ch])
    Bm, Cm = _f64(B), _f64(C)
    h0_r = None if h0 is None else _f64(np.asarray(h0).reshape(Bt * Dn, N)[sel])
    len_r = None if seq_lens is None else np.ascontiguousarray(
        np.asarray(seq_lens, dtype=np.int64)[rb])
    R = sel.size
    out = np.empty((R, L), np.float64)
    last = np.empty((R, N), np.float64)
    rc = _load().oracle_selective_scan(
        R, N, L, Bt, rb.ctypes.data_as(_i64p), _ptr(u_r), _ptr(dl_r), _ptr(z_r), _ptr(A_r),
        _ptr(Bm), _ptr(Cm), _ptr(D_r), _ptr(b_r), int(bool(softplus_flag)), _ptr(h0_r),
        None if len_r is None else len_r.ctypes.data_as(_i64p), _ptr(out), _ptr(last), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_selective_scan rejected its arguments")
    if rows is None:
        return out.reshape(Bt, Dn, L), last.reshape(Bt, Dn, N)
    return out, last


def selective_scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus_flag=True,
                       dout=None, rows=None, nthreads: int = 0, magnitude: bool = False, h0=None,
                       seq_lens=None, dlast=None):
    """fp64 gradients of L = sum(dout * out) for the forward scan from h_0 = 0.

    Inputs as selective_scan, plus dout (batch, d_inner, L).  Returns a dict:
      du, ddelta, dz (None without z): (batch, d_inner, L), or (len(rows), L) with rows;
      dA: (d_inner, d_state); dD, ddelta_bias: (d_inner,) -- each summed over the selected
      rows of that channel (with rows given: per-row arrays (len(rows), d_state) / (len(rows),));
      dB, dC: (batch, d_state, L), summed over the selected rows.
    dD / ddelta_bias are the gradients at D = 0 / bias = 0 when those are None.
    magnitude=True returns, in the same layout, the sum of |terms| behind each element.
    h0, seq_lens: as selective_scan; dlast: dL/d last_state (batch, d_inner, d_state), adding
    sum(dlast * last_state) to the loss.  The dict then also holds dh0 (dL/dh0, same shape as h0,
    or (len(rows), d_state) with rows).
    """
    u = np.asarray(u)
    Bt, Dn, L = u.shape
    N = np.asarray(A).shape[1]
    if rows is None:
        sel = np.arange(Bt * Dn, dtype=np.int64)
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    ch = sel % Dn
    rb = np.ascontiguousarray(sel // Dn)

    def rows_of(a):
        return None if a is None else _f64(np.asarray(a).reshape(Bt * Dn, L)[sel])

    R = sel.size
    du = np.empty((R, L)); dd = np.empty((R, L))
    dz = np.empty((R, L)) if z is not None else None
    dA = np.empty((R, N)); dD = np.empty(R); db = np.empty(R)
    dB = np.empty((Bt, N, L)); dC = np.empty((Bt, N, L))
    dh0 = np.empty((R, N))
    h0_r = None if h0 is None else _f64(np.asarray(h0).reshape(Bt * Dn, N)[sel])
    dl_r = None if dlast is None else _f64(np.asarray(dlast).reshape(Bt * Dn, N)[sel])
    len_r = None if seq_lens is None else np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int64)[rb])
    rc = _load().oracle_selective_scan_bwd(
        R, N, L, Bt, rb.ctypes.data_as(_i64p), _ptr(rows_of(u)), _ptr(rows_of(delta)),
        _ptr(rows_of(z)), _ptr(_f64(np.asarray(A)[ch])), _ptr(_f64(B)), _ptr(_f64(C)),
        _ptr(None if D is None else _f64(np.asarray(D)[ch])),
        _ptr(None if delta_bias is None else _f64(np.asarray(delta_bias)[ch])),
        int(bool(softplus_flag)), _ptr(h0_r), None if len_r is None else len_r.ctypes.data_as(_i64p),
        _ptr(dl_r), _ptr(rows_of(dout)), _ptr(du), _ptr(dd), _ptr(dz), _ptr(dA),
        _ptr(dB), _ptr(dC), _ptr(dD), _ptr(db), _ptr(dh0), int(bool(magnitude)), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_selective_scan_bwd rejected its arguments")
    if rows is not None:
        return dict(du=du, ddelta=dd, dz=dz, dA=dA, dB=dB, dC=dC, dD=dD, ddelta_bias=db, dh0=dh0)
    sh = (Bt, Dn, L)
    return dict(du=du.reshape(sh), ddelta=dd.reshape(sh),
                dz=None if dz is None else dz.reshape(sh),
                dA=dA.reshape(Bt, Dn, N).sum(0), dB=dB, dC=dC,
                dD=dD.reshape(Bt, Dn).sum(0), ddelta_bias=db.reshape(Bt, Dn).sum(0),
                dh0=dh0.reshape(Bt, Dn, N))


def causal_conv1d(x, weight, bias=None, state=None, silu=True, rows=None, nthreads: int = 0):
    """fp64 causal depthwise conv1d (+ silu).

    x: (batch, d_inner, L); weight: (d_inner, K); bias: (d_inner,); state: the K - 1 inputs before
    t = 0, (batch, d_inner, K - 1), oldest first (default zeros).  Returns (out, final_state):
    (batch, d_inner, L) and (batch, d_inner, K - 1) -- or (len(rows), ...) with rows.
    """
    x = np.asarray(x)
    Bt, Dn, L = x.shape
    K = np.asarray(weight).shape[1]
    sel = np.arange(Bt * Dn, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    ch = sel % Dn
    xr = _f64(x.reshape(Bt * Dn, L)[sel])
    st = None if state is None else _f64(np.asarray(state).reshape(Bt * Dn, K - 1)[sel])
    R = sel.size
    out = np.empty((R, L))
    fin = np.empty((R, max(K - 1, 0)))
    rc = _load().oracle_causal_conv1d(
        R, L, K, _ptr(xr), _ptr(_f64(np.asarray(weight)[ch])),
        _ptr(None if bias is None else _f64(np.asarray(bias)[ch])), _ptr(st), int(bool(silu)),
        _ptr(out), _ptr(fin), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_causal_conv1d rejected its arguments")
    if rows is None:
        return out.reshape(Bt, Dn, L), fin.reshape(Bt, Dn, K - 1)
    return out, fin


def selective_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                           rows=None, nthreads: int = 0):
    """One fp64 decode step.

    state: (batch, d_inner, d_state) float64, updated in place (rows=None) -- or, with
    rows given, a (len(rows), d_state) float64 array of those rows' states, updated in place.
    x, dt, z: (batch, d_inner); B, C: (batch, d_state); A: (d_inner, d_state).
    Returns out: (batch, d_inner), or (len(rows),) with rows.
    """
    x = np.asarray(x)
    Bt, Dn = x.shape
    N = np.asarray(A).shape[1]
    if rows is None:
        sel = np.arange(Bt * Dn, dtype=np.int64)
        if not (isinstance(state, np.ndarray) and state.dtype == np.float64
                and state.flags.c_contiguous and state.shape == (Bt, Dn, N)):
            raise ValueError("state must be a C-contiguous float64 (batch, d_inner, d_state) array")
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if not (isinstance(state, np.ndarray) and state.dtype == np.float64
                and state.flags.c_contiguous and state.shape == (sel.size, N)):
            raise ValueError("state must be a C-contiguous float64 (len(rows), d_state) array")
    ch = sel % Dn
    rb = np.ascontiguousarray(sel // Dn)

    def rows_of(a):
        return None if a is None else _f64(np.asarray(a).reshape(Bt * Dn)[sel])

    R = sel.size
    out = np.empty(R, np.float64)
    rc = _load().oracle_state_update(
        R, N, Bt, rb.ctypes.data_as(_i64p), _ptr(state), _ptr(rows_of(x)), _ptr(rows_of(dt)),
        _ptr(rows_of(z)), _ptr(_f64(np.asarray(A)[ch])), _ptr(_f64(B)), _ptr(_f64(C)),
        _ptr(None if D is None else _f64(np.asarray(D)[ch])),
        _ptr(None if dt_bias is None else _f64(np.asarray(dt_bias)[ch])), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_state_update rejected its arguments")
    return out.reshape(Bt, Dn) if rows is None else out


def ssd_scan(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus_flag=True, h0=None,
             pairs=None, magnitude=False, nthreads=0):
    """Mamba-2 SSD layer in fp64 (oracle_ssd_scan: the selective recurrence with one A per head,
    one delta per (batch, time, head) and B / C per (batch, time, group); heads in contiguous
    blocks of H / G per group).

    x, z: (Bt, L, H, P); dt: (Bt, L, H); B, C: (Bt, L, G, N); A, D, dt_bias: (H,);
    h0: (Bt, H, P, N) or None.  pairs: flat b * H + h indices to compute (default all).
    Returns (out (Bt, L, H, P), last_state (Bt, H, P, N)); entries of pairs not computed are NaN.
    With magnitude=True, every term in absolute value: the per-element error scale M.
    """
    x, dt, A, B, C = _f64(x), _f64(dt), _f64(A), _f64(B), _f64(C)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dt.shape != (Bt, L, H) or B.shape != (Bt, L, G, N) or C.shape != B.shape or A.shape != (H,):
        raise ValueError("ssd_scan: inconsistent shapes")
    D = None if D is None else _f64(D)
    z = None if z is None else _f64(z)
    dt_bias = None if dt_bias is None else _f64(dt_bias)
    h0 = None if h0 is None else _f64(h0)
    out = np.full((Bt, L, H, P), np.nan)
    last = np.full((Bt, H, P, N), np.nan)
    if pairs is not None:
        pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64))
        pp = pairs.ctypes.data_as(_i64p)
        npairs = pairs.size
    else:
        pp = ctypes.cast(None, _i64p)
        npairs = 0
    rc = _load().oracle_ssd_scan(Bt, L, H, P, G, N, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                 _ptr(z), _ptr(dt_bias), 1 if softplus_flag else 0, _ptr(h0), pp, npairs,
                                 _ptr(out), _ptr(last), 1 if magnitude else 0, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_ssd_scan: bad arguments")
    return out, last
