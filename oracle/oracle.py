"""ctypes front end of the fp64 CPU oracle (test infrastructure only).

Inputs may be torch tensors or numpy arrays in the library's layout:
  q, k   [B, T, Hq, dk]        v    [B, T, Hv, dv]
  g      [B, T, Hv, dk]        beta [B, T, Hv]
  cu_seqlens [N+1] (packed varlen, B must be 1) or None (fixed length, N = B)
  h0     [N, Hv, dk, dv] or None (zero state)
Every value is widened exactly to fp64 before the oracle sees it, so the oracle
receives the same numbers as the GPU.  Results are fp64 numpy arrays:
  o [B, T, Hv, dv],  hT [N, Hv, dk, dv].

The arithmetic lives in kda_oracle.c; this file only converts and marshals.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def load(path=None):
    """Loads (building on first use if absent) the oracle shared library.  With
    `path`, loads that build of kda_oracle.c instead and does not cache it."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    if path is None and not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path or _LIB_PATH)
    i64, dbl = ctypes.c_int64, ctypes.c_double
    lib.kda_oracle_recurrence.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, dbl, _ip, i64, i64, i64,
                                          i64, i64, _dp, _dp, _dp]
    lib.kda_oracle_recurrence.restype = ctypes.c_int
    lib.kda_oracle_chunked.argtypes = [_dp, _dp, _dp, _dp, _dp, dbl, _ip, i64, i64, i64, i64, i64,
                                       i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.kda_oracle_chunked.restype = ctypes.c_int
    lib.kda_oracle_num_chunks.argtypes = [_ip, i64, i64]
    lib.kda_oracle_num_chunks.restype = i64
    lib.kda_oracle_qg.argtypes = [_dp, _dp, _ip, i64, i64, i64, i64, i64, _dp]
    lib.kda_oracle_qg.restype = ctypes.c_int
    lib.kda_oracle_threads.argtypes = []
    lib.kda_oracle_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen on the CPU, exactly
        import torch
        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _prepare(q, k, v, g, beta, cu_seqlens, h0, alpha=None):
    q, k, v, g, beta, alpha, h0 = (_f64(t) for t in (q, k, v, g, beta, alpha, h0))
    B, T, Hq, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv, dk) or beta.shape != (B, T, Hv):
        raise ValueError("inconsistent input shapes")
    if cu_seqlens is None:
        N = B
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                                             dtype=np.int64))
        N = cu.shape[0] - 1
    if h0 is not None and h0.shape != (N, Hv, dk, dv):
        raise ValueError("h0 shape mismatch")
    if alpha is not None and alpha.shape != beta.shape:
        raise ValueError("alpha shape mismatch")
    return q, k, v, g, beta, alpha, h0, cu, (B, T, Hq, Hv, dk, dv, N)


def threads():
    """OpenMP threads the oracle runs on."""
    return int(load().kda_oracle_threads())


def num_chunks(cu, C):
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    return int(load().kda_oracle_num_chunks(cu.ctypes.data_as(_ip), cu.shape[0] - 1, C))


def recurrence(q, k, v, g, beta, scale, cu_seqlens=None, h0=None, alpha=None, lib=None):
    """Token-by-token fp64 recurrence; returns (o, hT).  alpha=None means alpha = beta.
    `lib` may name another build of kda_oracle.c (used by the mutation tests)."""
    lib = lib or load()
    q, k, v, g, beta, alpha, h0, cu, (B, T, Hq, Hv, dk, dv, N) = _prepare(q, k, v, g, beta, cu_seqlens,
                                                                          h0, alpha)
    o = np.zeros((B, T, Hv, dv), np.float64)
    hT = np.zeros((N, Hv, dk, dv), np.float64)
    rc = lib.kda_oracle_recurrence(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(alpha),
                                   float(scale), cu.ctypes.data_as(_ip), N, Hq, Hv, dk, dv, _ptr(h0),
                                   _ptr(o), _ptr(hT))
    if rc != 0:
        raise RuntimeError("oracle recurrence rejected its inputs")
    return o, hT


def chunked(q, k, v, g, beta, scale, cu_seqlens=None, h0=None, chunk=64, intermediates=False, lib=None):
    """fp64 chunked form; returns (o, hT) or (o, hT, dict of intermediates)."""
    lib = lib or load()
    q, k, v, g, beta, _, h0, cu, (B, T, Hq, Hv, dk, dv, N) = _prepare(q, k, v, g, beta, cu_seqlens, h0)
    C = int(chunk)
    o = np.zeros((B, T, Hv, dv), np.float64)
    hT = np.zeros((N, Hv, dk, dv), np.float64)
    inter = {}
    if intermediates:
        nc = num_chunks(cu, C)
        tt = B * T
        inter = dict(G=np.zeros((tt, Hv, dk)), Aqk=np.zeros((tt, Hv, C)), Akk=np.zeros((tt, Hv, C)),
                     T=np.zeros((tt, Hv, C)), W=np.zeros((tt, Hv, dk)), U=np.zeros((tt, Hv, dv)),
                     v_new=np.zeros((tt, Hv, dv)), h_c=np.zeros((nc, Hv, dk, dv)))
    p = {name: _ptr(inter.get(name)) for name in ("G", "Aqk", "Akk", "T", "W", "U", "v_new", "h_c")}
    rc = lib.kda_oracle_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                cu.ctypes.data_as(_ip), N, Hq, Hv, dk, dv, C, _ptr(h0), _ptr(o), _ptr(hT),
                                p["G"], p["Aqk"], p["Akk"], p["T"], p["W"], p["U"], p["v_new"], p["h_c"])
    if rc != 0:
        raise RuntimeError("oracle chunked form rejected its inputs")
    if intermediates:
        return o, hT, inter
    return o, hT


def qg(q, g, cu_seqlens=None, chunk=64, lib=None):
    """The optional QG output, q exp(G) with G the chunk-local inclusive cumsum of
    g, as an fp64 [B, T, Hv, dk] array (rows of tokens in no sequence are zero)."""
    lib = lib or load()
    q, g = _f64(q), _f64(g)
    B, T, Hq, dk = q.shape
    Hv = g.shape[2]
    if g.shape != (B, T, Hv, dk) or Hv % Hq:
        raise ValueError("inconsistent input shapes")
    if cu_seqlens is None:
        N, cu = B, np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                                             dtype=np.int64))
        N = cu.shape[0] - 1
    out = np.zeros((B, T, Hv, dk), np.float64)
    if lib.kda_oracle_qg(_ptr(q), _ptr(g), cu.ctypes.data_as(_ip), N, Hq, Hv, dk, int(chunk), _ptr(out)) != 0:
        raise RuntimeError("oracle qg rejected its inputs")
    return out
