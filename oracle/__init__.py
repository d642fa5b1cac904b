"""CPU fp64 oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and
it shares no code with it.  The arithmetic lives in ``oracle.c`` (plain
double-precision C, see that file's header for the definitions and the
passages they follow); this module only marshals numpy arrays through ctypes.

Every function takes a batch of G independent heads, arrays of shape
[G, rows, d] in float64 (anything else is converted), and returns float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.POINTER(ctypes.c_double)
_PI = ctypes.POINTER(ctypes.c_int64)
_PB = ctypes.POINTER(ctypes.c_uint8)
_I = ctypes.c_int64
_BM = [_PB, _I, _I, _I, _I]  # block mask, bq, bk, nqb, nkb


GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]


def compile_source(src: str, out: str) -> str:
    """Compile one C source of the oracle into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


class OracleLib:
    """ctypes binding of one compiled copy of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_attn_fwd.argtypes = [_I, _I, _I, _I, _P, _P, _P, _PI, ctypes.c_int, _I, _I, *_BM,
                                        ctypes.c_double, _P, _P]
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_fwd_online.argtypes = [_I, _I, _I, _I, _P, _P, _P, _PI, ctypes.c_int, _I, _I, *_BM,
                                               ctypes.c_double, _I, _P, _P]
        lib.oracle_attn_fwd_online.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _PI, ctypes.c_int, _I, _I, *_BM,
                                        ctypes.c_double, _PI, _I, _P, _PI, _I, _P, _P]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def fwd(self, q, k, v, causal: bool, scale: float, qpos=None, window=(-1, -1), block_mask=None,
            block=(128, 128)):
        """Three-pass forward.  Returns (o [G,nq,d], lse [G,nq]).

        qpos gives the key position of each query row (default i + nk - nq:
        rows aligned to the end of the keys, the identity when nq == nk).  Key
        j is visible to row i iff (not causal or j <= qpos[i]) and, for a
        window (wl, wr) with -1 meaning unbounded, qpos[i] - wl <= j <= qpos[i] + wr,
        and, for a block mask ([nqb, nkb] shared by all heads or [G, nqb, nkb],
        block = (bq, bk)), block_mask[qpos[i] // bq, j // bk] != 0.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        G, nq, d = q.shape
        nk = k.shape[1]
        if k.shape != (G, nk, d) or v.shape != (G, nk, d):
            raise ValueError("shape mismatch")
        qpos = _qpos(qpos, nq, nk)
        o = np.empty((G, nq, d), np.float64)
        lse = np.empty((G, nq), np.float64)
        bm = _block_mask(block_mask, block, G, qpos, nk)
        rc = self.lib.oracle_attn_fwd(G, nq, nk, d, _ptr(q), _ptr(k), _ptr(v), _iptr(qpos),
                                      int(bool(causal)), int(window[0]), int(window[1]), *bm, float(scale),
                                      _ptr(o), _ptr(lse))
        if rc != 0:
            raise MemoryError("oracle_attn_fwd failed (%d)" % rc)
        return o, lse

    def fwd_online(self, q, k, v, causal: bool, scale: float, block: int, qpos=None, window=(-1, -1),
                   block_mask=None, mask_block=(128, 128)):
        """Block-wise running-max forward (the validator).  Returns (o, lse)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        G, nq, d = q.shape
        nk = k.shape[1]
        qpos = _qpos(qpos, nq, nk)
        o = np.empty((G, nq, d), np.float64)
        lse = np.empty((G, nq), np.float64)
        bm = _block_mask(block_mask, mask_block, G, qpos, nk)
        rc = self.lib.oracle_attn_fwd_online(G, nq, nk, d, _ptr(q), _ptr(k), _ptr(v), _iptr(qpos),
                                             int(bool(causal)), int(window[0]), int(window[1]), *bm,
                                             float(scale), int(block), _ptr(o), _ptr(lse))
        if rc != 0:
            raise RuntimeError("oracle_attn_fwd_online failed (%d)" % rc)
        return o, lse

    def bwd(self, q, k, v, dout, causal: bool, scale: float, rows=None, keys=None, qpos=None,
            window=(-1, -1), block_mask=None, block=(128, 128)):
        """Analytic backward.  Returns (dq, dk, dv).

        q, dout: [G, nq, d]; k, v: [G, nk, d]; qpos and window as in fwd.
        rows / keys select which query rows of dq and which key rows of dk, dv
        are computed (default: all).  dq has shape [G, len(rows), d]; dk, dv
        [G, len(keys), d].  An empty selection computes nothing for that output.
        """
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        G, nq, d = q.shape
        nk = k.shape[1]
        if k.shape != (G, nk, d) or v.shape != (G, nk, d) or dout.shape != (G, nq, d):
            raise ValueError("shape mismatch")
        qpos = _qpos(qpos, nq, nk)
        rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        keys_a = None if keys is None else np.ascontiguousarray(keys, dtype=np.int64).reshape(-1)
        nrows = nq if rows_a is None else len(rows_a)
        nkeys = nk if keys_a is None else len(keys_a)
        for sel, n in ((rows_a, nq), (keys_a, nk)):
            if sel is not None and len(sel) and (sel.min() < 0 or sel.max() >= n):
                raise IndexError("row/key index out of range")
        dq = np.empty((G, nrows, d), np.float64)
        dk = np.empty((G, nkeys, d), np.float64)
        dv = np.empty((G, nkeys, d), np.float64)
        pad = np.zeros(1, np.int64)  # a valid pointer for an empty selection
        rp = None if rows_a is None else (rows_a if nrows else pad)
        kp = None if keys_a is None else (keys_a if nkeys else pad)
        bm = _block_mask(block_mask, block, G, qpos, nk)
        rc = self.lib.oracle_attn_bwd(G, nq, nk, d, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _iptr(qpos),
                                      int(bool(causal)), int(window[0]), int(window[1]), *bm, float(scale),
                                      _iptr(rp), nrows, _ptr(dq), _iptr(kp), nkeys, _ptr(dk), _ptr(dv))
        if rc != 0:
            raise MemoryError("oracle_attn_bwd failed (%d)" % rc)
        return dq, dk, dv


def _qpos(qpos, nq, nk):
    """Key positions of the query rows: rows aligned to the end of the keys by default."""
    if qpos is None:
        qpos = np.arange(nq) + (nk - nq)
    qpos = np.ascontiguousarray(qpos, dtype=np.int64)
    if qpos.shape != (nq,):
        raise ValueError("qpos must have one entry per query row")
    return qpos


def _block_mask(block_mask, block, G, qpos, nk):
    """ctypes arguments (pointer, bq, bk, nqb, nkb) of an optional block mask.

    The mask is kept alive by the returned pointer object's _keep attribute."""
    if block_mask is None:
        return (None, 1, 1, 1, 1)
    bq, bk = int(block[0]), int(block[1])
    bm = np.asarray(block_mask)
    if bm.ndim == 2:
        bm = np.broadcast_to(bm, (G,) + bm.shape)
    bm = np.ascontiguousarray(bm != 0, dtype=np.uint8)
    if bm.ndim != 3 or bm.shape[0] != G:
        raise ValueError("block mask must be [nqb, nkb] or [G, nqb, nkb]")
    nqb, nkb = bm.shape[1], bm.shape[2]
    if bq < 1 or bk < 1 or nkb * bk < nk or (len(qpos) and nqb * bq <= int(np.max(qpos))):
        raise ValueError("block mask does not cover every (row position, key)")
    ptr = bm.ctypes.data_as(_PB)
    ptr._keep = bm
    return (ptr, bq, bk, nqb, nkb)


def _load() -> OracleLib:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = OracleLib(_LIB)
    return _lib


def _f64(a) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if a.ndim == 2:
        a = a[None]
    if a.ndim != 3:
        raise ValueError("expected [G, rows, d] or [rows, d], got shape %r" % (a.shape,))
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P)


def _iptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_PI)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().num_threads()


def fwd(q, k, v, causal: bool, scale: float, qpos=None, window=(-1, -1), block_mask=None, block=(128, 128)):
    return _load().fwd(q, k, v, causal, scale, qpos, window, block_mask, block)


def fwd_online(q, k, v, causal: bool, scale: float, block: int, qpos=None, window=(-1, -1), block_mask=None,
               mask_block=(128, 128)):
    return _load().fwd_online(q, k, v, causal, scale, block, qpos, window, block_mask, mask_block)


def bwd(q, k, v, dout, causal: bool, scale: float, rows=None, keys=None, qpos=None, window=(-1, -1),
        block_mask=None, block=(128, 128)):
    return _load().bwd(q, k, v, dout, causal, scale, rows, keys, qpos, window, block_mask, block)


fwd.__doc__ = OracleLib.fwd.__doc__
fwd_online.__doc__ = OracleLib.fwd_online.__doc__
bwd.__doc__ = OracleLib.bwd.__doc__


def _segments(cu, total):
    cu = np.asarray(cu, dtype=np.int64).reshape(-1)
    if len(cu) < 1 or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cumulative lengths must start at 0, not decrease and end at the total")
    return [(int(cu[b]), int(cu[b + 1])) for b in range(len(cu) - 1)]


def fwd_varlen(q, k, v, cu_q, cu_k, causal: bool, scale: float, window=(-1, -1)):
    """Packed variable-length forward: q [H, total_q, d], k, v [H, total_k, d].

    Sequence b owns query rows cu_q[b]..cu_q[b+1]-1 and keys cu_k[b]..cu_k[b+1]-1
    of every head; each is attended on its own, rows aligned to the end of its
    keys.  Returns (o [H, total_q, d], lse [H, total_q]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, tq, d = q.shape
    sq, sk = _segments(cu_q, tq), _segments(cu_k, k.shape[1])
    if len(sq) != len(sk):
        raise ValueError("cu_q and cu_k describe different batch sizes")
    o = np.zeros((H, tq, d))
    lse = np.full((H, tq), -np.inf)
    for (q0, q1), (k0, k1) in zip(sq, sk):
        if q1 == q0:
            continue
        if k1 == k0:  # no keys at all: every row sees nothing
            continue
        o[:, q0:q1], lse[:, q0:q1] = fwd(q[:, q0:q1], k[:, k0:k1], v[:, k0:k1], causal, scale, window=window)
    return o, lse


def bwd_varlen(q, k, v, dout, cu_q, cu_k, causal: bool, scale: float, window=(-1, -1)):
    """Packed variable-length backward (layout as fwd_varlen).  Returns (dq, dk, dv)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    H, tq, d = q.shape
    sq, sk = _segments(cu_q, tq), _segments(cu_k, k.shape[1])
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for (q0, q1), (k0, k1) in zip(sq, sk):
        if q1 == q0 or k1 == k0:
            continue
        dq[:, q0:q1], dk[:, k0:k1], dv[:, k0:k1] = bwd(q[:, q0:q1], k[:, k0:k1], v[:, k0:k1], dout[:, q0:q1],
                                                       causal, scale, window=window)
    return dq, dk, dv
