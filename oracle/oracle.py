"""ctypes front of the fp64 FusedKV oracle (``fkv_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the product path never imports it.  It does
not import the HIP library or its Python package, and the HIP library does not
import it.

Pages cited (by title):
  [Deck]  "FusedKV: Reconstructing KV Caches with Cross-Layer Fusion"
  [Notes] "FusedKV:通过跨层融合重构 KV 缓存"

The arithmetic lives in ``fkv_oracle.c``; this file only marshals numpy arrays
(float32, or bfloat16 stored as raw uint16 bit patterns) into it and builds the
shared object with gcc.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fkv_oracle.c")
_SO_DEFAULT = os.path.join(_HERE, "liboracle.so")
# A test may point the loader at another build of the same source (the
# mutation test builds deliberately broken copies to show the pins catch them).
_SO = os.environ.get("FKV_ORACLE_SO", _SO_DEFAULT)
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 -fopenmp (IEEE semantics: no fast-math,
    so the sums stay sequential and in fp64)."""
    return build_from(_SRC, _SO_DEFAULT, force)


def build_from(src: str, so: str, force: bool = True) -> str:
    if force or not os.path.exists(so):
        tmp = so + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-o", tmp, src, "-lm"])
        os.replace(tmp, so)
    return so


class _View(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("sb", ctypes.c_int64),
                ("ss", ctypes.c_int64), ("sh", ctypes.c_int64)]


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
                ("seqlen_k", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("scale", ctypes.c_double)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.orc_attend.restype = ctypes.c_int
        lib.orc_attend.argtypes = [
            ctypes.POINTER(_Shape), ctypes.c_int, ctypes.c_void_p,
            _View, _View, _View, _View,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p]
        for name in ("orc_cache_capacity", "orc_cache_reads"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int64
            fn.argtypes = [ctypes.c_int] + [ctypes.c_int64] * 4
        lib.orc_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError("oracle inputs are float32, bfloat16 bit patterns (uint16) or float64, got %s" % a.dtype)


def _view(a: np.ndarray | None, code: int) -> _View:
    """A [B, S, H, D] array, possibly a strided view (e.g. of a [B, H, S, D]
    buffer); the channel axis must be contiguous."""
    if a is None:
        return _View(None, 0, 0, 0)
    if a.ndim != 4 or _dtype_code(a) != code:
        raise ValueError("cache views are 4-D [B, S, H, D] of the query's dtype")
    es = a.itemsize
    if a.strides[3] != es:
        raise ValueError("channel axis must be contiguous")
    return _View(a.ctypes.data, a.strides[0] // es, a.strides[1] // es, a.strides[2] // es)


def _weights(w):
    if w is None:
        return None, None
    w = np.ascontiguousarray(w, dtype=np.float32)
    return w, w.ctypes.data


def attend(q, k1, v1, kn=None, vn=None, *, k_w1=None, k_wn=None, v_w1=None,
           v_wn=None, causal=False, scale=None, seqlens_k=None, rows=None):
    """Oracle attention output of one layer.

    FusedKV when ``kn``/``vn`` and the four ``[Hkv, D]`` weight arrays are
    given; otherwise single-source attention over (k1, v1) -- FusedKV-Lite when
    called with (K^n, V^1), the plain control with a layer's own caches.

    q: [B, Sq, Hq, D]; caches: [B, Sk, Hkv, D] (any strides, channel axis
    contiguous).  Returns (O [rows, D] float64, LSE [rows] float64); with
    ``rows`` None the rows are all (b, h, p) in that order, i.e. O can be
    reshaped to [B, Hq, Sq, D].
    """
    lib = _load()
    code = _dtype_code(q)
    q = np.ascontiguousarray(q)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k1.shape[1], k1.shape[2]
    single = kn is None
    if k1.shape != (B, Sk, Hkv, D) or v1.shape != k1.shape:
        raise ValueError("cache shape mismatch")
    if not single and (kn.shape != k1.shape or vn.shape != k1.shape):
        raise ValueError("cache shape mismatch")
    wk1, pk1 = _weights(k_w1)
    wkn, pkn = _weights(k_wn)
    wv1, pv1 = _weights(v_w1)
    wvn, pvn = _weights(v_wn)
    if not single:
        for w in (wk1, wkn, wv1, wvn):
            if w is None or w.size != Hkv * D:
                raise ValueError("FusedKV needs four [Hkv, D] weight arrays")
    shape = _Shape(B, Sq, Sk, Hq, Hkv, D, code, 1 if causal else 0,
                   float(1.0 / math.sqrt(D) if scale is None else scale))
    sl = None
    if seqlens_k is not None:
        sl = np.ascontiguousarray(seqlens_k, dtype=np.int32)
    rr = None
    if rows is not None:
        rr = np.ascontiguousarray(rows, dtype=np.int64)
    n = rr.size if rr is not None else B * Hq * Sq
    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    rc = lib.orc_attend(
        ctypes.byref(shape), 1 if single else 0, q.ctypes.data,
        _view(k1, code), _view(kn, code), _view(v1, code), _view(vn, code),
        pk1, pkn, pv1, pvn,
        None if sl is None else sl.ctypes.data,
        None if rr is None else rr.ctypes.data, int(n),
        out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the call")
    return out, lse


def row_index(b, h, p, Hq, Sq):
    """Row number used by ``attend``'s ``rows`` argument."""
    return (b * Hq + h) * Sq + p


VANILLA, LITE, FUSEDKV = 0, 1, 2


def cache_capacity(method, L, S, Hkv, D):
    """Resident KV-cache elements of an L-layer model ([Deck] Table 1)."""
    return int(_load().orc_cache_capacity(method, L, S, Hkv, D))


def cache_reads(method, L, S, Hkv, D):
    """KV-cache elements read by one decode step over all L layers ([Deck]
    Table 1; [Notes] section 2.5)."""
    return int(_load().orc_cache_reads(method, L, S, Hkv, D))


def num_threads():
    return int(_load().orc_num_threads())
