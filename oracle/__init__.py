"""fp64 CPU oracle for causal grouped-query softmax attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code with the
HIP library in ``causal_gqa_flashattention_attn_amd`` and never imports it.

The arithmetic lives in ``oracle_attn.c`` (plain C, double precision, OpenMP, built with
``-O2`` and without fast-math); its header states what is computed and which passage of the
NanoEuler pages each step follows.  This module only marshals numpy arrays:

* ``attn_fwd(q, k, v, causal, rope_base, rope_pairing) -> (o, lse)``
* ``attn_bwd(q, k, v, dO, causal, rope_base, rope_pairing) -> (dq, dk, dv)``
* ``rope(x, base, pairing, inverse) -> x rotated``
* ``attn_decode(q, k, v, lens) -> (o, lse)``: one query per (batch, head) against a key/value
  cache [B, Hkv, Tc, D], keys 0 .. lens[b] - 1 visible
* ``attn_prefill(q, k, v) -> (o, lse)``: a chunk of Tq queries [B, Hq, Tq, D] at positions
  Tk - Tq .. Tk - 1 against keys [B, Hkv, Tk, D], causal

Shapes: q, dO: [B, Hq, T, D]; k, v: [B, Hkv, T, D]; lse: [B, Hq, T].  Inputs of any float
dtype are converted exactly to float64.  ``rope_base = 0`` disables RoPE.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_attn.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

__all__ = ["build", "attn_fwd", "attn_bwd", "attn_decode", "attn_prefill", "rope",
           "num_threads"]


def build() -> str:
    """Compiles ``oracle_attn.c`` into ``liboracle.so`` next to it and returns its path."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_attn_fwd.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i, ctypes.c_double, i]
    lib.oracle_attn_fwd.restype = i
    lib.oracle_attn_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i,
                                    ctypes.c_double, i]
    lib.oracle_attn_bwd.restype = i
    lib.oracle_attn_decode.argtypes = [dp, dp, dp, ctypes.POINTER(ctypes.c_int), dp, dp,
                                       i, i, i, i, i]
    lib.oracle_attn_decode.restype = i
    lib.oracle_attn_prefill.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i]
    lib.oracle_attn_prefill.restype = i
    lib.oracle_rope.argtypes = [dp, i, i, i, i, ctypes.c_double, i, i]
    lib.oracle_rope.restype = i
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, T, D]")
    B, Hq, T, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != (T, D):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    return B, Hq, k.shape[1], T, D


def _check(rc: int, what: str):
    if rc == -1:
        raise ValueError(f"{what}: invalid argument")
    if rc != 0:
        raise MemoryError(f"{what}: out of host memory")


def attn_fwd(q, k, v, causal: bool = True, rope_base: float = 0.0, rope_pairing: int = 0):
    """Returns (o [B,Hq,T,D], lse [B,Hq,T]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, T, D = _shapes(q, k, v)
    o = np.empty_like(q)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    rc = _load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, T,
                                 D, int(bool(causal)), float(rope_base), int(rope_pairing))
    _check(rc, "oracle_attn_fwd")
    return o, lse


def attn_bwd(q, k, v, dO, causal: bool = True, rope_base: float = 0.0, rope_pairing: int = 0):
    """Returns (dq, dk, dv) in float64, the gradient of sum(dO * o) with respect to q, k, v."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, Hq, Hkv, T, D = _shapes(q, k, v)
    if dO.shape != q.shape:
        raise ValueError("dO must have the shape of q")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = _load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, Hq, Hkv, T, D, int(bool(causal)),
                                 float(rope_base), int(rope_pairing))
    _check(rc, "oracle_attn_bwd")
    return dq, dk, dv


def attn_decode(q, k, v, lens):
    """q [B,Hq,D]; k, v [B,Hkv,Tc,D]; lens [B] -> (o [B,Hq,D], lse [B,Hq]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 3 or k.ndim != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, D], k and v [B, Hkv, Tc, D]")
    B, Hq, D = q.shape
    _, Hkv, Tc, Dk = k.shape
    if k.shape[0] != B or Dk != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    ln = np.ascontiguousarray(np.asarray(lens, dtype=np.int32).reshape(B))
    o = np.empty_like(q)
    lse = np.empty((B, Hq), dtype=np.float64)
    rc = _load().oracle_attn_decode(_ptr(q), _ptr(k), _ptr(v),
                                    ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), _ptr(o),
                                    _ptr(lse), B, Hq, Hkv, Tc, D)
    _check(rc, "oracle_attn_decode")
    return o, lse


def attn_prefill(q, k, v):
    """q [B,Hq,Tq,D] at positions Tk-Tq .. Tk-1; k, v [B,Hkv,Tk,D] -> (o [B,Hq,Tq,D],
    lse [B,Hq,Tq]) in float64, causal."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, Tq, D], k and v [B, Hkv, Tk, D]")
    B, Hq, Tq, D = q.shape
    _, Hkv, Tk, Dk = k.shape
    if k.shape[0] != B or Dk != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    o = np.empty_like(q)
    lse = np.empty((B, Hq, Tq), dtype=np.float64)
    rc = _load().oracle_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                     Tq, Tk, D)
    _check(rc, "oracle_attn_prefill")
    return o, lse


def rope(x, base: float, pairing: int = 0, inverse: bool = False) -> np.ndarray:
    """Rotates every [T, D] head of x [B, H, T, D] (a copy is returned)."""
    y = _f64(x).copy()
    B, H, T, D = y.shape
    rc = _load().oracle_rope(_ptr(y), B, H, T, D, float(base), int(pairing), int(bool(inverse)))
    _check(rc, "oracle_rope")
    return y


def num_threads() -> int:
    """OpenMP threads a parallel region of the oracle uses."""
    return int(_load().oracle_num_threads())
