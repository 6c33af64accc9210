"""Build and load the fp64 oracle library (oracle/attention.c).

TEST INFRASTRUCTURE ONLY: the product path never imports this module.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attention.c")
LIBRARY = os.path.join(_HERE, "liboracle_attention.so")
MODEL_SOURCE = os.path.join(_HERE, "model.c")
MODEL_LIBRARY = os.path.join(_HERE, "liboracle_model.so")
_lib = None
_model = None


def _compile(source, library, force):
    if not force and os.path.exists(library) and os.path.getmtime(library) >= os.path.getmtime(source):
        return library
    tmp = library + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                    "-o", tmp, source, "-lm"], check=True)
    os.replace(tmp, library)
    return library


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into oracle/."""
    _compile(MODEL_SOURCE, MODEL_LIBRARY, force)
    return _compile(SOURCE, LIBRARY, force)


def model_lib():
    global _model
    if _model is None:
        _compile(MODEL_SOURCE, MODEL_LIBRARY, False)
        L = ctypes.CDLL(MODEL_LIBRARY)
        L.oracle_linear.restype = None
        L.oracle_linear.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
        L.oracle_rmsnorm.restype = None
        L.oracle_rmsnorm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                     ctypes.c_void_p]
        _model = L
    return _model


def linear(a, w):
    """y = a W^T in fp64 with explicit loops (oracle/model.c): a [m][k], w [n][k] -> [m][n]."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    m, k = a.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("shape mismatch")
    out = np.empty((m, n), dtype=np.float64)
    model_lib().oracle_linear(m, n, k, a.ctypes.data, w.ctypes.data, out.ctypes.data)
    return out


def rmsnorm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w per row, fp64 (oracle/model.c)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    rows, dm = x.shape
    if w.shape != (dm,):
        raise ValueError("shape mismatch")
    out = np.empty_like(x)
    model_lib().oracle_rmsnorm(rows, dm, x.ctypes.data, w.ctypes.data, float(eps), out.ctypes.data)
    return out


def load(path: str):
    """Load a compiled copy of attention.c and return its entry point."""
    L = ctypes.CDLL(path)
    f = L.oracle_link_attention
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
    f._keepalive = L
    return f


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = load(LIBRARY)
    return _lib


def attention(k, v, key_pos, q, row_pos, rope_theta, entry=None, key_rot=None):
    """fp64 causal RoPE attention; see attention.c. Returns (out [R][Hq][d], lse [R][Hq]).

    ``key_rot`` (optional, [n_keys]) is the position each key is rotated by; by
    default its absolute position ``key_pos``.
    """
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    key_pos = np.ascontiguousarray(key_pos, dtype=np.int64)
    row_pos = np.ascontiguousarray(row_pos, dtype=np.int64)
    if key_rot is not None:
        key_rot = np.ascontiguousarray(key_rot, dtype=np.int64)
        if key_rot.shape != key_pos.shape:
            raise ValueError("shape mismatch")
    n_keys, hkv, d = k.shape
    n_rows, hq, dq = q.shape
    if v.shape != k.shape or dq != d or key_pos.shape != (n_keys,) or row_pos.shape != (n_rows,):
        raise ValueError("shape mismatch")
    out = np.empty((n_rows, hq, d), dtype=np.float64)
    lse = np.empty((n_rows, hq), dtype=np.float64)
    fn = entry if entry is not None else lib()
    rc = fn(n_keys, hkv, hq, d, k.ctypes.data, v.ctypes.data,
                                     key_pos.ctypes.data, None if key_rot is None else key_rot.ctypes.data,
                                     n_rows, q.ctypes.data,
                                     row_pos.ctypes.data, float(rope_theta),
                                     out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_link_attention failed with {rc}")
    return out, lse
