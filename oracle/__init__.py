"""CPU oracle for the fused attention forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg
may import this package.  The HIP library and its Python binding never do,
and nothing here imports them: the oracle and the GPU path share no code.

Two independent implementations of the same plain definition live here:
  * ``fa_oracle.c``  -- C, double precision, OpenMP over query rows
                        (``forward`` / ``forward_rows`` below);
  * ``oracle_np.py`` -- NumPy float64 (``oracle.oracle_np.attention_forward``).

Parity status: pinned.  The C oracle is checked against a 50-digit ``decimal``
brute force on tiny inputs, against closed forms (zero queries, a single key,
causal row 0, identical keys, constant values, identity values) and
invariants (row sums, shift and permutation invariance), against scipy's
``logsumexp``/``softmax`` on the same scores, and against the NumPy oracle.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfa_oracle.so")
_lib = None


def build(force=True):
    """Compile fa_oracle.c with gcc into oracle/libfa_oracle.so."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    if force or not os.path.exists(_LIB_PATH):
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.fa_oracle_fwd.restype = ctypes.c_int
        lib.fa_oracle_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int]
        lib.fa_oracle_max_threads.restype = ctypes.c_int
        lib.fa_oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def max_threads():
    """OpenMP threads the C oracle will use."""
    return _load().fa_oracle_max_threads()


def _c64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def forward(q, k, v, sm_scale, causal, lib=None):
    """C oracle over all rows.  q [B,H,Sq,D], k/v [B,H,Sk,D] float64.

    Returns (o [B,H,Sq,D], lse [B,H,Sq]) float64.
    """
    return forward_rows(q, k, v, sm_scale, causal, rows=None, lib=lib)


def forward_rows(q, k, v, sm_scale, causal, rows=None, lib=None):
    """C oracle over selected flat query rows ((b*H + h)*Sq + i).

    With rows=None every row is computed and the outputs keep their
    [B,H,Sq,...] shape; otherwise o is [len(rows), D] and lse [len(rows)].
    """
    lib = lib or _load()
    q, k, v = _c64(q), _c64(k), _c64(v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    assert k.shape == (B, H, Sk, D) and v.shape == (B, H, Sk, D)
    if rows is None:
        o = np.empty((B, H, Sq, D), np.float64)
        lse = np.empty((B, H, Sq), np.float64)
        rows_ptr, n = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        o = np.empty((rows.size, D), np.float64)
        lse = np.empty((rows.size,), np.float64)
        rows_ptr, n = rows.ctypes.data, rows.size
    rc = lib.fa_oracle_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                           lse.ctypes.data, B, H, Sq, Sk, D, rows_ptr, n,
                           float(sm_scale), int(bool(causal)))
    if rc != 0:
        raise ValueError(f"fa_oracle_fwd rejected its arguments (rc={rc})")
    return o, lse


def load_variant(path):
    """Load another build of fa_oracle.c (used by the planted-mistake tests)."""
    global _lib
    saved = _lib
    _lib = None
    try:
        lib = ctypes.CDLL(path)
        # reuse the prototype setup of _load on this handle
        lib.fa_oracle_fwd.restype = ctypes.c_int
        lib.fa_oracle_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int]
        return lib
    finally:
        _lib = saved
