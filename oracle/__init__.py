"""CPU oracle for the fused attention forward and its gradients -- TEST
INFRASTRUCTURE ONLY.

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg
may import this package.  The HIP library and its Python binding never do,
and nothing here imports them: the oracle and the GPU path share no code.

Two independent implementations of the same plain definitions live here:
  * ``fa_oracle.c``  -- C, double precision, OpenMP over query rows
                        (``forward`` / ``forward_rows`` below);
  * ``fa_oracle_bwd.c`` -- C, double precision, the gradients dQ, dK, dV
                        (``backward``, ``backward_dq_rows``, ``backward_dkv_rows``);
  * ``oracle_np.py`` -- NumPy float64 (``attention_forward``, ``attention_backward``).

Parity status: pinned.  The C oracle is checked against a 50-digit ``decimal``
brute force on tiny inputs, against closed forms (zero queries, a single key,
causal row 0, identical keys, constant values, identity values) and
invariants (row sums, shift and permutation invariance), against scipy's
``logsumexp``/``softmax`` on the same scores, and against the NumPy oracle.
The gradient oracle is checked against central finite differences of the
forward oracle, against torch autograd on the CPU in float64, against closed
forms (zero gradients for identical keys, constant values or zero dO) and
invariants (sum over keys of dK is 0, sum over keys of dV equals the sum of
dO), and against the NumPy oracle.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_SRC_BWD = os.path.join(_HERE, "fa_oracle_bwd.c")
_LIB_PATH = os.path.join(_HERE, "libfa_oracle.so")
_lib = None


def build(force=True):
    """Compile fa_oracle.c and fa_oracle_bwd.c with gcc into oracle/libfa_oracle.so."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           _SRC, _SRC_BWD, "-o", tmp, "-lm"]
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
        _bwd_prototypes(lib)
        _lib = lib
    return _lib


def _bwd_prototypes(lib):
    vp, i64, dbl, cint = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
    shape = [i64, i64, i64, i64, i64, dbl, cint]
    lib.fa_oracle_bwd.restype = cint
    lib.fa_oracle_bwd.argtypes = [vp] * 8 + shape
    lib.fa_oracle_bwd_dq_rows.restype = cint
    lib.fa_oracle_bwd_dq_rows.argtypes = [vp] * 4 + [vp, i64, vp] + shape
    lib.fa_oracle_bwd_dkv_rows.restype = cint
    lib.fa_oracle_bwd_dkv_rows.argtypes = [vp] * 4 + [vp, i64, vp, vp] + shape


def load_bwd_variant(path):
    """Load another build of fa_oracle_bwd.c alone (planted-mistake tests)."""
    lib = ctypes.CDLL(path)
    _bwd_prototypes(lib)
    return lib


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


def _bwd_shapes(q, k, v, dout):
    q, k, v, dout = _c64(q), _c64(k), _c64(v), _c64(dout)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    assert k.shape == (B, H, Sk, D) and v.shape == (B, H, Sk, D) and dout.shape == q.shape
    return q, k, v, dout, (B, H, Sq, Sk, D)


def backward(q, k, v, dout, sm_scale, causal, lib=None):
    """Gradients of O = attention(q, k, v) for the upstream gradient dout.

    Returns (dq, dk, dv, delta) float64 with delta[B,H,Sq] = rowsum(dout * O).
    """
    lib = lib or _load()
    q, k, v, dout, (B, H, Sq, Sk, D) = _bwd_shapes(q, k, v, dout)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    delta = np.empty((B, H, Sq), np.float64)
    rc = lib.fa_oracle_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                           dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, delta.ctypes.data,
                           B, H, Sq, Sk, D, float(sm_scale), int(bool(causal)))
    if rc != 0:
        raise ValueError(f"fa_oracle_bwd rejected its arguments (rc={rc})")
    return dq, dk, dv, delta


def backward_dq_rows(q, k, v, dout, sm_scale, causal, rows, lib=None):
    """dQ of the flat query rows ((b*H + h)*Sq + i); returns [len(rows), D]."""
    lib = lib or _load()
    q, k, v, dout, (B, H, Sq, Sk, D) = _bwd_shapes(q, k, v, dout)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    dq = np.empty((rows.size, D), np.float64)
    rc = lib.fa_oracle_bwd_dq_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                   rows.ctypes.data, rows.size, dq.ctypes.data, B, H, Sq, Sk, D,
                                   float(sm_scale), int(bool(causal)))
    if rc != 0:
        raise ValueError(f"fa_oracle_bwd_dq_rows rejected its arguments (rc={rc})")
    return dq


def backward_dkv_rows(q, k, v, dout, sm_scale, causal, keys, lib=None):
    """dK and dV of the flat key rows ((b*H + h)*Sk + j); returns two [len(keys), D]."""
    lib = lib or _load()
    q, k, v, dout, (B, H, Sq, Sk, D) = _bwd_shapes(q, k, v, dout)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    dk = np.empty((keys.size, D), np.float64)
    dv = np.empty((keys.size, D), np.float64)
    rc = lib.fa_oracle_bwd_dkv_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                    dout.ctypes.data, keys.ctypes.data, keys.size, dk.ctypes.data,
                                    dv.ctypes.data, B, H, Sq, Sk, D, float(sm_scale),
                                    int(bool(causal)))
    if rc != 0:
        raise ValueError(f"fa_oracle_bwd_dkv_rows rejected its arguments (rc={rc})")
    return dk, dv
