"""CPU fp64 oracle for shared-history cross-attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The product path
(``shared_history_candidate_amd``) never imports, links or runs anything here.

The arithmetic lives in ``xattn_oracle.c`` (plain fp64 loops, OpenMP over
output rows).  This module only compiles it with gcc and marshals numpy arrays.
Each function states the passage it follows; see the C file for the readings
taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "xattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        Lg = ctypes.c_long
        lib.oracle_project.argtypes = [Lg, I, I, P, P, P]
        lib.oracle_forward.argtypes = [I, P, P, I, I, I, P, P, P, P, P, Lg, P]
        lib.oracle_probs.argtypes = [I, P, P, I, I, I, P, P, P, Lg, I, P]
        lib.oracle_plan.argtypes = [I, P, P, I, I, P, P, P, Lg, P]
        lib.oracle_output.argtypes = [Lg, I, I, P, P, P, P, P]
        lib.oracle_forward_prefix.argtypes = [I, P, P, I, I, I, P, P, P, P, P, P, Lg, P]
        lib.oracle_backward.argtypes = [I, P, P, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
        for f in (lib.oracle_project, lib.oracle_forward, lib.oracle_probs, lib.oracle_plan,
                  lib.oracle_output, lib.oracle_forward_prefix, lib.oracle_backward):
            f.restype = I
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def set_threads(n: int) -> None:
    """Set the OpenMP thread count used by the oracle (results do not depend on it)."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


def project(Z, wt, q: int) -> np.ndarray:
    """TSP projection (ReST reading note, s.3.3.2 Eq. (8) on Eq. (7)'s W_Q):
    Q[row] = Z[row] @ wt[row % q].T, with wt[s] stored output-major [d_out, d_in]."""
    Z = _f64(Z)
    wt = _f64(wt)
    d = Z.shape[-1]
    Z2 = Z.reshape(-1, d)
    Q = np.empty_like(Z2)
    rc = _load().oracle_project(Z2.shape[0], q, d, _ptr(Z2), _ptr(wt), _ptr(Q))
    if rc != 0:
        raise ValueError("oracle_project: invalid arguments")
    return Q.reshape(Z.shape)


def output(Z, wgo, O, wo, q: int) -> np.ndarray:
    """Output gate and projection of Eq. (7) (ReST reading note, s.3.3.1) with
    the per-slot gate weights of Eq. (8) (s.3.3.2):
    Y[row] = (O[row] * sigmoid(Z[row] @ wgo[row % q].T)) @ wo.T, weights stored
    output-major.  Z, O: [rows, d] (or [cand, q, d]); returns [rows, d]."""
    wgo = _f64(wgo)
    d = wgo.shape[-1]
    Z2 = _f64(Z).reshape(-1, d)
    O2 = _f64(O).reshape(-1, d)
    assert Z2.shape == O2.shape
    Y = np.empty_like(Z2)
    rc = _load().oracle_output(Z2.shape[0], q, d, _ptr(Z2), _ptr(wgo), _ptr(O2),
                               _ptr(_f64(wo)), _ptr(Y))
    if rc != 0:
        raise ValueError("oracle_output: invalid arguments")
    return Y


def forward(cu_kv, cu_cand, q: int, heads: int, Z, wt, K, V=None, rows=None,
            kv_len=None) -> np.ndarray:
    """Cross-attention of Eq. (7) (ReST reading note s.3.3.1) without gate/W_o,
    per-slot W_Q of Eq. (8), K = V = H when V is None, separate K/V otherwise
    (TransX report s.2).  kv_len (one int per candidate, optional) limits each
    candidate to a prefix of its request's memory (ReST reading note s.3.5,
    ULT).  Returns O [n_rows, d] (all rows c*q+s when rows is None)."""
    cu_kv = _i32(cu_kv)
    cu_cand = _i32(cu_cand)
    R = len(cu_kv) - 1
    Z = _f64(Z)
    d = Z.shape[-1]
    Z2 = Z.reshape(-1, d)
    wt = _f64(wt)
    K = _f64(K).reshape(-1, d)
    Vd = _f64(V).reshape(-1, d) if V is not None else None
    if rows is not None:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n_out = len(rows_a)
    else:
        rows_a = None
        n_out = Z2.shape[0]
    O = np.empty((n_out, d), dtype=np.float64)
    if kv_len is not None:
        kl = _i32(kv_len)
        assert kl.shape == (int(cu_cand[-1]),)
        rc = _load().oracle_forward_prefix(R, _ptr(cu_kv), _ptr(cu_cand), q, d, heads,
                                           _ptr(Z2), _ptr(wt), _ptr(K), _ptr(Vd), _ptr(kl),
                                           _ptr(rows_a), n_out if rows_a is not None else 0,
                                           _ptr(O))
    else:
        rc = _load().oracle_forward(R, _ptr(cu_kv), _ptr(cu_cand), q, d, heads, _ptr(Z2),
                                    _ptr(wt), _ptr(K), _ptr(Vd), _ptr(rows_a),
                                    n_out if rows_a is not None else 0, _ptr(O))
    if rc != 0:
        raise ValueError("oracle_forward: invalid arguments")
    return O


def probs(cu_kv, cu_cand, q: int, heads: int, Z, wt, K, row: int, head: int) -> np.ndarray:
    """Softmax weights of one (row, head) over its request's memory rows (Eq. (7))."""
    cu_kv = _i32(cu_kv)
    cu_cand = _i32(cu_cand)
    R = len(cu_kv) - 1
    Z = _f64(Z)
    d = Z.shape[-1]
    Z2 = Z.reshape(-1, d)
    r = int(np.searchsorted(cu_cand * q, row, side="right") - 1)
    L = int(cu_kv[r + 1] - cu_kv[r])
    p = np.zeros(max(L, 1), dtype=np.float64)
    rc = _load().oracle_probs(R, _ptr(cu_kv), _ptr(cu_cand), q, d, heads, _ptr(Z2),
                              _ptr(_f64(wt)), _ptr(_f64(K).reshape(-1, d)), row, head, _ptr(p))
    if rc != 0:
        raise ValueError("oracle_probs: invalid arguments")
    return p[:L]


def plan(cu_kv, cu_cand, q: int, tile_m: int, with_row_req: bool = True):
    """Integer varlen plan: (cu_q, row_req, tiles[n,4]) with the ordering rule in
    xattn_oracle.c (requests by L desc, ties by index; blocks then slots)."""
    cu_kv = _i32(cu_kv)
    cu_cand = _i32(cu_cand)
    R = len(cu_kv) - 1
    cu_q = np.zeros(R + 1, dtype=np.int32)
    total_rows = int(cu_cand[-1]) * q
    row_req = np.zeros(max(total_rows, 1), dtype=np.int32) if with_row_req else None
    n = ctypes.c_long(0)
    lib = _load()
    rc = lib.oracle_plan(R, _ptr(cu_kv), _ptr(cu_cand), q, tile_m, _ptr(cu_q), None, None, 0,
                         ctypes.byref(n))
    if rc != 0:
        raise ValueError("oracle_plan: invalid arguments")
    tiles = np.zeros((max(n.value, 1), 4), dtype=np.int32)
    rc = lib.oracle_plan(R, _ptr(cu_kv), _ptr(cu_cand), q, tile_m, _ptr(cu_q), _ptr(row_req),
                         _ptr(tiles), n.value, ctypes.byref(n))
    if rc != 0:
        raise ValueError("oracle_plan: invalid arguments")
    return cu_q, (row_req[:total_rows] if with_row_req else None), tiles[: n.value]


def backward(cu_kv, cu_cand, q: int, heads: int, Z, wt, K, V, dO, kv_len=None) -> dict:
    """Gradients of <dO, forward(...)> (the backward pass of the cross-attention;
    ReST reading note s.3.3.1 Eq. (7) with Eq. (8)'s per-slot W_Q, TransX
    report s.2: candidate gradients summed back into the one memory).
    Returns dQ, dZ [rows, d], dwt [q, d, d] (output-major like wt), dK
    [total_kv, d] (the gradient of H, both roles, when V is None) and dV
    (None when V is None).  kv_len: optional per-candidate prefix cutoff as
    in forward()."""
    cu_kv = _i32(cu_kv)
    cu_cand = _i32(cu_cand)
    R = len(cu_kv) - 1
    wt = _f64(wt)
    d = wt.shape[-1]
    Z2 = _f64(Z).reshape(-1, d)
    dO2 = _f64(dO).reshape(-1, d)
    assert Z2.shape == dO2.shape
    K2 = _f64(K).reshape(-1, d)
    V2 = _f64(V).reshape(-1, d) if V is not None else None
    kl = _i32(kv_len) if kv_len is not None else None
    if kl is not None:
        assert kl.shape == (int(cu_cand[-1]),)
    out = {"dQ": np.empty_like(Z2), "dZ": np.empty_like(Z2), "dwt": np.empty_like(wt),
           "dK": np.empty_like(K2), "dV": np.empty_like(V2) if V2 is not None else None}
    rc = _load().oracle_backward(R, _ptr(cu_kv), _ptr(cu_cand), q, d, heads, _ptr(Z2), _ptr(wt),
                                 _ptr(K2), _ptr(V2), _ptr(kl), _ptr(dO2), _ptr(out["dQ"]),
                                 _ptr(out["dZ"]), _ptr(out["dwt"]), _ptr(out["dK"]),
                                 _ptr(out["dV"]))
    if rc != 0:
        raise ValueError("oracle_backward: invalid arguments")
    return out
