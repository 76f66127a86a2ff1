"""ctypes wrapper around kda_oracle.c -- test infrastructure only.

Builds ``liboracle_kda.so`` next to the C file with gcc when it is missing or
older than the source. All arrays are fp64 (exact upcasts of stored values).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_kda.so")
_handle = None


def library_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, fp64, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC,
                        "-lm", "-lpthread"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load(path: str):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_forward.argtypes = [dp, dp, dp, dp, dp,
                                       ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_uint8), dp, dp, ctypes.c_int32]
    lib.kda_oracle_forward.restype = ctypes.c_int
    lib.kda_oracle_forward_from.argtypes = [dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32), dp,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.POINTER(ctypes.c_uint8), dp, dp,
                                            ctypes.c_int32]
    lib.kda_oracle_forward_from.restype = ctypes.c_int
    lib.kda_oracle_forward_ex.argtypes = [dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32), dp,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_uint8), dp, dp, ctypes.c_int32]
    lib.kda_oracle_forward_ex.restype = ctypes.c_int
    lib.kda_oracle_backward.argtypes = [dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32), dp,
                                        ctypes.c_int32, dp, dp, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, dp, dp, dp, dp, dp, dp,
                                        ctypes.c_int32]
    lib.kda_oracle_backward.restype = ctypes.c_int
    return lib


def _lib():
    global _handle
    if _handle is None:
        build()
        _handle = _load(_LIB)
    return _handle


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def forward(q, k, v, log_alpha, beta, cu_seqlens, heads: Optional[Sequence[int]] = None,
            threads: Optional[int] = None, _library=None, initial_state=None,
            qk_l2norm: bool = False):
    """Token-by-token fp64 recurrence.

    q, k, log_alpha: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; cu_seqlens: [N+1];
    initial_state: [N, H, dk, dv] or None (zero states); qk_l2norm: divide q_t and k_t
    by their Euclidean length before the recurrence (zero vectors stay zero). Returns (out [T, H, dv],
    final_state [N, H, dk, dv]) in fp64. With ``heads`` only those head slices are
    computed (other rows of ``out`` are NaN and the other final states zero, or the
    initial state where one is given).
    """
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    la = np.ascontiguousarray(log_alpha, np.float64)
    b = np.ascontiguousarray(beta, np.float64)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    T, H, dk = k.shape
    dv = v.shape[2]
    assert q.shape == k.shape == la.shape and v.shape[:2] == (T, H) and b.shape == (T, H)
    N = len(cu) - 1
    assert N >= 0 and cu[0] == 0 and cu[-1] == T
    out = np.full((T, H, dv), np.nan)
    fs = np.zeros((N, H, dk, dv))
    mask = None
    if heads is not None:
        mask = np.zeros(H, np.uint8)
        mask[list(heads)] = 1
    if threads is None:
        threads = min(os.cpu_count() or 1, 64)
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, np.float64)
        assert s0.shape == (N, H, dk, dv)
        fs[:] = s0
    lib = _lib() if _library is None else _library
    rc = lib.kda_oracle_forward_ex(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                   _ptr(v, ctypes.c_double), _ptr(la, ctypes.c_double),
                                   _ptr(b, ctypes.c_double), _ptr(cu, ctypes.c_int32),
                                   _ptr(s0, ctypes.c_double), int(bool(qk_l2norm)), N, H, dk, dv,
                                     _ptr(mask, ctypes.c_uint8), _ptr(out, ctypes.c_double),
                                     _ptr(fs, ctypes.c_double), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_forward failed (bad arguments or out of memory)")
    return out, fs


def backward(q, k, v, log_alpha, beta, cu_seqlens, d_out, d_final_state=None, initial_state=None,
             qk_l2norm: bool = False, threads: Optional[int] = None, _library=None):
    """Reverse-mode fp64 gradients of L = sum(d_out * out) + sum(d_final_state * final_state).

    Shapes as forward(); d_out like out, d_final_state like final_state (None = 0).
    Returns (dq, dk, dv, dlog_alpha, dbeta, d_initial_state) in fp64; d_initial_state is
    the gradient with respect to the initial states (zero states when none are given).
    """
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    la = np.ascontiguousarray(log_alpha, np.float64)
    b = np.ascontiguousarray(beta, np.float64)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    do = np.ascontiguousarray(d_out, np.float64)
    T, H, dk = k.shape
    dv = v.shape[2]
    N = len(cu) - 1
    assert q.shape == k.shape == la.shape and v.shape == do.shape == (T, H, dv) and b.shape == (T, H)
    assert N >= 0 and cu[0] == 0 and cu[-1] == T
    dfs = None if d_final_state is None else np.ascontiguousarray(d_final_state, np.float64)
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, np.float64)
    for x in (dfs, s0):
        assert x is None or x.shape == (N, H, dk, dv)
    g = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(la), np.zeros_like(b)]
    ds0 = np.zeros((N, H, dk, dv))
    if threads is None:
        threads = min(os.cpu_count() or 1, 64)
    lib = _lib() if _library is None else _library
    P = ctypes.c_double
    rc = lib.kda_oracle_backward(_ptr(q, P), _ptr(k, P), _ptr(v, P), _ptr(la, P), _ptr(b, P),
                                 _ptr(cu, ctypes.c_int32), _ptr(s0, P), int(bool(qk_l2norm)),
                                 _ptr(do, P), _ptr(dfs, P), N, H, dk, dv, *[_ptr(x, P) for x in g],
                                 _ptr(ds0, P), int(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_backward failed (bad arguments or out of memory)")
    return (*g, ds0)


def forward_from(path: str):
    """A forward() bound to another build of the same C source (mutation tests)."""
    lib = _load(path)

    def fwd(*args, **kw):
        return forward(*args, _library=lib, **kw)
    return fwd


def backward_from(path: str):
    """A backward() bound to another build of the same C source (mutation tests)."""
    lib = _load(path)

    def bwd(*args, **kw):
        return backward(*args, _library=lib, **kw)
    return bwd
