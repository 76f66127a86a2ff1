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
_CONV_SRC = os.path.join(_HERE, "short_conv_oracle.c")
_CONV_LIB = os.path.join(_HERE, "liboracle_short_conv.so")
_handle = None
_conv_handle = None


def library_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile the oracles with gcc (plain -O2, fp64, pthreads)."""
    for src, lib in ((_SRC, _LIB), (_CONV_SRC, _CONV_LIB)):
        if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src):
            tmp = lib + f".tmp{os.getpid()}"
            subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, src,
                            "-lm", "-lpthread"], check=True)
            os.replace(tmp, lib)
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


def _load_conv(path: str):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.kda_oracle_short_conv.argtypes = [dp, dp, dp, ip, ip, ip] + [ctypes.c_int32] * 6 + [dp]
    lib.kda_oracle_short_conv.restype = ctypes.c_int
    if hasattr(lib, "kda_oracle_short_conv_backward"):
        lib.kda_oracle_short_conv_backward.argtypes = [dp, dp, dp, ip, ip, ip] + [ctypes.c_int32] * 6 + [dp] * 4
        lib.kda_oracle_short_conv_backward.restype = ctypes.c_int
    return lib


def short_conv(x, w_text, w_vis, cu_seqlens, text_len, grid, _library=None):
    """Direct fp64 modality-aware short convolution.

    x: [T, C]; w_text: [kx, C]; w_vis: [kt, kh, kw, C]; cu_seqlens: [N+1]; text_len: [N];
    grid: [N, 3] (frames, height, width) with text_len + frames*height*width = each sample's
    length. Returns y [T, C] in fp64.
    """
    global _conv_handle
    x = np.ascontiguousarray(x, np.float64)
    wt = np.ascontiguousarray(w_text, np.float64)
    wv = np.ascontiguousarray(w_vis, np.float64)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    tl = np.ascontiguousarray(text_len, np.int32)
    gr = np.ascontiguousarray(grid, np.int32).reshape(-1, 3)
    T, C = x.shape
    N = len(cu) - 1
    assert wt.shape[1] == C and wv.shape[3] == C and tl.shape == (N,) and gr.shape == (N, 3)
    y = np.zeros((T, C))
    if _library is None:
        if _conv_handle is None:
            build()
            _conv_handle = _load_conv(_CONV_LIB)
        lib = _conv_handle
    else:
        lib = _library
    P = ctypes.c_double
    I = ctypes.c_int32
    rc = lib.kda_oracle_short_conv(_ptr(x, P), _ptr(wt, P), _ptr(wv, P), _ptr(cu, I), _ptr(tl, I),
                                   _ptr(gr, I), N, C, wt.shape[0], wv.shape[0], wv.shape[1],
                                   wv.shape[2], _ptr(y, P))
    if rc != 0:
        raise RuntimeError("kda_oracle_short_conv failed (bad arguments)")
    return y


def short_conv_backward(x, w_text, w_vis, cu_seqlens, text_len, grid, dy, _library=None):
    """Reverse mode of short_conv: the gradients (dx [T, C], dw_text [kx, C], dw_vis
    [kt, kh, kw, C]) of a loss with gradient dy [T, C] with respect to y, in fp64."""
    global _conv_handle
    x = np.ascontiguousarray(x, np.float64)
    wt = np.ascontiguousarray(w_text, np.float64)
    wv = np.ascontiguousarray(w_vis, np.float64)
    g = np.ascontiguousarray(dy, np.float64)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    tl = np.ascontiguousarray(text_len, np.int32)
    gr = np.ascontiguousarray(grid, np.int32).reshape(-1, 3)
    T, C = x.shape
    N = len(cu) - 1
    assert g.shape == x.shape and wt.shape[1] == C and wv.shape[3] == C and tl.shape == (N,) and gr.shape == (N, 3)
    dx = np.zeros((T, C))
    dwt = np.zeros(wt.shape)
    dwv = np.zeros(wv.shape)
    if _library is None:
        if _conv_handle is None:
            build()
            _conv_handle = _load_conv(_CONV_LIB)
        lib = _conv_handle
    else:
        lib = _library
    P = ctypes.c_double
    I = ctypes.c_int32
    rc = lib.kda_oracle_short_conv_backward(_ptr(x, P), _ptr(wt, P), _ptr(wv, P), _ptr(cu, I), _ptr(tl, I),
                                            _ptr(gr, I), N, C, wt.shape[0], wv.shape[0], wv.shape[1],
                                            wv.shape[2], _ptr(g, P), _ptr(dx, P), _ptr(dwt, P), _ptr(dwv, P))
    if rc != 0:
        raise RuntimeError("kda_oracle_short_conv_backward failed (bad arguments)")
    return dx, dwt, dwv


def short_conv_backward_from(path: str):
    """short_conv_backward() bound to another build of the same C source (mutation tests)."""
    lib = _load_conv(path)

    def conv_bwd(*args, **kw):
        return short_conv_backward(*args, _library=lib, **kw)
    return conv_bwd


def short_conv_from(path: str):
    """short_conv() bound to another build of the same C source (mutation tests)."""
    lib = _load_conv(path)

    def conv(*args, **kw):
        return short_conv(*args, _library=lib, **kw)
    return conv
