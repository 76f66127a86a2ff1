"""Python binding of libkda (ctypes). Argument marshalling only.

Every step of the scan runs in the HIP kernels of libkda.so; there is no
fallback. If the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1
KDA_OPT_QK_L2NORM = 1   # kda_forward_ex option: unit-length q_t, k_t
STATUS = {0: "KDA_OK", 1: "KDA_E_NULL", 2: "KDA_E_DTYPE", 3: "KDA_E_SHAPE", 4: "KDA_E_ALIGN",
          5: "KDA_E_UNSUPPORTED", 6: "KDA_E_SEQLENS", 7: "KDA_E_HIP"}

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def library() -> ctypes.CDLL:
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m delta_rule_recurrent_kda_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        lib.kda_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                    vp]
        lib.kda_forward.restype = ctypes.c_int
        lib.kda_status_str.argtypes = [ctypes.c_int]
        lib.kda_status_str.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_version.argtypes = []
        lib.kda_version.restype = ctypes.c_int32
        lib.kda_forward_from_state.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int, vp]
        lib.kda_forward_from_state.restype = ctypes.c_int
        lib.kda_forward_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int, ctypes.c_uint32, vp]
        lib.kda_forward_ex.restype = ctypes.c_int
        lib.kda_forward_noalloc.argtypes = lib.kda_forward_ex.argtypes
        lib.kda_forward_noalloc.restype = ctypes.c_int
        lib.kda_backward.argtypes = [vp] * 15 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                                 ctypes.c_uint32, vp]
        lib.kda_backward.restype = ctypes.c_int
        lib.kda_backward_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.c_int32]
        lib.kda_backward_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_short_conv.argtypes = [vp] * 7 + [ctypes.c_int64] + [ctypes.c_int32] * 6 + [ctypes.c_int, vp]
        lib.kda_short_conv.restype = ctypes.c_int
        lib.kda_short_conv_backward.argtypes = [vp] * 10 + [ctypes.c_int64] + [ctypes.c_int32] * 6 + [ctypes.c_int, vp]
        lib.kda_short_conv_backward.restype = ctypes.c_int
        lib.kda_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
        lib.kda_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_timing_enable.argtypes = [ctypes.c_int32]
        lib.kda_timing_enable.restype = ctypes.c_int
        lib.kda_timing_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_double)]
        lib.kda_timing_read.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def kda_forward_raw(q, k, v, log_alpha, beta, cu_seqlens, out, final_state, total_tokens: int,
                    num_seqs: int, num_heads: int, d_k: int, d_v: int, dtype: int,
                    stream: Optional[int]) -> int:
    """Direct C call with integer device addresses; returns the status code."""
    return library().kda_forward(q, k, v, log_alpha, beta, cu_seqlens, out, final_state,
                                 int(total_tokens), int(num_seqs), int(num_heads), int(d_k),
                                 int(d_v), int(dtype), stream)


def kda_forward_from_state_raw(q, k, v, log_alpha, beta, cu_seqlens, initial_state, out,
                               final_state, total_tokens: int, num_seqs: int, num_heads: int,
                               d_k: int, d_v: int, dtype: int, stream: Optional[int]) -> int:
    """Direct C call of kda_forward_from_state; returns the status code."""
    return library().kda_forward_from_state(q, k, v, log_alpha, beta, cu_seqlens, initial_state,
                                            out, final_state, int(total_tokens), int(num_seqs),
                                            int(num_heads), int(d_k), int(d_v), int(dtype), stream)


def kda_forward_ex_raw(q, k, v, log_alpha, beta, cu_seqlens, initial_state, out, final_state,
                       total_tokens: int, num_seqs: int, num_heads: int, d_k: int, d_v: int,
                       dtype: int, options: int, stream: Optional[int]) -> int:
    """Direct C call of kda_forward_ex; returns the status code."""
    return library().kda_forward_ex(q, k, v, log_alpha, beta, cu_seqlens, initial_state, out,
                                    final_state, int(total_tokens), int(num_seqs), int(num_heads),
                                    int(d_k), int(d_v), int(dtype), int(options), stream)


def kda_forward_noalloc_raw(q, k, v, log_alpha, beta, cu_seqlens, initial_state, out, final_state,
                            total_tokens: int, num_seqs: int, num_heads: int, d_k: int, d_v: int,
                            dtype: int, options: int, stream: Optional[int]) -> int:
    """Direct C call of kda_forward_noalloc; returns the status code."""
    return library().kda_forward_noalloc(q, k, v, log_alpha, beta, cu_seqlens, initial_state, out,
                                         final_state, int(total_tokens), int(num_seqs), int(num_heads),
                                         int(d_k), int(d_v), int(dtype), int(options), stream)


def forward_noalloc(q, k, v, log_alpha, beta, cu_seqlens, out, final_state=None, initial_state=None,
                    qk_l2norm: bool = False, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Enqueue the scan through kda_forward_noalloc into caller-owned ``out`` (and
    ``final_state``); the library allocates nothing (same tensors as kda_forward)."""
    T, N, H, dk, dv, dt = _check(q, k, v, log_alpha, beta, cu_seqlens, out, final_state,
                                 initial_state)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = kda_forward_noalloc_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                 _ptr(cu_seqlens), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                 T, N, H, dk, dv, dt, KDA_OPT_QK_L2NORM if qk_l2norm else 0,
                                 stream.cuda_stream)
    if st != 0:
        raise KdaError(st, library().kda_last_error().decode())


def workspace_bytes(total_tokens: int, num_seqs: int, num_heads: int, d_k: int, d_v: int,
                    dtype: int) -> int:
    return int(library().kda_workspace_bytes(int(total_tokens), int(num_seqs), int(num_heads),
                                             int(d_k), int(d_v), int(dtype)))


def timing_enable(on: bool) -> None:
    library().kda_timing_enable(1 if on else 0)


def release() -> None:
    """kda_release: give the workspace memory that earlier calls freed back to the driver."""
    st = library().kda_release()
    if st != 0:
        raise KdaError(st, library().kda_last_error().decode())


def timing_read(kernel: str):
    """(launches, total milliseconds) of the named kernel since the last read."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    st = library().kda_timing_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms))
    if st != 0:
        raise KdaError(st, library().kda_last_error().decode())
    return int(n.value), float(ms.value)


def _check(q, k, v, log_alpha, beta, cu_seqlens, out, final_state, initial_state):
    tensors = {"q": q, "k": k, "v": v, "log_alpha": log_alpha, "beta": beta,
               "cu_seqlens": cu_seqlens, "out": out}
    if final_state is not None:
        tensors["final_state"] = final_state
    if initial_state is not None:
        tensors["initial_state"] = initial_state
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype == torch.bfloat16:
        dt = KDA_BF16
    elif q.dtype == torch.float32:
        dt = KDA_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name in ("k", "v", "log_alpha", "beta", "out"):
        if tensors[name].dtype != q.dtype:
            raise ValueError(f"{name} dtype {tensors[name].dtype} != q dtype {q.dtype}")
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    for name in ("final_state", "initial_state"):
        if name in tensors and tensors[name].dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape != (T, H, dv) or \
            out.shape != (T, H, dv) or beta.shape != (T, H) or cu_seqlens.dim() != 1:
        raise ValueError("inconsistent shapes")
    N = cu_seqlens.numel() - 1
    for name in ("final_state", "initial_state"):
        if name in tensors and tensors[name].shape != (N, H, dk, dv):
            raise ValueError(f"{name} must be [N, H, d_k, d_v]")
    return T, N, H, dk, dv, dt


def kda_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                beta: torch.Tensor, cu_seqlens: torch.Tensor, out: torch.Tensor,
                final_state: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None,
                initial_state: Optional[torch.Tensor] = None, qk_l2norm: bool = False) -> None:
    """Enqueue the KDA forward scan on ``stream`` (default: torch's current stream).

    q, k, log_alpha: [T, H, d_k]; v, out: [T, H, d_v]; beta: [T, H] (one dtype,
    float32 or bfloat16); cu_seqlens: int32 [N+1]; final_state and initial_state:
    float32 [N, H, d_k, d_v] or None. All on the same GPU, contiguous. With an
    initial_state the call goes to kda_forward_from_state; with qk_l2norm (q_t and
    k_t normalised to unit length inside the scan) to kda_forward_ex.
    """
    T, N, H, dk, dv, dt = _check(q, k, v, log_alpha, beta, cu_seqlens, out, final_state,
                                 initial_state)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if qk_l2norm:
        st = kda_forward_ex_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                _ptr(cu_seqlens), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                T, N, H, dk, dv, dt, KDA_OPT_QK_L2NORM, stream.cuda_stream)
    elif initial_state is None:
        st = kda_forward_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                             _ptr(cu_seqlens), _ptr(out), _ptr(final_state), T, N, H, dk, dv, dt,
                             stream.cuda_stream)
    else:
        st = kda_forward_from_state_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                        _ptr(cu_seqlens), _ptr(initial_state), _ptr(out),
                                        _ptr(final_state), T, N, H, dk, dv, dt, stream.cuda_stream)
    if st != 0:
        raise KdaError(st, library().kda_last_error().decode())


def forward(q, k, v, log_alpha, beta, cu_seqlens, with_state: bool = True,
            stream: Optional[torch.cuda.Stream] = None, initial_state=None, qk_l2norm: bool = False):
    """Allocate outputs and run the scan. Returns (out, final_state or None)."""
    T, H, _ = q.shape
    N = cu_seqlens.numel() - 1
    out = torch.empty((T, H, v.shape[2]), dtype=q.dtype, device=q.device)
    fs = torch.empty((N, H, q.shape[2], v.shape[2]), dtype=torch.float32, device=q.device) \
        if with_state else None
    kda_forward(q, k, v, log_alpha, beta, cu_seqlens, out, fs, stream, initial_state, qk_l2norm)
    return out, fs


def kda_backward_raw(q, k, v, log_alpha, beta, cu_seqlens, initial_state, d_out, d_final_state, dq,
                     dk, dv, dlog_alpha, dbeta, d_initial_state, total_tokens: int, num_seqs: int,
                     num_heads: int, d_k: int, d_v: int, dtype: int, options: int,
                     stream: Optional[int]) -> int:
    """Direct C call of kda_backward; returns the status code."""
    return library().kda_backward(q, k, v, log_alpha, beta, cu_seqlens, initial_state, d_out,
                                  d_final_state, dq, dk, dv, dlog_alpha, dbeta, d_initial_state,
                                  int(total_tokens), int(num_seqs), int(num_heads), int(d_k),
                                  int(d_v), int(dtype), int(options), stream)


def backward_workspace_bytes(total_tokens: int, num_seqs: int, num_heads: int, d_k: int,
                             d_v: int) -> int:
    return int(library().kda_backward_workspace_bytes(int(total_tokens), int(num_seqs),
                                                      int(num_heads), int(d_k), int(d_v)))


def backward(q, k, v, log_alpha, beta, cu_seqlens, d_out, d_final_state=None, initial_state=None,
             qk_l2norm: bool = False, with_initial_grad: bool = True,
             stream: Optional[torch.cuda.Stream] = None):
    """Gradients of the scan: returns (dq, dk, dv, dlog_alpha, dbeta, d_initial_state or None).

    Inputs as kda_forward; d_out like out; d_final_state float32 [N, H, d_k, d_v] or None.
    Gradients come back in the data dtype, d_initial_state in float32.
    """
    out_like = torch.empty_like(v)
    T, N, H, dk, dv, dt = _check(q, k, v, log_alpha, beta, cu_seqlens, out_like, d_final_state,
                                 initial_state)
    if d_out.shape != v.shape or d_out.dtype != q.dtype or not d_out.is_cuda or not d_out.is_contiguous():
        raise ValueError("d_out must be a contiguous GPU tensor shaped and typed like out")
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(log_alpha),
         torch.empty_like(beta)]
    dinit = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device) if with_initial_grad else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = kda_backward_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(cu_seqlens),
                          _ptr(initial_state), _ptr(d_out), _ptr(d_final_state), *[_ptr(x) for x in g],
                          _ptr(dinit), T, N, H, dk, dv, dt, KDA_OPT_QK_L2NORM if qk_l2norm else 0,
                          stream.cuda_stream)
    if st != 0:
        raise KdaError(st, library().kda_last_error().decode())
    return (*g, dinit)


def short_conv_raw(x, w_text, w_vis, cu_seqlens, text_len, grid, y, total_tokens: int, num_seqs: int,
                   channels: int, k_text: int, k_t: int, k_h: int, k_w: int, dtype: int,
                   stream: Optional[int]) -> int:
    """Direct C call of kda_short_conv; returns the status code."""
    return library().kda_short_conv(x, w_text, w_vis, cu_seqlens, text_len, grid, y, int(total_tokens),
                                    int(num_seqs), int(channels), int(k_text), int(k_t), int(k_h),
                                    int(k_w), int(dtype), stream)


def _conv_check(x, w_text, w_vis, cu_seqlens, text_len, grid, outs):
    """Shapes, dtypes and devices of a short-convolution call; returns (T, C, N, dtype code)."""
    if x.dim() != 2 or w_text.dim() != 2 or w_vis.dim() != 4:
        raise ValueError("x must be [T, C], w_text [k, C], w_vis [kt, kh, kw, C]")
    T, C = x.shape
    if w_text.shape[1] != C or w_vis.shape[3] != C:
        raise ValueError("weights must have the channels of x last")
    for name, t, dt in (("w_text", w_text, torch.float32), ("w_vis", w_vis, torch.float32),
                        ("cu_seqlens", cu_seqlens, torch.int32), ("text_len", text_len, torch.int32),
                        ("grid", grid, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} GPU tensor")
    N = cu_seqlens.numel() - 1
    if text_len.numel() != N or grid.numel() != 3 * N:
        raise ValueError("text_len must be [N] and grid [N, 3]")
    if x.dtype == torch.bfloat16:
        dt = KDA_BF16
    elif x.dtype == torch.float32:
        dt = KDA_F32
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    for name, t, like, like_name in outs:
        if t.dtype != like.dtype or t.shape != like.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor of the shape and dtype of {like_name}")
    for name, t in (("w_text", w_text), ("w_vis", w_vis), ("cu_seqlens", cu_seqlens), ("text_len", text_len),
                    ("grid", grid), *((o[0], o[1]) for o in outs)):
        if t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")
    return T, C, N, dt


def short_conv(x, w_text, w_vis, cu_seqlens, text_len, grid, y=None,
               stream: Optional[torch.cuda.Stream] = None):
    """The modality-aware short convolution: x [T, C] (float32 or bfloat16); w_text [k, C] and
    w_vis [kt, kh, kw, C] float32; cu_seqlens [N+1], text_len [N], grid [N, 3] int32. Returns y."""
    if y is None and x.dim() == 2 and x.is_cuda:
        y = torch.empty_like(x)
    T, C, N, dt = _conv_check(x, w_text, w_vis, cu_seqlens, text_len, grid, [("y", y, x, "x")] if y is not None else [])
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = short_conv_raw(_ptr(x), _ptr(w_text), _ptr(w_vis), _ptr(cu_seqlens), _ptr(text_len), _ptr(grid),
                        _ptr(y), T, N, C, w_text.shape[0], w_vis.shape[0], w_vis.shape[1], w_vis.shape[2],
                        dt, stream.cuda_stream)
    if st != 0:
        raise KdaError(st, library().kda_last_error().decode())
    return y


def short_conv_backward_raw(x, w_text, w_vis, cu_seqlens, text_len, grid, dy, dx, dw_text, dw_vis,
                            total_tokens: int, num_seqs: int, channels: int, k_text: int, k_t: int, k_h: int,
                            k_w: int, dtype: int, stream: Optional[int]) -> int:
    """Direct C call of kda_short_conv_backward; returns the status code."""
    return library().kda_short_conv_backward(x, w_text, w_vis, cu_seqlens, text_len, grid, dy, dx, dw_text,
                                             dw_vis, int(total_tokens), int(num_seqs), int(channels), int(k_text),
                                             int(k_t), int(k_h), int(k_w), int(dtype), stream)


def short_conv_backward(x, w_text, w_vis, cu_seqlens, text_len, grid, dy, dx=None, dw_text=None, dw_vis=None,
                        stream: Optional[torch.cuda.Stream] = None):
    """Reverse mode of short_conv: dy [T, C] of the dtype of x. Returns (dx, dw_text, dw_vis), dx of the
    dtype of x and the weight gradients float32 of the weights' shapes."""
    if x.dim() == 2 and x.is_cuda:
        dx = torch.empty_like(x) if dx is None else dx
        dw_text = torch.empty_like(w_text) if dw_text is None else dw_text
        dw_vis = torch.empty_like(w_vis) if dw_vis is None else dw_vis
    outs = [("dy", dy, x, "x"), ("dx", dx, x, "x"), ("dw_text", dw_text, w_text, "w_text"),
            ("dw_vis", dw_vis, w_vis, "w_vis")]
    if any(o[1] is None for o in outs):
        raise ValueError("x must be a [T, C] GPU tensor")
    T, C, N, dt = _conv_check(x, w_text, w_vis, cu_seqlens, text_len, grid, outs)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = short_conv_backward_raw(_ptr(x), _ptr(w_text), _ptr(w_vis), _ptr(cu_seqlens), _ptr(text_len), _ptr(grid),
                                 _ptr(dy), _ptr(dx), _ptr(dw_text), _ptr(dw_vis), T, N, C, w_text.shape[0],
                                 w_vis.shape[0], w_vis.shape[1], w_vis.shape[2], dt, stream.cuda_stream)
    if st != 0:
        raise KdaError(st, library().kda_last_error().decode())
    return dx, dw_text, dw_vis
