"""MI355X-native exact attention: Python binding of the C-ABI library libfa.so.

The binding only marshals arguments.  Every step of the attention forward and
backward runs in the HIP kernels of ``libfa.so`` (built from ``csrc/`` for
gfx950); PyTorch supplies device memory and the current stream.  If the
library is missing, every call raises -- there is no fallback path.

Raw entry points, same names and argument order as ``include/fa.h``:
    fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, stream) -> int
    fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, n_splits,
                   workspace, workspace_bytes, stream) -> int
    fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, dtype, n_splits) -> int
    fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, causal,
           dtype, deterministic, workspace, workspace_bytes, stream) -> int
    fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype, deterministic) -> int
    fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, dtype,
                   stream) -> int
    fa_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, d, scale, window_left, window_right,
                  dtype, stream) -> int
    fa_bwd_window(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, window_left,
                  window_right, dtype, deterministic, workspace, workspace_bytes, stream) -> int
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, d, scale, window_left, window_right, dtype,
                  stream) -> int
    fa_bwd_varlen(q, k, v, o, lse, dO, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, H,
                  total_q, total_k, max_seqlen_q, max_seqlen_k, d, scale, window_left,
                  window_right, dtype, deterministic, workspace, workspace_bytes, stream) -> int
    fa_bwd_varlen_workspace_bytes(H, total_q, d, dtype, deterministic) -> int
    fa_strerror(status) -> str
(pointer arguments are integers: device addresses, 0 for NULL)

Tensor helpers that allocate the outputs with torch and raise ``FAError`` on a
non-zero status:
    attention_forward(q, k, v, scale=None, causal=False, window=None) -> (o, lse)
    attention_forward_splitkv(q, k, v, scale=None, causal=False, n_splits=0) -> (o, lse)
    attention_backward(q, k, v, o, lse, do, scale=None, causal=False, window=None,
                       deterministic=True) -> (dq, dk, dv)
    attention_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                             max_seqlen_k, scale=None, causal=False, window=None) -> (o, lse)
    attention_backward_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                              max_seqlen_k, scale=None, causal=False, window=None,
                              deterministic=True) -> (dq, dk, dv)
``window`` is a local window (wl, wr): key j is visible to query i iff
i + (Nk - Nq) - wl <= j <= i + (Nk - Nq) + wr, a side None for no bound; it
replaces ``causal`` (giving both raises ValueError).  The varlen helpers take
head-major packed tensors q, o [H, total_q, d], k, v [H, total_k, d] and int32
device offsets cu_seqlens [B+1]; every sequence attends within itself.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FA_F32", "FA_BF16", "FAError", "library_path", "load_library",
    "fa_fwd", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes", "fa_bwd",
    "fa_bwd_workspace_bytes", "fa_bwd_noalloc", "fa_fwd_window", "fa_bwd_window", "fa_fwd_varlen",
    "fa_bwd_varlen", "fa_bwd_varlen_workspace_bytes", "fa_strerror",
    "attention_forward_varlen", "attention_backward_varlen",
    "attention_forward", "attention_forward_splitkv", "attention_backward",
]

FA_F32 = 0
FA_BF16 = 1

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where} failed with status {status}: {fa_strerror(status)}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, "libfa.so")


def load_library() -> ctypes.CDLL:
    """Load libfa.so from the package directory (built in-tree); raise if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_attention_20_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_soft_exp2.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_fwd_soft_exp2.restype = i
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.fa_fwd_splitkv_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_fwd_window.restype = i
    lib.fa_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i,
                                  i, vp, sz, vp]
    lib.fa_bwd_window.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                  f, i, i, i, i, vp, sz, vp]
    lib.fa_bwd_varlen.restype = i
    lib.fa_bwd_varlen_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd_varlen_workspace_bytes.restype = sz
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _p(x):
    return None if not x else ctypes.c_void_p(int(x))


def fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, stream) -> int:
    return load_library().fa_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Nq, Nk, d,
                                 float(scale), int(causal), int(dtype), _p(stream))


def fa_fwd_soft_exp2(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, period, stream) -> int:
    return load_library().fa_fwd_soft_exp2(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Nq, Nk, d,
                                           float(scale), int(causal), int(dtype), int(period), _p(stream))


def fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, n_splits,
                   workspace, workspace_bytes, stream) -> int:
    return load_library().fa_fwd_splitkv(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Nq, Nk, d,
                                         float(scale), int(causal), int(dtype), int(n_splits),
                                         _p(workspace), int(workspace_bytes), _p(stream))


def fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, dtype, n_splits) -> int:
    return int(load_library().fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, dtype, n_splits))


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, dtype,
           deterministic, workspace, workspace_bytes, stream) -> int:
    return load_library().fa_bwd(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq), _p(dk),
                                 _p(dv), B, H, Nq, Nk, d, float(scale), int(causal), int(dtype),
                                 int(deterministic), _p(workspace), int(workspace_bytes),
                                 _p(stream))


def fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, dtype,
                   stream) -> int:
    return load_library().fa_bwd_noalloc(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq),
                                         _p(dk), _p(dv), B, H, Nq, Nk, d, float(scale), int(causal),
                                         int(dtype), _p(stream))


def fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype, deterministic) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, Nq, Nk, d, dtype, int(deterministic)))


def fa_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, d, scale, window_left, window_right, dtype,
                  stream) -> int:
    return load_library().fa_fwd_window(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Nq, Nk, d,
                                        float(scale), int(window_left), int(window_right),
                                        int(dtype), _p(stream))


def fa_bwd_window(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, scale, window_left,
                  window_right, dtype, deterministic, workspace, workspace_bytes, stream) -> int:
    return load_library().fa_bwd_window(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq),
                                        _p(dk), _p(dv), B, H, Nq, Nk, d, float(scale),
                                        int(window_left), int(window_right), int(dtype),
                                        int(deterministic), _p(workspace), int(workspace_bytes),
                                        _p(stream))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, d, scale, window_left, window_right, dtype,
                  stream) -> int:
    return load_library().fa_fwd_varlen(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(cu_seqlens_q),
                                        _p(cu_seqlens_k), B, H, total_q, total_k, max_seqlen_q,
                                        max_seqlen_k, d, float(scale), int(window_left),
                                        int(window_right), int(dtype), _p(stream))


def fa_bwd_varlen(q, k, v, o, lse, dO, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, H, total_q,
                  total_k, max_seqlen_q, max_seqlen_k, d, scale, window_left, window_right,
                  dtype, deterministic, workspace, workspace_bytes, stream) -> int:
    return load_library().fa_bwd_varlen(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq),
                                        _p(dk), _p(dv), _p(cu_seqlens_q), _p(cu_seqlens_k), B, H,
                                        total_q, total_k, max_seqlen_q, max_seqlen_k, d,
                                        float(scale), int(window_left), int(window_right),
                                        int(dtype), int(deterministic), _p(workspace),
                                        int(workspace_bytes), _p(stream))


def fa_bwd_varlen_workspace_bytes(H, total_q, d, dtype, deterministic) -> int:
    return int(load_library().fa_bwd_varlen_workspace_bytes(H, total_q, d, dtype,
                                                             int(deterministic)))


def fa_strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


# ---------------------------------------------------------------------------
# torch tensor helpers (memory and stream plumbing only)
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _check(t, name, shape, dtype, dev):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev} (the device of q)")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(dev):
    """The current stream of q's device; calls run under a guard that makes
    that device current, so the launch and the pointers agree."""
    import torch
    return torch.cuda.current_stream(dev).cuda_stream


def _ws_args(workspace, dev):
    """(pointer, size in bytes) of an optional caller-given workspace."""
    if workspace is None:
        return 0, 0
    if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _window_args(causal, window):
    """(window_left, window_right) of the C ABI (-1 = unbounded), or None
    when the call takes the causal flag."""
    if window is None:
        return None
    if causal:
        raise ValueError("give either causal or a window, not both")
    wl, wr = window
    return (-1 if wl is None else int(wl), -1 if wr is None else int(wr))


def attention_forward(q, k, v, scale=None, causal=False, out=None, lse=None, want_lse=True,
                      window=None, soft_exp2=0):
    """O = softmax(scale * q k^T) v and the natural-log LSE, via fa_fwd (or
    fa_fwd_window when a local ``window`` is given, or fa_fwd_soft_exp2 when
    ``soft_exp2`` is 2, 4 or 8: one exponential in that many by a polynomial
    on the FMA pipe; bf16, no window).

    q [B,H,Nq,d], k and v [B,H,Nk,d]; bf16 or fp32; contiguous; on the GPU.
    Returns (o, lse); lse is None when want_lse is False and none is given.
    """
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dt = q.dtype
    _check(q, "q", (B, H, Nq, d), dt, q.device)
    _check(k, "k", (B, H, Nk, d), dt, q.device)
    _check(v, "v", (B, H, Nk, d), dt, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", (B, H, Nq, d), dt, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", (B, H, Nq), torch.float32, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    w = _window_args(causal, window)
    lse_p = lse.data_ptr() if lse is not None else 0
    if soft_exp2 and w is not None:
        raise ValueError("soft_exp2 takes the causal or unmasked forward, not a window")
    name = "fa_fwd_window" if w is not None else "fa_fwd_soft_exp2" if soft_exp2 else "fa_fwd"
    with torch.cuda.device(q.device):
        if w is not None:
            st = fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_p,
                               B, H, Nq, Nk, d, scale, w[0], w[1], _dtype_code(q), _stream(q.device))
        elif soft_exp2:
            st = fa_fwd_soft_exp2(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_p,
                                  B, H, Nq, Nk, d, scale, causal, _dtype_code(q), soft_exp2,
                                  _stream(q.device))
        else:
            st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_p,
                        B, H, Nq, Nk, d, scale, causal, _dtype_code(q), _stream(q.device))
    if st != 0:
        raise FAError(st, name)
    return out, lse


def attention_forward_splitkv(q, k, v, scale=None, causal=False, n_splits=0, workspace=None):
    """attention_forward through fa_fwd_splitkv (bf16 only): the key range of
    each query tile is split over several workgroups whose partial results are
    merged by their LSE.  n_splits = 0 lets the library choose."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dt = q.dtype
    _check(q, "q", (B, H, Nq, d), dt, q.device)
    _check(k, "k", (B, H, Nk, d), dt, q.device)
    _check(v, "v", (B, H, Nk, d), dt, q.device)
    code = _dtype_code(q)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    need = fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, code, n_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    with torch.cuda.device(q.device):
        st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, Nq, Nk, d, scale, causal, code, n_splits,
                            *_ws_args(workspace, q.device), _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_fwd_splitkv")
    return out, lse


def attention_backward(q, k, v, o, lse, do, scale=None, causal=False, workspace=None,
                       window=None, deterministic=True):
    """dq, dk, dv of sum(do * o) via fa_bwd, or fa_bwd_window (bf16 or fp32).
    ``o`` and ``lse`` are the outputs of ``attention_forward`` for the same
    inputs and mask.  ``deterministic`` (the default, and the faster mode on
    MI355X) runs the bitwise-repeatable kernels; False runs the single
    key-side kernel that sums dQ with fp32 atomics (bf16 only: fp32 inputs
    always take the deterministic kernels)."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dt = q.dtype
    for t, n, s in ((q, "q", (B, H, Nq, d)), (k, "k", (B, H, Nk, d)), (v, "v", (B, H, Nk, d)),
                    (o, "o", (B, H, Nq, d)), (do, "do", (B, H, Nq, d))):
        _check(t, n, s, dt, q.device)
    _check(lse, "lse", (B, H, Nq), torch.float32, q.device)
    code = _dtype_code(q)
    need = fa_bwd_workspace_bytes(B, H, Nq, Nk, d, code, deterministic)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    w = _window_args(causal, window)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    ws = _ws_args(workspace, q.device)
    with torch.cuda.device(q.device):
        if w is None:
            st = fa_bwd(*ptrs, B, H, Nq, Nk, d, scale, causal, code, deterministic, *ws,
                        _stream(q.device))
        else:
            st = fa_bwd_window(*ptrs, B, H, Nq, Nk, d, scale, w[0], w[1], code, deterministic, *ws,
                               _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_bwd" if w is None else "fa_bwd_window")
    return dq, dk, dv


def _mask_args(causal, window):
    """(window_left, window_right) of the C ABI for a causal flag or a window."""
    w = _window_args(causal, window)
    if w is not None:
        return w
    return (-1, 0) if causal else (-1, -1)


def _check_cu(cu, name, B, dev):
    import torch
    if not cu.is_cuda or cu.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() != B + 1 or not cu.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of B + 1 = {B + 1} offsets")


def attention_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                             scale=None, causal=False, window=None, out=None, lse=None):
    """Attention over a packed variable-length batch via fa_fwd_varlen (bf16).

    q [H, total_q, d], k and v [H, total_k, d] (head-major packing); sequence b
    owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and the matching
    key rows; every length must be at most max_seqlen_q / max_seqlen_k.
    Returns (o [H, total_q, d], lse [H, total_q]); rows outside every
    sequence are left as they were in ``out`` / ``lse`` (uninitialised when
    those are not given).
    """
    import torch
    H, Tq, d = q.shape
    Tk = k.shape[1]
    B = cu_seqlens_q.numel() - 1
    _check(q, "q", (H, Tq, d), q.dtype, q.device)
    _check(k, "k", (H, Tk, d), q.dtype, q.device)
    _check(v, "v", (H, Tk, d), q.dtype, q.device)
    _check_cu(cu_seqlens_q, "cu_seqlens_q", B, q.device)
    _check_cu(cu_seqlens_k, "cu_seqlens_k", B, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", (H, Tq, d), q.dtype, q.device)
    if lse is None:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    _check(lse, "lse", (H, Tq), torch.float32, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    wl, wr = _mask_args(causal, window)
    with torch.cuda.device(q.device):
        st = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, Tq, Tk,
                           int(max_seqlen_q), int(max_seqlen_k), d, scale, wl, wr, _dtype_code(q),
                           _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_fwd_varlen")
    return out, lse


def attention_backward_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                              max_seqlen_k, scale=None, causal=False, window=None,
                              workspace=None, deterministic=True):
    """dq, dk, dv of sum(do * o) for ``attention_forward_varlen`` via
    fa_bwd_varlen (bf16); the same packing, offsets and mask as the forward.
    ``deterministic`` as in ``attention_backward``."""
    import torch
    H, Tq, d = q.shape
    Tk = k.shape[1]
    B = cu_seqlens_q.numel() - 1
    for t, n, s in ((q, "q", (H, Tq, d)), (k, "k", (H, Tk, d)), (v, "v", (H, Tk, d)),
                    (o, "o", (H, Tq, d)), (do, "do", (H, Tq, d))):
        _check(t, n, s, q.dtype, q.device)
    _check(lse, "lse", (H, Tq), torch.float32, q.device)
    _check_cu(cu_seqlens_q, "cu_seqlens_q", B, q.device)
    _check_cu(cu_seqlens_k, "cu_seqlens_k", B, q.device)
    code = _dtype_code(q)
    need = fa_bwd_varlen_workspace_bytes(H, Tq, d, code, deterministic)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    wl, wr = _mask_args(causal, window)
    with torch.cuda.device(q.device):
        st = fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, Tq, Tk,
                           int(max_seqlen_q), int(max_seqlen_k), d, scale, wl, wr, code,
                           deterministic, *_ws_args(workspace, q.device), _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_bwd_varlen")
    return dq, dk, dv
