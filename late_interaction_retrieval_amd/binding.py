"""Thin ctypes binding over libmaxsim.so, with the C entry points' names.

Only argument marshalling happens here: tensors become device pointers, the
current torch stream becomes the hipStream_t, and a non-zero status becomes a
``MaxSimError``.  Every step of the computation runs in the HIP kernels; there
is no CPU fallback: if the library was not built, importing this module raises.
PyTorch is used for device memory (outputs the caller does not pass are
allocated with torch) and streams.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmaxsim.so")

MAXSIM_OK = 0
MAXSIM_ERR_NULL = 1
MAXSIM_ERR_SHAPE = 2
MAXSIM_ERR_UNSUPPORTED = 3
MAXSIM_ERR_ALIGN = 4
MAXSIM_ERR_WORKSPACE = 5
MAXSIM_ERR_HIP = 6
MAXSIM_ERR_SCRATCH = 7
MAXSIM_F16 = 0
MAXSIM_BF16 = 1

# name -> (restype, argtypes); must match include/maxsim.h
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
SIGNATURES = {
    "maxsim_fwd": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "maxsim_fwd_varlen": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _P, _P, _P]),
    "maxsim_fwd_i8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _P, _P, _P]),
    "maxsim_bwd_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32]),
    "maxsim_bwd": (ctypes.c_int, [_P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]),
    "maxsim_bwd_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "maxsim_bwd_noalloc": (ctypes.c_int, [_P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "maxsim_bwd_varlen_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32]),
    "maxsim_bwd_varlen": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _P, _P,
                                         _P, _P, _P, ctypes.c_size_t, _P]),
    "maxsim_bwd_scatter_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "maxsim_bwd_scatter": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I64, _I32, _P, _P,
                                          _P, ctypes.c_size_t, _P]),
    "maxsim_bwd_prefer_scatter": (ctypes.c_int, [_I32, _I32, _I32, _I64]),
    "maxsim_fwd_host_stream_staging_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32]),
    "maxsim_fwd_host_stream": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P,
                                              ctypes.c_size_t, _P, _P, _P]),
    "maxsim_chamfer_fwd_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "maxsim_chamfer_fwd": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "maxsim_chamfer_bwd_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "maxsim_chamfer_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "maxsim_fwd_pairs": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I64, _I32, _P, _P, _P]),
    "maxsim_topk": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P, _P]),
    "maxsim_two_stage_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "maxsim_two_stage_topk": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I64, _I32, _I32,
                                             _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "maxsim_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


class MaxSimError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().maxsim_status_string(status).decode()
        super().__init__("%s: %s (status %d)" % (where, msg, status))


_lib = None


def lib():
    """The loaded libmaxsim.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmaxsim.so is not built; run `python -m late_interaction_retrieval_amd.build` "
                              "(or __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


lib()  # fail loudly at import time if the native library is missing


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != MAXSIM_OK:
        raise MaxSimError(status, where)


def _dtype_code(t):
    if t.dtype == torch.float16:
        return MAXSIM_F16
    if t.dtype == torch.bfloat16:
        return MAXSIM_BF16
    raise TypeError("Q and D must be float16 or bfloat16, got %s" % t.dtype)


def _need(t, name, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def maxsim_fwd(Q, D, d_lens=None, scores=None, argmax=None, with_argmax=True, stream=None):
    """Padded forward.  Q [Nq, Lq, 128], D [B, Ld, 128] (fp16/bf16), d_lens [B] int32 or None.

    Returns (scores [Nq, B] fp32, argmax [Nq, B, Lq] int32 or None).
    """
    Nq, Lq, d = Q.shape
    B, Ld, d2 = D.shape
    if d2 != d or Q.dtype != D.dtype:
        raise ValueError("Q and D must share dtype and width")
    _need(Q, "Q")
    _need(D, "D", device=Q.device)
    if d_lens is not None:
        _need(d_lens, "d_lens", torch.int32, Q.device)
    if scores is None:
        scores = torch.empty((Nq, B), dtype=torch.float32, device=Q.device)
    _need(scores, "scores", torch.float32, Q.device)
    if argmax is None and with_argmax:
        argmax = torch.empty((Nq, B, Lq), dtype=torch.int32, device=Q.device)
    if argmax is not None:
        _need(argmax, "argmax", torch.int32, Q.device)
    st = lib().maxsim_fwd(_ptr(Q), _ptr(D), _ptr(d_lens), Nq, Lq, B, Ld, d, _dtype_code(Q),
                          _ptr(scores), _ptr(argmax), _stream(Q, stream))
    _check(st, "maxsim_fwd")
    return scores, argmax


def maxsim_fwd_varlen(Q, D_packed, cu_seqlens, max_Ld, scores=None, argmax=None, with_argmax=True,
                      stream=None):
    """Padding-free forward.  D_packed [T, 128], cu_seqlens [B+1] int32 on the device."""
    Nq, Lq, d = Q.shape
    T, d2 = D_packed.shape
    B = cu_seqlens.shape[0] - 1
    if d2 != d or Q.dtype != D_packed.dtype:
        raise ValueError("Q and D_packed must share dtype and width")
    _need(Q, "Q")
    _need(D_packed, "D_packed", device=Q.device)
    _need(cu_seqlens, "cu_seqlens", torch.int32, Q.device)
    if scores is None:
        scores = torch.empty((Nq, B), dtype=torch.float32, device=Q.device)
    _need(scores, "scores", torch.float32, Q.device)
    if argmax is None and with_argmax:
        argmax = torch.empty((Nq, B, Lq), dtype=torch.int32, device=Q.device)
    if argmax is not None:
        _need(argmax, "argmax", torch.int32, Q.device)
    st = lib().maxsim_fwd_varlen(_ptr(Q), _ptr(D_packed), _ptr(cu_seqlens), Nq, Lq, B, T, int(max_Ld), d,
                                 _dtype_code(Q), _ptr(scores), _ptr(argmax), _stream(Q, stream))
    _check(st, "maxsim_fwd_varlen")
    return scores, argmax


def maxsim_fwd_i8(Q, q_scale, D_packed, d_scale, cu_seqlens, max_Ld, scores=None, argmax=None,
                  with_argmax=True, stream=None):
    """INT8 x INT8 padding-free forward (int8 rows, fp32 per-token scales)."""
    Nq, Lq, d = Q.shape
    T, d2 = D_packed.shape
    B = cu_seqlens.shape[0] - 1
    if d2 != d:
        raise ValueError("Q and D_packed must share the width")
    _need(Q, "Q", torch.int8)
    _need(D_packed, "D_packed", torch.int8, Q.device)
    _need(q_scale, "q_scale", torch.float32, Q.device)
    _need(d_scale, "d_scale", torch.float32, Q.device)
    _need(cu_seqlens, "cu_seqlens", torch.int32, Q.device)
    if scores is None:
        scores = torch.empty((Nq, B), dtype=torch.float32, device=Q.device)
    _need(scores, "scores", torch.float32, Q.device)
    if argmax is None and with_argmax:
        argmax = torch.empty((Nq, B, Lq), dtype=torch.int32, device=Q.device)
    if argmax is not None:
        _need(argmax, "argmax", torch.int32, Q.device)
    st = lib().maxsim_fwd_i8(_ptr(Q), _ptr(q_scale), _ptr(D_packed), _ptr(d_scale), _ptr(cu_seqlens), Nq, Lq,
                             B, T, int(max_Ld), d, _ptr(scores), _ptr(argmax), _stream(Q, stream))
    _check(st, "maxsim_fwd_i8")
    return scores, argmax


def maxsim_bwd_workspace_bytes(Nq, B, Lq, Ld):
    return int(lib().maxsim_bwd_workspace_bytes(Nq, B, Lq, Ld))


def maxsim_bwd(Q, D, argmax, grad_scores, dQ=None, dD=None, row_ptr=None, col_idx=None, workspace=None,
               stream=None):
    """Backward over padded documents.  Returns (dQ, dD, row_ptr, col_idx)."""
    Nq, Lq, d = Q.shape
    B, Ld, _ = D.shape
    dev = Q.device
    _need(Q, "Q")
    _need(D, "D", device=dev)
    _need(argmax, "argmax", torch.int32, dev)
    _need(grad_scores, "grad_scores", torch.float32, dev)
    if dQ is None:
        dQ = torch.empty((Nq, Lq, d), dtype=torch.float32, device=dev)
    if dD is None:
        dD = torch.empty((B, Ld, d), dtype=torch.float32, device=dev)
    if row_ptr is None:
        row_ptr = torch.empty(B * Ld + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(Nq * B * Lq, dtype=torch.int32, device=dev)
    nbytes = maxsim_bwd_workspace_bytes(Nq, B, Lq, Ld)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    for t, n in ((dQ, "dQ"), (dD, "dD"), (row_ptr, "row_ptr"), (col_idx, "col_idx"), (workspace, "workspace")):
        _need(t, n, device=dev)
    st = lib().maxsim_bwd(_ptr(Q), _ptr(D), _dtype_code(Q), _ptr(argmax), _ptr(grad_scores), Nq, Lq, B, Ld, d,
                          _ptr(dQ), _ptr(dD), _ptr(row_ptr), _ptr(col_idx), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(Q, stream))
    _check(st, "maxsim_bwd")
    return dQ, dD, row_ptr, col_idx


def maxsim_bwd_noalloc(Q, D, argmax, grad_scores, dQ, dD, row_ptr, col_idx, stream=None):
    """maxsim_bwd without a workspace and without allocating: the library's own
    per-device scratch array serves as the workspace, and every output is the
    caller's.  Returns (dQ, dD, row_ptr, col_idx)."""
    Nq, Lq, d = Q.shape
    B, Ld, _ = D.shape
    dev = Q.device
    _need(Q, "Q")
    _need(D, "D", device=dev)
    _need(argmax, "argmax", torch.int32, dev)
    _need(grad_scores, "grad_scores", torch.float32, dev)
    for t, n, dt, numel in ((dQ, "dQ", torch.float32, Nq * Lq * d), (dD, "dD", torch.float32, B * Ld * d),
                            (row_ptr, "row_ptr", torch.int32, B * Ld + 1),
                            (col_idx, "col_idx", torch.int32, Nq * B * Lq)):
        _need(t, n, dt, dev)
        if t.numel() < numel:
            raise ValueError("%s holds %d elements, needs %d" % (n, t.numel(), numel))
    st = lib().maxsim_bwd_noalloc(_ptr(Q), _ptr(D), _dtype_code(Q), _ptr(argmax), _ptr(grad_scores), Nq, Lq, B, Ld,
                                  d, _ptr(dQ), _ptr(dD), _ptr(row_ptr), _ptr(col_idx), _stream(Q, stream))
    _check(st, "maxsim_bwd_noalloc")
    return dQ, dD, row_ptr, col_idx


def maxsim_bwd_varlen_workspace_bytes(Nq, B, Lq, max_Ld):
    return int(lib().maxsim_bwd_varlen_workspace_bytes(Nq, B, Lq, max_Ld))


def maxsim_bwd_varlen(Q, D_packed, cu_seqlens, max_Ld, argmax, grad_scores, dQ=None, dD=None, row_ptr=None,
                      col_idx=None, workspace=None, stream=None):
    """Backward over a packed corpus.  Returns (dQ [Nq, Lq, d], dD [T, d], row_ptr [T+1], col_idx
    [Nq*B*Lq], of which the first row_ptr[T] entries are defined)."""
    Nq, Lq, d = Q.shape
    T, d2 = D_packed.shape
    B = cu_seqlens.shape[0] - 1
    if d2 != d or Q.dtype != D_packed.dtype:
        raise ValueError("Q and D_packed must share dtype and width")
    dev = Q.device
    _need(Q, "Q")
    _need(D_packed, "D_packed", device=dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(argmax, "argmax", torch.int32, dev)
    _need(grad_scores, "grad_scores", torch.float32, dev)
    if dQ is None:
        dQ = torch.empty((Nq, Lq, d), dtype=torch.float32, device=dev)
    if dD is None:
        dD = torch.empty((T, d), dtype=torch.float32, device=dev)
    if row_ptr is None:
        row_ptr = torch.empty(T + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(Nq * B * Lq, dtype=torch.int32, device=dev)
    nbytes = maxsim_bwd_varlen_workspace_bytes(Nq, B, Lq, int(max_Ld))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    for t, n in ((dQ, "dQ"), (dD, "dD"), (row_ptr, "row_ptr"), (col_idx, "col_idx"), (workspace, "workspace")):
        _need(t, n, device=dev)
    st = lib().maxsim_bwd_varlen(_ptr(Q), _ptr(D_packed), _ptr(cu_seqlens), _dtype_code(Q), _ptr(argmax),
                                 _ptr(grad_scores), Nq, Lq, B, T, int(max_Ld), d, _ptr(dQ), _ptr(dD), _ptr(row_ptr),
                                 _ptr(col_idx), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(Q, stream))
    _check(st, "maxsim_bwd_varlen")
    return dQ, dD, row_ptr, col_idx


def maxsim_bwd_prefer_scatter(Nq, Lq, B, rows):
    return bool(lib().maxsim_bwd_prefer_scatter(Nq, Lq, B, rows))


def maxsim_bwd_scatter_workspace_bytes(Nq, B, Lq):
    return int(lib().maxsim_bwd_scatter_workspace_bytes(Nq, B, Lq))


def maxsim_bwd_scatter(Q, D, argmax, grad_scores, cu_seqlens=None, max_Ld=None, dQ=None, dD=None, workspace=None,
                       stream=None):
    """Backward with dD by atomic scatter (no CSR).  D is [B, Ld, d] (padded) or, with cu_seqlens,
    D_packed [T, d] with max_Ld the longest document.  Returns (dQ, dD)."""
    Nq, Lq, d = Q.shape
    dev = Q.device
    _need(Q, "Q")
    _need(D, "D", device=dev)
    _need(argmax, "argmax", torch.int32, dev)
    _need(grad_scores, "grad_scores", torch.float32, dev)
    if D.dtype != Q.dtype or D.shape[-1] != d:
        raise ValueError("Q and D must share dtype and width")
    if cu_seqlens is None:
        B, Ld, _ = D.shape
        T = 0
    else:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        B = cu_seqlens.shape[0] - 1
        T = D.shape[0]
        Ld = int(max_Ld)
    if dQ is None:
        dQ = torch.empty((Nq, Lq, d), dtype=torch.float32, device=dev)
    if dD is None:
        dD = torch.empty(D.shape, dtype=torch.float32, device=dev)
    _need(dQ, "dQ", torch.float32, dev)
    _need(dD, "dD", torch.float32, dev)
    if workspace is None:
        workspace = torch.empty(max(256, maxsim_bwd_scatter_workspace_bytes(Nq, B, Lq)), dtype=torch.uint8,
                                device=dev)
    _need(workspace, "workspace", device=dev)
    st = lib().maxsim_bwd_scatter(_ptr(Q), _ptr(D), _ptr(cu_seqlens), _dtype_code(Q), _ptr(argmax),
                                  _ptr(grad_scores), Nq, Lq, B, Ld, T, d, _ptr(dQ), _ptr(dD), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(Q, stream))
    _check(st, "maxsim_bwd_scatter")
    return dQ, dD


class MaxSimFunction(torch.autograd.Function):
    """score = MaxSim(Q, D) as an autograd op: the forward saves the argmax and the
    backward builds the inverse-grid CSR and the gradients (paper Section 4.2).
    With deterministic=False the backward may take the atomic-scatter dD instead,
    where the dispatch rule (maxsim_bwd_prefer_scatter) expects it to be faster."""

    @staticmethod
    def forward(ctx, Q, D, cu_seqlens, max_Ld, deterministic):
        if cu_seqlens is None:
            scores, argmax = maxsim_fwd(Q, D)
        else:
            scores, argmax = maxsim_fwd_varlen(Q, D, cu_seqlens, max_Ld)
        ctx.save_for_backward(Q, D, argmax, cu_seqlens)
        ctx.max_Ld = max_Ld
        ctx.deterministic = deterministic
        return scores

    @staticmethod
    def backward(ctx, grad_scores):
        Q, D, argmax, cu = ctx.saved_tensors
        g = grad_scores.float().contiguous()
        Nq, Lq, _ = Q.shape
        B = argmax.shape[1]
        rows = D.shape[0] * D.shape[1] if cu is None else D.shape[0]
        if not ctx.deterministic and maxsim_bwd_prefer_scatter(Nq, Lq, B, rows):
            dQ, dD = maxsim_bwd_scatter(Q, D, argmax, g, cu_seqlens=cu, max_Ld=ctx.max_Ld)
        elif cu is None:
            dQ, dD, _, _ = maxsim_bwd(Q, D, argmax, g)
        else:
            dQ, dD, _, _ = maxsim_bwd_varlen(Q, D, cu, ctx.max_Ld, argmax, g)
        return dQ.to(Q.dtype), dD.to(D.dtype), None, None, None


def maxsim(Q, D, cu_seqlens=None, max_Ld=None, deterministic=True):
    """MaxSim scores [Nq, B] of every query against every document, with autograd
    support.  D is [B, Ld, d], or packed [T, d] with cu_seqlens [B+1] and max_Ld."""
    if cu_seqlens is not None and max_Ld is None:
        raise ValueError("max_Ld is required with cu_seqlens")
    return MaxSimFunction.apply(Q, D, cu_seqlens, max_Ld, deterministic)


def maxsim_fwd_host_stream_staging_bytes(Nq, Lq, Ld, block_docs, with_argmax):
    return int(lib().maxsim_fwd_host_stream_staging_bytes(Nq, Lq, Ld, block_docs, int(bool(with_argmax))))


def maxsim_fwd_host_stream(Q, D_host, block_docs, cu_seqlens_host=None, cu_seqlens=None, max_Ld=None, d_lens=None,
                           scores=None, argmax=None, with_argmax=False, staging=None, stream=None):
    """Score a corpus held in host memory (a CPU tensor, pinned for full speed) block by block.
    Padded: D_host [B, Ld, 128].  Packed: D_host [T, 128], cu_seqlens_host (CPU int32 [B+1]),
    cu_seqlens (the same on the device) and max_Ld.  Returns (scores [Nq, B], argmax or None).
    The copies run after this returns: keep D_host alive until the stream has finished."""
    Nq, Lq, d = Q.shape
    dev = Q.device
    _need(Q, "Q")
    if D_host.is_cuda or not D_host.is_contiguous():
        raise ValueError("D_host must be a contiguous host tensor")
    if D_host.dtype != Q.dtype or D_host.shape[-1] != d:
        raise ValueError("Q and D_host must share dtype and width")
    if cu_seqlens_host is None:
        B, Ld, _ = D_host.shape
    else:
        if cu_seqlens_host.is_cuda or cu_seqlens_host.dtype != torch.int32 or not cu_seqlens_host.is_contiguous():
            raise ValueError("cu_seqlens_host must be a contiguous host int32 tensor")
        if cu_seqlens is None or max_Ld is None:
            raise ValueError("a packed corpus needs cu_seqlens on the device and max_Ld")
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        B = cu_seqlens_host.shape[0] - 1
        Ld = int(max_Ld)
    if d_lens is not None:
        _need(d_lens, "d_lens", torch.int32, dev)
    if scores is None:
        scores = torch.empty((Nq, B), dtype=torch.float32, device=dev)
    _need(scores, "scores", torch.float32, dev)
    if argmax is None and with_argmax:
        argmax = torch.empty((Nq, B, Lq), dtype=torch.int32, device=dev)
    if argmax is not None:
        _need(argmax, "argmax", torch.int32, dev)
    nbytes = maxsim_fwd_host_stream_staging_bytes(Nq, Lq, Ld, block_docs, argmax is not None)
    if staging is None:
        staging = torch.empty(max(256, nbytes), dtype=torch.uint8, device=dev)
    _need(staging, "staging", device=dev)
    st = lib().maxsim_fwd_host_stream(_ptr(Q), ctypes.c_void_p(D_host.data_ptr()),
                                      None if cu_seqlens_host is None else ctypes.c_void_p(cu_seqlens_host.data_ptr()),
                                      _ptr(cu_seqlens), _ptr(d_lens), Nq, Lq, B, Ld, d, _dtype_code(Q),
                                      int(block_docs), _ptr(staging), staging.numel(), _ptr(scores), _ptr(argmax),
                                      _stream(Q, stream))
    _check(st, "maxsim_fwd_host_stream")
    return scores, argmax


def _clouds(P, Q):
    if P.dim() == 2:
        P = P.unsqueeze(0)
    if Q.dim() == 2:
        Q = Q.unsqueeze(0)
    _need(P, "P", torch.float32)
    _need(Q, "Q", torch.float32, P.device)
    if P.shape[0] != Q.shape[0] or P.shape[2] != 3 or Q.shape[2] != 3:
        raise ValueError("P [Bt, N, 3] and Q [Bt, M, 3] must share Bt")
    return P, Q


def maxsim_chamfer_fwd(P, Q, workspace=None, stream=None):
    """Nearest neighbours both ways between P [Bt, N, 3] and Q [Bt, M, 3] (fp32):
    (dist_p [Bt, N], idx_p, dist_q [Bt, M], idx_q); squared distances."""
    P, Q = _clouds(P, Q)
    Bt, N, _ = P.shape
    M = Q.shape[1]
    dev = P.device
    dist_p = torch.empty((Bt, N), dtype=torch.float32, device=dev)
    idx_p = torch.empty((Bt, N), dtype=torch.int32, device=dev)
    dist_q = torch.empty((Bt, M), dtype=torch.float32, device=dev)
    idx_q = torch.empty((Bt, M), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(256, int(lib().maxsim_chamfer_fwd_workspace_bytes(Bt, N, M))), dtype=torch.uint8,
                                device=dev)
    st = lib().maxsim_chamfer_fwd(_ptr(P), _ptr(Q), Bt, N, M, _ptr(dist_p), _ptr(idx_p), _ptr(dist_q), _ptr(idx_q),
                                  _ptr(workspace), workspace.numel(), _stream(P, stream))
    _check(st, "maxsim_chamfer_fwd")
    return dist_p, idx_p, dist_q, idx_q


def maxsim_chamfer_bwd(P, Q, idx_p, idx_q, grad_p, grad_q, workspace=None, stream=None):
    """Gradients of sum grad_p*dist_p + sum grad_q*dist_q through the saved selections:
    (dP, dQ, row_ptr_p, col_idx_p, row_ptr_q, col_idx_q)."""
    P, Q = _clouds(P, Q)
    Bt, N, _ = P.shape
    M = Q.shape[1]
    dev = P.device
    for t, n in ((idx_p, "idx_p"), (idx_q, "idx_q")):
        _need(t, n, torch.int32, dev)
    for t, n in ((grad_p, "grad_p"), (grad_q, "grad_q")):
        _need(t, n, torch.float32, dev)
    dP = torch.empty((Bt, N, 3), dtype=torch.float32, device=dev)
    dQ = torch.empty((Bt, M, 3), dtype=torch.float32, device=dev)
    rp_p = torch.empty(Bt * N + 1, dtype=torch.int32, device=dev)
    ci_p = torch.empty(max(1, Bt * M), dtype=torch.int32, device=dev)
    rp_q = torch.empty(Bt * M + 1, dtype=torch.int32, device=dev)
    ci_q = torch.empty(max(1, Bt * N), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(256, int(lib().maxsim_chamfer_bwd_workspace_bytes(Bt, N, M))), dtype=torch.uint8,
                                device=dev)
    st = lib().maxsim_chamfer_bwd(_ptr(P), _ptr(Q), _ptr(idx_p), _ptr(idx_q), _ptr(grad_p), _ptr(grad_q), Bt, N, M,
                                  _ptr(dP), _ptr(dQ), _ptr(rp_p), _ptr(ci_p), _ptr(rp_q), _ptr(ci_q),
                                  _ptr(workspace), workspace.numel(), _stream(P, stream))
    _check(st, "maxsim_chamfer_bwd")
    return dP, dQ, rp_p, ci_p, rp_q, ci_q


class ChamferFunction(torch.autograd.Function):
    """(dist_p, dist_q) with autograd: the forward saves the nearest-neighbour
    indices, the backward inverts them (paper Section 4.2, Chamfer distance)."""

    @staticmethod
    def forward(ctx, P, Q):
        dist_p, idx_p, dist_q, idx_q = maxsim_chamfer_fwd(P, Q)
        ctx.save_for_backward(P, Q, idx_p, idx_q)
        return dist_p, dist_q

    @staticmethod
    def backward(ctx, grad_p, grad_q):
        P, Q, idx_p, idx_q = ctx.saved_tensors
        dP, dQ, _, _, _, _ = maxsim_chamfer_bwd(P, Q, idx_p, idx_q, grad_p.float().contiguous(),
                                                grad_q.float().contiguous())
        return dP.reshape(P.shape), dQ.reshape(Q.shape)


def chamfer_distance(P, Q):
    """The page's Chamfer distance per batch item, mean_p min_q |p-q|^2 +
    mean_q min_p |q-p|^2, for P [Bt, N, 3] and Q [Bt, M, 3] fp32, with autograd.

    Caller-side convenience, not a library operation: the nearest-neighbour
    distances and their gradients come from maxsim_chamfer_fwd and
    maxsim_chamfer_bwd; the mean over points that turns them into the loss
    is a torch reduction here (its backward hands the per-point weights 1/N
    and 1/M to maxsim_chamfer_bwd)."""
    dist_p, dist_q = ChamferFunction.apply(P, Q)
    return dist_p.mean(dim=-1) + dist_q.mean(dim=-1)


def maxsim_fwd_pairs(Q, D_packed, cu_seqlens, pair_q, pair_b, scores=None, argmax=None, with_argmax=False,
                     stream=None):
    """Scores [P] (and argmax [P, Lq]) of the listed (query, document) pairs over a packed corpus."""
    Nq, Lq, d = Q.shape
    T, d2 = D_packed.shape
    B = cu_seqlens.shape[0] - 1
    P = pair_q.shape[0]
    if d2 != d or Q.dtype != D_packed.dtype:
        raise ValueError("Q and D_packed must share dtype and width")
    dev = Q.device
    _need(Q, "Q")
    _need(D_packed, "D_packed", device=dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(pair_q, "pair_q", torch.int32, dev)
    _need(pair_b, "pair_b", torch.int32, dev)
    if pair_b.shape[0] != P:
        raise ValueError("pair_q and pair_b must have the same length")
    if scores is None:
        scores = torch.empty(P, dtype=torch.float32, device=dev)
    _need(scores, "scores", torch.float32, dev)
    if argmax is None and with_argmax:
        argmax = torch.empty((P, Lq), dtype=torch.int32, device=dev)
    if argmax is not None:
        _need(argmax, "argmax", torch.int32, dev)
    st = lib().maxsim_fwd_pairs(_ptr(Q), _ptr(D_packed), _ptr(cu_seqlens), _dtype_code(Q), _ptr(pair_q),
                                _ptr(pair_b), P, Nq, Lq, B, T, d, _ptr(scores), _ptr(argmax), _stream(Q, stream))
    _check(st, "maxsim_fwd_pairs")
    return scores, argmax


def maxsim_topk(scores, K, ids=None, top_idx=None, top_score=None, stream=None):
    """Per row of scores [Nq, B] fp32: (top_idx [Nq, K] int32, top_score [Nq, K]), best first,
    equal scores by ascending id (ids [Nq, B] int32 if given, else the column)."""
    Nq, B = scores.shape
    dev = scores.device
    _need(scores, "scores", torch.float32)
    if ids is not None:
        _need(ids, "ids", torch.int32, dev)
        if ids.shape != scores.shape:
            raise ValueError("ids must have the shape of scores")
    if top_idx is None:
        top_idx = torch.empty((Nq, K), dtype=torch.int32, device=dev)
    if top_score is None:
        top_score = torch.empty((Nq, K), dtype=torch.float32, device=dev)
    _need(top_idx, "top_idx", torch.int32, dev)
    _need(top_score, "top_score", torch.float32, dev)
    st = lib().maxsim_topk(_ptr(scores), _ptr(ids), Nq, B, K, _ptr(top_idx), _ptr(top_score),
                           _stream(scores, stream))
    _check(st, "maxsim_topk")
    return top_idx, top_score


def maxsim_two_stage_workspace_bytes(Nq, B, K1):
    return int(lib().maxsim_two_stage_workspace_bytes(Nq, B, K1))


def maxsim_two_stage_topk(Q8, q_scale, D8, d_scale, Q16, D16, cu_seqlens, max_Ld, K1, K2, workspace=None,
                          stream=None):
    """INT8 scan of the whole corpus, each query's K1 best re-scored in fp16 / bf16 from Q16 / D16,
    the K2 best kept.  Returns (cand [Nq, K1], cand_score8, top_idx [Nq, K2], top_score)."""
    Nq, Lq, d = Q8.shape
    T = D8.shape[0]
    B = cu_seqlens.shape[0] - 1
    dev = Q8.device
    _need(Q8, "Q8", torch.int8)
    _need(D8, "D8", torch.int8, dev)
    _need(q_scale, "q_scale", torch.float32, dev)
    _need(d_scale, "d_scale", torch.float32, dev)
    _need(Q16, "Q16", device=dev)
    _need(D16, "D16", device=dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if Q16.shape != Q8.shape or D16.shape != D8.shape or Q16.dtype != D16.dtype:
        raise ValueError("Q16 / D16 must be the fp16 or bf16 rows of Q8 / D8")
    nbytes = maxsim_two_stage_workspace_bytes(Nq, B, K1)
    if workspace is None:
        workspace = torch.empty(max(256, nbytes), dtype=torch.uint8, device=dev)
    cand = torch.empty((Nq, K1), dtype=torch.int32, device=dev)
    cand8 = torch.empty((Nq, K1), dtype=torch.float32, device=dev)
    top_idx = torch.empty((Nq, K2), dtype=torch.int32, device=dev)
    top_score = torch.empty((Nq, K2), dtype=torch.float32, device=dev)
    st = lib().maxsim_two_stage_topk(_ptr(Q8), _ptr(q_scale), _ptr(D8), _ptr(d_scale), _ptr(Q16), _ptr(D16),
                                     _ptr(cu_seqlens), _dtype_code(Q16), Nq, Lq, B, T, int(max_Ld), d, K1, K2,
                                     _ptr(cand), _ptr(cand8), _ptr(top_idx), _ptr(top_score), _ptr(workspace),
                                     workspace.numel(), _stream(Q8, stream))
    _check(st, "maxsim_two_stage_topk")
    return cand, cand8, top_idx, top_score
