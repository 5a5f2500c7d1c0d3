"""ctypes binding of libfa2.so (include/fa2.h): argument marshalling only.

Every step of the attention forward and backward passes runs in the
library's gfx950 kernels.  There is no fallback: if the library is missing or does not load,
the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

# The in-tree build; FA2_LIBRARY names another build of the same C ABI (the
# CPU tests use it for a sanitizer build of the argument checks).
LIB_PATH = os.environ.get("FA2_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfa2.so")

FA2_OK = 0
FA2_ERR_INVALID_ARG = 1
FA2_ERR_UNSUPPORTED = 2
FA2_ERR_MISALIGNED = 3
FA2_ERR_NO_DEVICE = 4
FA2_ERR_LAUNCH = 5
FA2_ERR_SCRATCH_LIMIT = 6
FA2_NOALLOC_SCRATCH_BYTES = 8 << 20   # the fixed scratch of fa2_fwd_splitkv_noalloc

EXPORTED = ("fa2_fwd", "fa2_bwd", "fa1_fwd", "fa1_workspace_bytes", "fa2_fwd_splitkv",
            "fa2_fwd_splitkv_noalloc", "fa2_splitkv_splits", "fa2_splitkv_workspace_bytes", "fa2_lse_merge",
            "fa2_status_string", "fa2_last_hip_error", "fa2_version")

_lock = threading.Lock()
_lib = None


class Fa2Error(RuntimeError):
    """A non-zero status from fa2_fwd or fa2_bwd."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa2.so once and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m exact_attention_fwd_amd._build` "
                "(or __graft_entry__.build()); there is no non-HIP fallback")
        lib = ctypes.CDLL(path)
        lib.fa2_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa2_fwd.restype = ctypes.c_int
        lib.fa2_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa2_bwd.restype = ctypes.c_int
        lib.fa1_fwd.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_size_t] + [ctypes.c_int] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa1_fwd.restype = ctypes.c_int
        lib.fa1_workspace_bytes.argtypes = [ctypes.c_int] * 4
        lib.fa1_workspace_bytes.restype = ctypes.c_size_t
        lib.fa2_fwd_splitkv.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_size_t] + [
            ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa2_fwd_splitkv.restype = ctypes.c_int
        lib.fa2_fwd_splitkv_noalloc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa2_fwd_splitkv_noalloc.restype = ctypes.c_int
        lib.fa2_splitkv_splits.argtypes = [ctypes.c_int] * 6
        lib.fa2_splitkv_splits.restype = ctypes.c_int
        lib.fa2_splitkv_workspace_bytes.argtypes = [ctypes.c_int] * 6
        lib.fa2_splitkv_workspace_bytes.restype = ctypes.c_size_t
        lib.fa2_lse_merge.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
        lib.fa2_lse_merge.restype = ctypes.c_int
        lib.fa2_status_string.argtypes = [ctypes.c_int]
        lib.fa2_status_string.restype = ctypes.c_char_p
        lib.fa2_last_hip_error.argtypes = []
        lib.fa2_last_hip_error.restype = ctypes.c_int
        lib.fa2_version.argtypes = []
        lib.fa2_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def fa2_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> int:
    """The C entry point, same arguments: q, k, v, o, lse are device
    addresses (ints), stream a hipStream_t as an int (0 = null stream).
    Returns the fa2_status code."""
    return load_library().fa2_fwd(q, k, v, o, lse, int(B), int(H), int(N), int(d),
                                  float(scale), int(bool(causal)), stream)


def fa2_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream) -> int:
    """The C entry point, same arguments (device addresses as ints)."""
    return load_library().fa2_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, int(B), int(H),
                                  int(N), int(d), float(scale), int(bool(causal)), stream)


def fa1_fwd(q, k, v, o, lse, ws, ws_bytes, B, H, N, d, scale, causal, stream) -> int:
    """The C entry point of the FlashAttention-1-order comparator."""
    return load_library().fa1_fwd(q, k, v, o, lse, ws, int(ws_bytes), int(B), int(H), int(N),
                                  int(d), float(scale), int(bool(causal)), stream)


def fa1_workspace_bytes(B, H, N, d) -> int:
    return load_library().fa1_workspace_bytes(int(B), int(H), int(N), int(d))


def fa2_fwd_splitkv(q, k, v, o, lse, ws, ws_bytes, B, H, Nq, Nk, d, scale, n_splits, stream) -> int:
    """The C entry point of the split key/value forward (device addresses as ints)."""
    return load_library().fa2_fwd_splitkv(q, k, v, o, lse, ws, int(ws_bytes), int(B), int(H),
                                          int(Nq), int(Nk), int(d), float(scale), int(n_splits),
                                          stream)


def fa2_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, n_splits, stream) -> int:
    """The C entry point of the split key/value forward that allocates
    nothing (the library's fixed scratch holds the partial results)."""
    return load_library().fa2_fwd_splitkv_noalloc(q, k, v, o, lse, int(B), int(H), int(Nq),
                                                  int(Nk), int(d), float(scale), int(n_splits),
                                                  stream)


def fa2_splitkv_splits(B, H, Nq, Nk, d, n_splits=0) -> int:
    return load_library().fa2_splitkv_splits(int(B), int(H), int(Nq), int(Nk), int(d), int(n_splits))


def fa2_splitkv_workspace_bytes(B, H, Nq, Nk, d, n_splits=0) -> int:
    return load_library().fa2_splitkv_workspace_bytes(int(B), int(H), int(Nq), int(Nk), int(d),
                                                      int(n_splits))


def fa2_lse_merge(o_parts, lse_parts, o, lse, n_parts, rows, d, stream) -> int:
    return load_library().fa2_lse_merge(o_parts, lse_parts, o, lse, int(n_parts), int(rows),
                                        int(d), stream)


def fa2_status_string(status: int) -> str:
    return load_library().fa2_status_string(int(status)).decode()


def fa2_last_hip_error() -> int:
    return load_library().fa2_last_hip_error()


def fa2_version() -> str:
    return load_library().fa2_version().decode()


def _check_qkv(named):
    import torch

    first = named[0][1]
    for name, t in named:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor")
        if t.dtype != torch.float16:
            raise ValueError(f"{name} must be float16")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
        if t.shape != first.shape:
            raise ValueError(f"{name} must have the shape of {named[0][0]}")
        if t.device != first.device:
            raise ValueError(f"{name} must be on the device of {named[0][0]}")


def _out(t, like, dtype, shape, name):
    import torch

    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() \
            or t.device != like.device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return t


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """O, LSE = attention forward of torch fp16 CUDA tensors [B, H, N, d].

    torch supplies device memory and the stream only; ``out`` (fp16
    [B, H, N, d]) and ``lse`` (fp32 [B, H, N]) may be passed to reuse
    buffers.  ``scale`` defaults to 1/sqrt(d).  Raises ValueError for bad
    tensors and Fa2Error for a non-zero library status.
    """
    import torch

    _check_qkv((("q", q), ("k", k), ("v", v)))
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    out = _out(out, q, torch.float16, q.shape, "out")
    lse = _out(lse, q, torch.float32, (B, H, N), "lse")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     B, H, N, d, scale, causal, stream)
    if status != FA2_OK:
        raise Fa2Error(status, f"fa2_fwd failed: {fa2_status_string(status)} "
                               f"(hip error {fa2_last_hip_error()})")
    return out, lse


def bwd(q, k, v, o, lse, dout, scale=None, causal=False, dq=None, dk=None, dv=None,
        delta=None, stream=None):
    """dQ, dK, dV (and delta) of the attention forward, on torch tensors.

    q, k, v, o, dout are fp16 CUDA tensors [B, H, N, d] (o and lse the
    forward's outputs for the same arguments), lse fp32 [B, H, N].  Output
    buffers may be passed to reuse memory; ``delta`` (fp32 [B, H, N]) is the
    workspace the library fills with dO . O per row.  ``scale`` defaults to
    1/sqrt(d).  Returns (dq, dk, dv, delta).
    """
    import torch

    _check_qkv((("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)))
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    if lse is None:
        raise ValueError("lse must be the forward's LSE output for the same q, k, v")
    lse = _out(lse, q, torch.float32, (B, H, N), "lse")
    dq = _out(dq, q, torch.float16, q.shape, "dq")
    dk = _out(dk, q, torch.float16, q.shape, "dk")
    dv = _out(dv, q, torch.float16, q.shape, "dv")
    delta = _out(delta, q, torch.float32, (B, H, N), "delta")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = fa2_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                     delta.data_ptr(), B, H, N, d, scale, causal, stream)
    if status != FA2_OK:
        raise Fa2Error(status, f"fa2_bwd failed: {fa2_status_string(status)} "
                               f"(hip error {fa2_last_hip_error()})")
    return dq, dk, dv, delta


def fwd_fa1(q, k, v, scale=None, causal=False, out=None, lse=None, workspace=None, stream=None):
    """The same forward pass in the FlashAttention-1 loop order (the
    comparator of ``fwd``).  ``workspace`` is a uint8 CUDA tensor of at least
    fa1_workspace_bytes(B, H, N, d) bytes (allocated if None).  Returns
    (o, lse)."""
    import torch

    _check_qkv((("q", q), ("k", k), ("v", v)))
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    out = _out(out, q, torch.float16, q.shape, "out")
    lse = _out(lse, q, torch.float32, (B, H, N), "lse")
    need = fa1_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = fa1_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     workspace.data_ptr(), workspace.numel() * workspace.element_size(), B, H, N,
                     d, scale, causal, stream)
    if status != FA2_OK:
        raise Fa2Error(status, f"fa1_fwd failed: {fa2_status_string(status)} "
                               f"(hip error {fa2_last_hip_error()})")
    return out, lse


def fwd_splitkv(q, k, v, scale=None, n_splits=0, out=None, lse=None, workspace=None, stream=None):
    """Non-causal attention of q [B, H, Nq, d] over k, v [B, H, Nk, d] with
    the keys split across workgroups (0 = the library's choice); returns
    (o, lse).  ``workspace`` (uint8 CUDA tensor) is allocated when needed."""
    import torch

    _check_qkv((("k", k), ("v", v)))
    _check_qkv((("q", q),))
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape[:2] != q.shape[:2] or k.shape[3] != d or k.device != q.device:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d], on one device")
    if scale is None:
        scale = d ** -0.5
    out = _out(out, q, torch.float16, q.shape, "out")
    lse = _out(lse, q, torch.float32, (B, H, Nq), "lse")
    need = fa2_splitkv_workspace_bytes(B, H, Nq, Nk, d, n_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = fa2_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), ws_ptr, ws_bytes, B, H, Nq, Nk, d, scale, n_splits,
                             stream)
    if status != FA2_OK:
        raise Fa2Error(status, f"fa2_fwd_splitkv failed: {fa2_status_string(status)} "
                               f"(hip error {fa2_last_hip_error()})")
    return out, lse


def fwd_splitkv_noalloc(q, k, v, out, lse, scale=None, n_splits=0, stream=None):
    """``fwd_splitkv`` through the entry point that allocates nothing: the
    caller passes the outputs (``out`` fp16 [B, H, Nq, d], ``lse`` fp32
    [B, H, Nq]) and the partial results go to the library's fixed scratch
    buffer (FA2_NOALLOC_SCRATCH_BYTES per GPU).  Calls on one GPU must not
    overlap in time.  Returns (out, lse)."""
    import torch

    _check_qkv((("k", k), ("v", v)))
    _check_qkv((("q", q),))
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape[:2] != q.shape[:2] or k.shape[3] != d or k.device != q.device:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d], on one device")
    if out is None or lse is None:
        raise ValueError("out and lse must be passed: this entry point allocates nothing")
    if scale is None:
        scale = d ** -0.5
    out = _out(out, q, torch.float16, q.shape, "out")
    lse = _out(lse, q, torch.float32, (B, H, Nq), "lse")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = fa2_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, H, Nq, Nk, d, scale, n_splits, stream)
    if status != FA2_OK:
        raise Fa2Error(status, f"fa2_fwd_splitkv_noalloc failed: {fa2_status_string(status)} "
                               f"(hip error {fa2_last_hip_error()})")
    return out, lse


def lse_merge(o_parts, lse_parts, out=None, lse=None, stream=None):
    """Merge partial results: o_parts fp32 [S, ..., d], lse_parts fp32 [S, ...]
    (CUDA tensors) -> (o fp16 [..., d], lse fp32 [...])."""
    import torch

    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts and lse_parts must be float32")
    if not (o_parts.is_cuda and lse_parts.is_cuda and o_parts.is_contiguous()
            and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous CUDA tensors")
    if tuple(o_parts.shape[:-1]) != tuple(lse_parts.shape) or o_parts.dim() < 2:
        raise ValueError("o_parts must be [S, ..., d] and lse_parts [S, ...]")
    S, d = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts.numel() // S
    out = _out(out, o_parts, torch.float16, o_parts.shape[1:], "out")
    lse = _out(lse, o_parts, torch.float32, lse_parts.shape[1:], "lse")
    if stream is None:
        stream = torch.cuda.current_stream(o_parts.device).cuda_stream
    status = fa2_lse_merge(o_parts.data_ptr(), lse_parts.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), S, rows, d, stream)
    if status != FA2_OK:
        raise Fa2Error(status, f"fa2_lse_merge failed: {fa2_status_string(status)} "
                               f"(hip error {fa2_last_hip_error()})")
    return out, lse
