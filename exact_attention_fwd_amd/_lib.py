"""ctypes binding of libfa2.so (include/fa2.h): argument marshalling only.

Every step of the attention forward pass runs in the library's gfx950
kernels.  There is no fallback: if the library is missing or does not load,
the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa2.so")

FA2_OK = 0
FA2_ERR_INVALID_ARG = 1
FA2_ERR_UNSUPPORTED = 2
FA2_ERR_MISALIGNED = 3
FA2_ERR_NO_DEVICE = 4
FA2_ERR_LAUNCH = 5

EXPORTED = ("fa2_fwd", "fa2_status_string", "fa2_last_hip_error", "fa2_version")

_lock = threading.Lock()
_lib = None


class Fa2Error(RuntimeError):
    """A non-zero status from fa2_fwd."""

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


def fa2_status_string(status: int) -> str:
    return load_library().fa2_status_string(int(status)).decode()


def fa2_last_hip_error() -> int:
    return load_library().fa2_last_hip_error()


def fa2_version() -> str:
    return load_library().fa2_version().decode()


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """O, LSE = attention forward of torch fp16 CUDA tensors [B, H, N, d].

    torch supplies device memory and the stream only; ``out`` (fp16
    [B, H, N, d]) and ``lse`` (fp32 [B, H, N]) may be passed to reuse
    buffers.  ``scale`` defaults to 1/sqrt(d).  Raises ValueError for bad
    tensors and Fa2Error for a non-zero library status.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor")
        if t.dtype != torch.float16:
            raise ValueError(f"{name} must be float16")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have the same shape")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k and v must be on one device")
    B, H, N, d = q.shape
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.float16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous fp16 tensor shaped like q")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     B, H, N, d, scale, causal, stream)
    if status != FA2_OK:
        raise Fa2Error(status, f"fa2_fwd failed: {fa2_status_string(status)} "
                               f"(hip error {fa2_last_hip_error()})")
    return out, lse
