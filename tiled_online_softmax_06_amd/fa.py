"""ctypes binding of libfa.so (include/fa.h).  Argument marshalling only.

torch tensors supply device memory and the current HIP stream; the library
does every step of the attention computation in its own kernels.  There is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

FA_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libfa.so")


def load_library():
    """Load libfa.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.fa_forward.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa_forward.restype = ctypes.c_int
        lib.fa_forward_gqa.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa_forward_gqa.restype = ctypes.c_int
        lib.fa_backward.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 5 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa_backward.restype = ctypes.c_int
        lib.fa_forward_split.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.fa_forward_split.restype = ctypes.c_int
        lib.fa_forward_split_noalloc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
        lib.fa_forward_split_noalloc.restype = ctypes.c_int
        lib.fa_split_workspace_bytes.argtypes = [ctypes.c_int64] * 5
        lib.fa_split_workspace_bytes.restype = ctypes.c_int64
        lib.fa_split_suggest.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
        lib.fa_split_suggest.restype = ctypes.c_int64
        lib.fa_merge.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 4 + [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        lib.fa_merge.restype = ctypes.c_int
        lib.fa_forward_fp8.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [ctypes.c_float] * 4 + [
            ctypes.c_int, ctypes.c_void_p]
        lib.fa_forward_fp8.restype = ctypes.c_int
        lib.fa_status_string.argtypes = [ctypes.c_int]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_version.argtypes = []
        lib.fa_version.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def status_string(code: int) -> str:
    return load_library().fa_status_string(int(code)).decode()


def forward_into(q, k, v, o, lse, scale: float | None = None, stream=None) -> None:
    """O and LSE are written in place; all five tensors are on one GPU.

    q, o: (B, H, N, d); k, v: (B, H_kv, N, d) with H_kv dividing H (H_kv < H:
    grouped-query attention through fa_forward_gqa; H_kv = H: fa_forward)."""
    lib = load_library()
    _check_forward(q, k, v, o, lse)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    handle = _stream_handle(q, stream)
    with torch.cuda.device(q.device):
        if k.shape[1] == H:
            rc = lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                B, H, N, d, float(scale), FA_DTYPE[q.dtype], handle)
        else:
            rc = lib.fa_forward_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    B, H, k.shape[1], N, d, float(scale), FA_DTYPE[q.dtype], handle)
    if rc != 0:
        raise RuntimeError(f"fa_forward failed: {status_string(rc)} ({rc})")


def _stream_handle(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_forward(q, k, v, o, lse):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (B, H, N, d) row-major")
    if q.dtype not in FA_DTYPE or k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError(f"q, k, v, o must share one of {list(FA_DTYPE)}")
    if lse.dtype != torch.float32:
        raise ValueError("lse must be float32")
    if q.dim() != 4 or o.shape != q.shape or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, o must have shape (B, H, N, d) and k, v one shape (B, H_kv, N, d)")
    if k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:] or k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise ValueError("k, v must be (B, H_kv, N, d) with H_kv dividing H")
    if tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must have shape (B, H, N)")


def split_suggest(B: int, H: int, N: int, d: int, dtype) -> int:
    """The library's split count for these sizes (1: no split pays off)."""
    return int(load_library().fa_split_suggest(B, H, N, d, FA_DTYPE[dtype]))


def split_workspace_bytes(B: int, H: int, N: int, d: int, splits: int) -> int:
    n = int(load_library().fa_split_workspace_bytes(B, H, N, d, splits))
    if n < 0:
        raise ValueError("invalid sizes for a key split")
    return n


def forward_split_into(q, k, v, o, lse, workspace, splits: int, scale: float | None = None, stream=None) -> None:
    """forward_into with the keys cut into `splits` ranges merged afterwards;
    workspace: a contiguous GPU tensor of at least split_workspace_bytes(...)
    bytes (any dtype), which receives the fp32 partial results."""
    lib = load_library()
    _check_forward(q, k, v, o, lse)
    if tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must have shape (B, H, N)")
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    handle = _stream_handle(q, stream)
    with torch.cuda.device(q.device):
        rc = lib.fa_forward_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, k.shape[1], N, d, float(scale), FA_DTYPE[q.dtype], int(splits),
                                  ws_ptr, ws_bytes, handle)
    if rc != 0:
        raise RuntimeError(f"fa_forward_split failed: {status_string(rc)} ({rc})")


def forward_split_noalloc_into(q, k, v, o, lse, splits: int, scale: float | None = None, stream=None) -> None:
    """forward_split_into without a workspace: the partial results go to the
    library's fixed per-GPU scratch (fa_forward_split_noalloc; nothing is
    allocated).  Calls that overlap in time on one GPU share that scratch."""
    lib = load_library()
    _check_forward(q, k, v, o, lse)
    if tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must have shape (B, H, N)")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    handle = _stream_handle(q, stream)
    with torch.cuda.device(q.device):
        rc = lib.fa_forward_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                          B, H, k.shape[1], N, d, float(scale), FA_DTYPE[q.dtype], int(splits),
                                          handle)
    if rc != 0:
        raise RuntimeError(f"fa_forward_split_noalloc failed: {status_string(rc)} ({rc})")


def forward_split(q, k, v, splits: int | None = None, scale: float | None = None):
    """(O, LSE) as forward(), computed over key ranges merged afterwards.
    splits=None takes split_suggest(); the workspace comes from torch."""
    B, H, N, d = q.shape
    if splits is None:
        splits = split_suggest(B, H, N, d, q.dtype)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ws = torch.empty(max(split_workspace_bytes(B, H, N, d, splits), 16), dtype=torch.uint8, device=q.device)
    forward_split_into(q, k, v, o, lse, ws, splits, scale)
    return o, lse


def merge_into(o_parts, lse_parts, o, lse, stream=None) -> None:
    """Merge normalised partial results: o_parts (G, S, M, d) and lse_parts
    (G, S, M) float32 into o (G, M, d) of o's dtype and lse (G, M)."""
    lib = load_library()
    for name, t in (("o_parts", o_parts), ("lse_parts", lse_parts), ("o", o), ("lse", lse)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32 or lse.dtype != torch.float32:
        raise ValueError("o_parts, lse_parts and lse must be float32")
    if o.dtype not in FA_DTYPE:
        raise ValueError(f"o must be one of {list(FA_DTYPE)}")
    if o_parts.dim() != 4 or tuple(lse_parts.shape) != tuple(o_parts.shape[:3]):
        raise ValueError("o_parts must be (G, S, M, d) and lse_parts (G, S, M)")
    G, S, M, d = o_parts.shape
    if tuple(o.shape) != (G, M, d) or tuple(lse.shape) != (G, M):
        raise ValueError("o must be (G, M, d) and lse (G, M)")
    handle = _stream_handle(o, stream)
    with torch.cuda.device(o.device):
        rc = lib.fa_merge(o_parts.data_ptr(), lse_parts.data_ptr(), G, S, M, d, o.data_ptr(), lse.data_ptr(),
                          FA_DTYPE[o.dtype], handle)
    if rc != 0:
        raise RuntimeError(f"fa_merge failed: {status_string(rc)} ({rc})")


def merge(o_parts, lse_parts, dtype=torch.float32):
    G, S, M, d = o_parts.shape
    o = torch.empty((G, M, d), dtype=dtype, device=o_parts.device)
    lse = torch.empty((G, M), dtype=torch.float32, device=o_parts.device)
    merge_into(o_parts, lse_parts, o, lse)
    return o, lse


FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


def forward_fp8_into(q8, k8, v8, descale, o, lse, scale: float | None = None, stream=None) -> None:
    """FP8 forward: q8, k8, v8 hold OCP e4m3 codes (torch.float8_e4m3fn or
    raw uint8), descale = (q_descale, k_descale, v_descale) the per-tensor
    factors of their values; o (B, H, N, d) in bf16 / fp16 / fp32 and lse
    (B, H, N) float32 are written."""
    lib = load_library()
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8), ("o", o), ("lse", lse)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q8.dtype not in FP8_DTYPES or k8.dtype not in FP8_DTYPES or v8.dtype not in FP8_DTYPES:
        raise ValueError("q8, k8, v8 must be float8_e4m3fn (or uint8 codes)")
    if o.dtype not in FA_DTYPE or lse.dtype != torch.float32:
        raise ValueError("o must be float32 / float16 / bfloat16 and lse float32")
    if q8.dim() != 4 or o.shape != q8.shape or k8.dim() != 4 or v8.shape != k8.shape:
        raise ValueError("q8, o must be (B, H, N, d) and k8, v8 one shape (B, H_kv, N, d)")
    if k8.shape[0] != q8.shape[0] or k8.shape[2:] != q8.shape[2:] or k8.shape[1] < 1 or q8.shape[1] % k8.shape[1]:
        raise ValueError("k8, v8 must be (B, H_kv, N, d) with H_kv dividing H")
    if tuple(lse.shape) != tuple(q8.shape[:3]):
        raise ValueError("lse must have shape (B, H, N)")
    B, H, N, d = q8.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (float(x) for x in descale)
    handle = _stream_handle(q8, stream)
    with torch.cuda.device(q8.device):
        rc = lib.fa_forward_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                B, H, k8.shape[1], N, d, float(scale), dq, dk, dv, FA_DTYPE[o.dtype], handle)
    if rc != 0:
        raise RuntimeError(f"fa_forward_fp8 failed: {status_string(rc)} ({rc})")


def forward_fp8(q8, k8, v8, descale, scale: float | None = None, out_dtype=torch.bfloat16):
    """Returns (O, LSE) of the FP8 forward; O in out_dtype."""
    o = torch.empty(q8.shape, dtype=out_dtype, device=q8.device)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    forward_fp8_into(q8, k8, v8, descale, o, lse, scale)
    return o, lse


def forward(q, k, v, scale: float | None = None, splits: int | None = 1):
    """Returns (O, LSE): O like q, LSE float32 (B, H, N), natural log.

    splits: 1 runs fa_forward (one launch, no workspace); None takes the
    library's suggested key-split count and, when that is above 1, runs
    fa_forward_split with a workspace from torch (same result up to
    rounding; faster when few heads leave compute units idle)."""
    if splits is None:
        B, H, N, d = q.shape
        splits = split_suggest(B, H, N, d, q.dtype)
    if splits > 1:
        return forward_split(q, k, v, splits, scale)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    forward_into(q, k, v, o, lse, scale)
    return o, lse


def backward_into(q, k, v, o, do, lse, dq, dk, dv, dws, scale: float | None = None, stream=None) -> None:
    """Gradients of forward(q, k, v) for upstream gradient do, written in place.

    q, o, do, dq: (B, H, N, d); k, v, dk, dv: (B, H_kv, N, d); lse: the
    forward's (B, H, N) float32 LSE; dws: (B, H, N) float32 workspace (gets
    rowsum(do * o)).  fp16 / bf16 only."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("lse", lse), ("dq", dq),
                    ("dk", dk), ("dv", dv), ("dws", dws)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("backward supports float16 and bfloat16")
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's dtype")
    if lse.dtype != torch.float32 or dws.dtype != torch.float32:
        raise ValueError("lse and dws must be float32")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if (o.shape != q.shape or do.shape != q.shape or dq.shape != q.shape or v.shape != k.shape
            or dk.shape != k.shape or dv.shape != k.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]
            or tuple(lse.shape) != (B, H, N) or tuple(dws.shape) != (B, H, N)):
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        rc = lib.fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                             lse.data_ptr(), dws.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                             B, H, Hkv, N, d, float(scale), FA_DTYPE[q.dtype], handle)
    if rc != 0:
        raise RuntimeError(f"fa_backward failed: {status_string(rc)} ({rc})")


def backward(q, k, v, o, do, lse, scale: float | None = None):
    """Returns (dq, dk, dv) for the forward outputs (o, lse) of (q, k, v)."""
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dws = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    backward_into(q, k, v, o, do, lse, dq, dk, dv, dws, scale)
    return dq, dk, dv
