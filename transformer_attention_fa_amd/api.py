"""Thin Python binding of libfa.so (include/fa.h) over ctypes.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch is used for device memory and for the
current stream; there is no CPU or PyTorch fallback -- if libfa.so is missing
or a call fails, an exception is raised.

Entry points mirror the C names: ``fwd`` (fa_fwd, bf16; with ``window=W``
fa_fwd_window), ``fwd_f32`` (fa_fwd_f32), ``decode`` (fa_decode; with
``window=W`` fa_decode_window), ``decode_noalloc`` (fa_decode_noalloc),
``decode_paged`` (fa_decode_paged),
``decode_fp8`` (fa_decode_fp8), ``decode_workspace_bytes``.
``scale=None`` means 1/sqrt(d), like the ``softmax_scale=None`` default of the
flash_attn_func usage shown in "Attention mechanism evolution: MHA -> MLA,
Flash Attention" (toolsku.com), Flash Attention section.
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3

EXPORTED = ("fa_fwd", "fa_fwd_window", "fa_fwd_f32", "fa_decode", "fa_decode_noalloc",
            "fa_decode_window", "fa_decode_paged", "fa_decode_fp8", "fa_decode_workspace_bytes",
            "fa_status_string", "fa_last_error")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def open_library(path: str):
    """Open a build of the library at `path` (its own handle) and declare the C
    signatures."""
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run `python -m transformer_attention_fa_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_window.restype = i
    lib.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_f32.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_decode.restype = i
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_decode_noalloc.restype = i
    lib.fa_decode_window.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_decode_window.restype = i
    lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_decode_paged.restype = i
    lib.fa_decode_fp8.argtypes = [vp, vp, vp, f, f, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_decode_fp8.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    return lib


def load():
    """Open libfa.so (built in-tree; FA_LIBRARY names another build, such as
    the race-hunting libfa_debug_barriers.so) once per process."""
    global _lib
    if _lib is None:
        _lib = open_library(os.environ.get("FA_LIBRARY") or LIB_PATH)
    return _lib


def check(status: int) -> None:
    if status != FA_OK:
        lib = load()
        raise FAError(status, f"{lib.fa_status_string(status).decode()}: {lib.fa_last_error().decode()}")


def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _require(t, name, dtype, ndim, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major, d fastest)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _fwd(fn, dtype, q, k, v, causal, scale, out, lse, mask_arg=None):
    torch = _torch()
    _require(q, "q", dtype, 4)
    _require(k, "k", dtype, 4, q.device)
    _require(v, "v", dtype, 4, q.device)
    B, H, N_q, d = q.shape
    Bk, H_kv, N_k, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", dtype, 4, q.device)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have the shape of q")
    if lse is None:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    elif lse is not False:
        _require(lse, "lse", torch.float32, 3, q.device)
        if tuple(lse.shape) != (B, H, N_q):
            raise ValueError("lse must have shape [B, H, N_q]")
    lse_t = None if lse is False else lse
    with torch.cuda.device(q.device):
        check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse_t),
                 B, H, H_kv, N_q, N_k, d, float(scale),
                 int(bool(causal)) if mask_arg is None else int(mask_arg), _stream(q.device)))
    return out, lse_t


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, window=None):
    """fa_fwd: bf16 q [B,H,N_q,d], k/v [B,H_kv,N_k,d] -> (o bf16 [B,H,N_q,d], lse fp32 [B,H,N_q]).

    Pass ``lse=False`` to skip the log-sum-exp output.  ``window=W`` calls
    fa_fwd_window (causal sliding window of W keys; ``causal`` must be true).
    """
    torch = _torch()
    if window is None:
        return _fwd(load().fa_fwd, torch.bfloat16, q, k, v, causal, scale, out, lse)
    if not causal:
        raise ValueError("a sliding window is causal: pass causal=True")
    return _fwd(load().fa_fwd_window, torch.bfloat16, q, k, v, True, scale, out, lse, mask_arg=int(window))


def fwd_f32(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """fa_fwd_f32: the same with fp32 tensors."""
    torch = _torch()
    return _fwd(load().fa_fwd_f32, torch.float32, q, k, v, causal, scale, out, lse)


def decode_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, d, num_splits))


def _decode_outputs(q, num_splits, out, lse, workspace):
    """Workspace, o [B,H,d] (bf16) and lse [B,H] (fp32, or False for none) of a
    decode call: allocated when not given, shape-checked when given (the
    kernels write B*H rows of d values and B*H lse values)."""
    torch = _torch()
    B, H, d = q.shape
    if workspace is None:
        # need == 0 means the arguments are invalid: the library call reports why
        need = decode_workspace_bytes(B, H, d, num_splits)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace is not False:           # False: the entry point needs none
        _require(workspace, "workspace", torch.uint8, 1, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", torch.bfloat16, 3, q.device)
        if tuple(out.shape) != (B, H, d):
            raise ValueError(f"out must have shape {(B, H, d)}, got {tuple(out.shape)}")
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    elif lse is not False:
        _require(lse, "lse", torch.float32, 2, q.device)
        if tuple(lse.shape) != (B, H):
            raise ValueError(f"lse must have shape {(B, H)}, got {tuple(lse.shape)}")
    return workspace, out, (None if lse is False else lse)


def decode(q, k_cache, v_cache, seq_lens, num_splits: int = 16, scale: float | None = None,
           out=None, lse=None, workspace=None, window=None):
    """fa_decode: q [B,H,d], caches [B,H_kv,N_max,d] (bf16), seq_lens [B] int32 on the device.

    Returns (o bf16 [B,H,d], lse fp32 [B,H]).  ``workspace`` (uint8 tensor) may
    be passed to avoid an allocation per call.  ``window=W`` calls
    fa_decode_window (the query sees the last W rows of its cache).
    """
    torch = _torch()
    _require(q, "q", torch.bfloat16, 3)
    _require(k_cache, "k_cache", torch.bfloat16, 4, q.device)
    _require(v_cache, "v_cache", torch.bfloat16, 4, q.device)
    _require(seq_lens, "seq_lens", torch.int32, 1, q.device)
    B, H, d = q.shape
    Bk, H_kv, N_max, dk = k_cache.shape
    if Bk != B or dk != d or tuple(v_cache.shape) != tuple(k_cache.shape) or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    workspace, out, lse_t = _decode_outputs(q, num_splits, out, lse, workspace)
    with torch.cuda.device(q.device):
        if window is None:
            check(load().fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                   out.data_ptr(), _ptr(lse_t), B, H, H_kv, N_max, d, float(scale),
                                   int(num_splits), workspace.data_ptr(), workspace.numel(), _stream(q.device)))
        else:
            check(load().fa_decode_window(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                          seq_lens.data_ptr(), out.data_ptr(), _ptr(lse_t), B, H, H_kv, N_max, d,
                                          float(scale), int(window), int(num_splits), workspace.data_ptr(),
                                          workspace.numel(), _stream(q.device)))
    return out, lse_t


def decode_noalloc(q, k_cache, v_cache, seq_lens, num_splits: int = 16, scale: float | None = None,
                   out=None, lse=None):
    """fa_decode_noalloc: fa_decode with its split partials in the library's
    per-GPU scratch array (no workspace; the library allocates nothing).  Calls
    that overlap on one GPU race on that array.  ``out`` and ``lse`` are
    allocated here when not given; pass them to allocate nothing at all."""
    torch = _torch()
    _require(q, "q", torch.bfloat16, 3)
    _require(k_cache, "k_cache", torch.bfloat16, 4, q.device)
    _require(v_cache, "v_cache", torch.bfloat16, 4, q.device)
    _require(seq_lens, "seq_lens", torch.int32, 1, q.device)
    B, H, d = q.shape
    Bk, H_kv, N_max, dk = k_cache.shape
    if Bk != B or dk != d or tuple(v_cache.shape) != tuple(k_cache.shape) or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _, out, lse_t = _decode_outputs(q, num_splits, out, lse, workspace=False)
    with torch.cuda.device(q.device):
        check(load().fa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
                                       out.data_ptr(), _ptr(lse_t), B, H, H_kv, N_max, d, float(scale),
                                       int(num_splits), _stream(q.device)))
    return out, lse_t


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, num_splits: int = 16, scale: float | None = None,
                 out=None, lse=None, workspace=None):
    """fa_decode_paged: q [B,H,d]; page pools [num_pages,H_kv,page_size,d] (bf16);
    block_table [B,max_blocks] and seq_lens [B] int32 on the device."""
    torch = _torch()
    _require(q, "q", torch.bfloat16, 3)
    _require(k_pages, "k_pages", torch.bfloat16, 4, q.device)
    _require(v_pages, "v_pages", torch.bfloat16, 4, q.device)
    _require(block_table, "block_table", torch.int32, 2, q.device)
    _require(seq_lens, "seq_lens", torch.int32, 1, q.device)
    B, H, d = q.shape
    num_pages, H_kv, page_size, dk = k_pages.shape
    if dk != d or tuple(v_pages.shape) != tuple(k_pages.shape) or block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, page pools, block_table and seq_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    workspace, out, lse_t = _decode_outputs(q, num_splits, out, lse, workspace)
    with torch.cuda.device(q.device):
        check(load().fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                     block_table.shape[1], seq_lens.data_ptr(), out.data_ptr(), _ptr(lse_t),
                                     B, H, H_kv, num_pages, page_size, d, float(scale), int(num_splits),
                                     workspace.data_ptr(), workspace.numel(), _stream(q.device)))
    return out, lse_t


def decode_fp8(q, k_cache, v_cache, k_scale: float, v_scale: float, seq_lens, num_splits: int = 16,
               scale: float | None = None, out=None, lse=None, workspace=None):
    """fa_decode_fp8: q [B,H,d] bf16; caches [B,H_kv,N_max,d] uint8 E4M3 codes with
    per-tensor scales (keys k_scale * code, values v_scale * code)."""
    torch = _torch()
    _require(q, "q", torch.bfloat16, 3)
    _require(k_cache, "k_cache", torch.uint8, 4, q.device)
    _require(v_cache, "v_cache", torch.uint8, 4, q.device)
    _require(seq_lens, "seq_lens", torch.int32, 1, q.device)
    B, H, d = q.shape
    Bk, H_kv, N_max, dk = k_cache.shape
    if Bk != B or dk != d or tuple(v_cache.shape) != tuple(k_cache.shape) or seq_lens.shape[0] != B:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    workspace, out, lse_t = _decode_outputs(q, num_splits, out, lse, workspace)
    with torch.cuda.device(q.device):
        check(load().fa_decode_fp8(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), float(k_scale),
                                   float(v_scale), seq_lens.data_ptr(), out.data_ptr(), _ptr(lse_t), B, H, H_kv,
                                   N_max, d, float(scale), int(num_splits), workspace.data_ptr(), workspace.numel(),
                                   _stream(q.device)))
    return out, lse_t
