"""fp64 CPU oracle for exact attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package imports
nothing from the product: the two sides share only the seeded input
generators, which hold none of the method's arithmetic.

``attn_oracle.c`` computes the plain definition of attention (scores, masked
softmax, weighted sum of values, log-sum-exp) in double precision; see the
header of that file for the passages it follows.  ``online.py`` holds the
pages' tiled online-softmax algorithm and the split-KV merge, in fp64, as a
second test reference.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "libattn_oracle.so")

F32, BF16, F64 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) next to its source."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    vp, dp, lp, ip = ctypes.c_void_p, ctypes.c_double, ctypes.c_long, ctypes.c_int
    lib.oracle_attention.argtypes = [vp, vp, vp, ip, vp, vp, lp, lp, lp, lp, lp, lp, dp, ip, lp]
    lib.oracle_attention.restype = ip
    lib.oracle_attention_rows.argtypes = [vp, vp, vp, ip, vp, lp, vp, vp,
                                          lp, lp, lp, lp, lp, lp, dp, ip, lp]
    lib.oracle_attention_rows.restype = ip
    lib.oracle_decode.argtypes = [vp, vp, vp, ip, vp, vp, vp, lp, lp, lp, lp, lp, dp, lp]
    lib.oracle_decode.restype = ip
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ip
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load_library(_LIB)
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_num_threads())


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:       # bf16 bit patterns
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs must be float32, float64 or bf16 bits (uint16), got {a.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _prep(*arrays):
    arrays = [np.ascontiguousarray(a) for a in arrays]
    codes = {_dtype_code(a) for a in arrays}
    if len(codes) != 1:
        raise TypeError("q, k and v must share one storage dtype")
    return arrays, codes.pop()


def _window(window, causal=True) -> int:
    if window is None or window <= 0:
        return 0
    if not causal:
        raise ValueError("a sliding window is causal")
    return int(window)


def attention(q, k, v, scale: float, causal: bool, window=None):
    """O [B,H,N_q,d] and LSE [B,H,N_q] in fp64 for q [B,H,N_q,d], k/v [B,H_kv,N_k,d].
    ``window`` (keys, causal only): row i sees the ``window`` keys ending at its
    last causally visible key."""
    (q, k, v), code = _prep(q, k, v)
    B, H, N_q, d = q.shape
    Bk, H_kv, N_k, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    o = np.empty((B, H, N_q, d), np.float64)
    lse = np.empty((B, H, N_q), np.float64)
    rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), code, _ptr(o), _ptr(lse),
                                  B, H, H_kv, N_q, N_k, d, float(scale), int(bool(causal)),
                                  _window(window, causal))
    if rc != 0:
        raise ValueError(f"oracle_attention failed with code {rc}")
    return o, lse


def attention_rows(q, k, v, rows, scale: float, causal: bool, window=None):
    """O and LSE for the (b, h, i) query rows listed in ``rows`` only."""
    (q, k, v), code = _prep(q, k, v)
    B, H, N_q, d = q.shape
    _, H_kv, N_k, _ = k.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    rc = _load().oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), code, _ptr(rows), n,
                                       _ptr(o), _ptr(lse), B, H, H_kv, N_q, N_k, d,
                                       float(scale), int(bool(causal)), _window(window, causal))
    if rc != 0:
        raise ValueError(f"oracle_attention_rows failed with code {rc}")
    return o, lse


def decode(q, k_cache, v_cache, seq_lens, scale: float, window=None):
    """One decode step: O [B,H,d] and LSE [B,H] in fp64; with ``window`` the
    query sees only the last ``window`` cached rows."""
    (q, k_cache, v_cache), code = _prep(q, k_cache, v_cache)
    B, H, d = q.shape
    _, H_kv, N_max, _ = k_cache.shape
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if lens.shape != (B,):
        raise ValueError("seq_lens must have one entry per sequence")
    o = np.empty((B, H, d), np.float64)
    lse = np.empty((B, H), np.float64)
    rc = _load().oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), code, _ptr(lens),
                               _ptr(o), _ptr(lse), B, H, H_kv, N_max, d, float(scale), _window(window))
    if rc != 0:
        raise ValueError(f"oracle_decode failed with code {rc}")
    return o, lse


def gather_pages(pages, block_table, seq_lens):
    """Contiguous cache [B,H_kv,N,d] from a paged pool [P,H_kv,page_size,d].

    Logical row r of sequence b is row r % page_size of physical page
    block_table[b, r // page_size] ("Attention variants" §5: the KV cache is
    cut into fixed-size blocks managed like virtual-memory pages).  Rows at or
    past seq_lens[b] are left as NaN and never read by decode().
    """
    pages = np.asarray(pages)
    bt = np.asarray(block_table)
    lens = np.asarray(seq_lens)
    P, H_kv, ps, d = pages.shape
    B = bt.shape[0]
    n = int(bt.shape[1]) * ps
    fill = np.uint16(0x7FC0) if pages.dtype == np.uint16 else np.nan
    out = np.full((B, H_kv, n, d), fill, dtype=pages.dtype)
    for b in range(B):
        r = np.arange(int(lens[b]))
        out[b, :, :len(r)] = pages[bt[b, r // ps], :, r % ps].transpose(1, 0, 2)
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale: float):
    """decode() on a paged cache: gather each sequence's rows, then decode."""
    k = gather_pages(k_pages, block_table, seq_lens)
    v = gather_pages(v_pages, block_table, seq_lens)
    return decode(q, k, v, seq_lens, scale)


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode FP8 E4M3 bytes (the OCP 8-bit format with 4 exponent bits, bias 7,
    3 mantissa bits, no infinities, NaN = S.1111.111) to float64.

    exponent field 0:     (-1)^s * 2^-6 * m/8        (subnormals and zeros)
    exponent field 1..15: (-1)^s * 2^(e-7) * (1 + m/8), except e = 15, m = 7: NaN
    The pages store the KV cache in FP8 without naming the variant; this is the
    variant MI355X (gfx950) converts in hardware.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    out = sign * mag
    out[(e == 15) & ((c & 0x7) == 7)] = np.nan
    return out


def decode_fp8(q, k_codes, v_codes, k_scale: float, v_scale: float, seq_lens, scale: float, window=None):
    """decode() on an FP8 E4M3 cache with one scale per tensor: the cache holds
    K / k_scale and V / v_scale, so the attended keys are k_scale * e4m3(K) and
    the values v_scale * e4m3(V) ("Attention variants" §5: KV cache stored in
    FP8 to halve the bytes a memory-bound decode step reads)."""
    k = e4m3_to_f64(k_codes) * float(k_scale)
    v = e4m3_to_f64(v_codes) * float(v_scale)
    qd = np.asarray(q)
    if qd.dtype == np.uint16:
        qd = (qd.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return decode(np.ascontiguousarray(qd, dtype=np.float64), k, v, seq_lens, scale, window)
