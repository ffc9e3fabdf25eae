"""Seeded synthetic inputs and the named workloads.

This module is the only thing the HIP path and the fp64 oracle share.  It
draws the numbers and lays them out; it holds none of the attention
arithmetic.  It depends on numpy only.

Recipe (no page prints a seed or a generator, so this one is ours):
  * every tensor is i.i.d. N(0, 1), drawn as float32 by numpy's PCG64;
  * a tensor is drawn in independent blocks of one (batch, head) slab each,
    block (t, b, h) from ``default_rng([seed, t, b, h])`` with t = 0, 1, 2 for
    Q, K, V; blocks are drawn on a thread pool and the result does not depend
    on the thread count;
  * bf16 workloads round the float32 draw to bf16 with round-to-nearest-even;
    both sides then read the same rounded values;
  * "K rows scaled by 2" multiplies every element of K by 2 after rounding
    (exact in binary floating point);
  * decode: ``seq_lens`` are integers uniform on [lo, hi] (both ends included)
    from ``default_rng([seed, 100])``; q from ``default_rng([seed, 0])``;
    cache rows [0, len_b) of (b, g) from blocks t = 1 (K) and t = 2 (V); rows
    at or beyond len_b are padding and hold ``pad`` (quiet-NaN bits by
    default, so that a kernel that reads them cannot pass).

Shapes follow the pages' head layout, row-major with d fastest:
q [B,H,N_q,d], k/v [B,H_kv,N_k,d]; decode q [B,H,d], caches [B,H_kv,N_max,d].
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16_QNAN = 0x7FC0


# --------------------------------------------------------------------------
# bf16 storage helpers (bit patterns in uint16)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_QNAN
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_blocks(seed: int, tag: int, n_b: int, n_h: int, shape, rows=None) -> np.ndarray:
    """Array [n_b, n_h, *shape] of N(0,1) float32, block (b, h) from its own stream.

    ``rows`` (optional, per b) limits block (b, h) to its first rows[b] rows of
    shape[0]; the remaining rows are left as zeros for the caller to fill.
    """
    out = np.zeros((n_b, n_h) + tuple(shape), dtype=np.float32)

    def fill(bh):
        b, h = divmod(bh, n_h)
        rng = np.random.default_rng([seed, tag, b, h])
        if rows is None:
            out[b, h] = rng.standard_normal(shape, dtype=np.float32)
        else:
            n = int(rows[b])
            out[b, h, :n] = rng.standard_normal((n,) + tuple(shape[1:]), dtype=np.float32)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n_b * n_h)))
    return out


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    H: int
    H_kv: int
    N_q: int
    N_k: int
    d: int
    causal: bool
    dtype: str            # "bf16" or "f32"
    seed: int
    k_scale: float = 1.0  # every K element multiplied by this (exact power of two)
    window: int = 0       # sliding window in keys (causal only); 0 = none

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Algorithmic FLOPs: 4*B*H*N_q*N_k*d, halved when causal (square
        problems); 4*B*H*d*(visible query-key pairs) with a sliding window or a
        non-square causal problem."""
        if self.window or (self.causal and self.N_q != self.N_k):
            return 4.0 * self.B * self.H * self.d * visible_pairs(self.N_q, self.N_k, self.causal, self.window)
        f = 4.0 * self.B * self.H * self.N_q * self.N_k * self.d
        return f / 2 if self.causal else f


def visible_pairs(n_q: int, n_k: int, causal: bool, window: int = 0) -> int:
    """Number of (query, key) pairs the mask lets through: row i sees keys up to
    i + (n_k - n_q) when causal, and only the last `window` of them with a window."""
    if not causal:
        return n_q * n_k
    i = np.arange(n_q, dtype=np.int64)
    hi = np.minimum(n_k, i + (n_k - n_q) + 1)
    lo = np.maximum(0, i + (n_k - n_q) - window + 1) if window else np.zeros_like(i)
    return int(np.maximum(0, hi - lo).sum())


@dataclass(frozen=True)
class Decode:
    name: str
    B: int
    H: int
    H_kv: int
    d: int
    len_lo: int
    len_hi: int
    N_max: int
    num_splits: int
    seed: int
    dtype: str = "bf16"
    window: int = 0       # the query sees the last `window` cached rows; 0 = all
    page_size: int = 0    # paged cache: rows per page; 0 = contiguous cache
    k_scale: float = 1.0  # FP8 cache (dtype "e4m3"): keys are k_scale * code
    v_scale: float = 1.0  # ... and values v_scale * code

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads: shapes echo the pages' worked examples (B=8, H=32,
# N=8192; H=32 with 8 KV groups; d = 4096/32 = 128; sequence lengths 1K-32K).
SINGLE_HEAD_F32 = Prefill("single_head_f32", 1, 1, 1, 256, 256, 64, False, "f32", 1)
SINGLE_HEAD_F32_CAUSAL = Prefill("single_head_f32_causal", 1, 1, 1, 256, 256, 64, True, "f32", 1)
MHA_PREFILL = Prefill("mha_prefill_b8_h32_n2048_d128_causal", 8, 32, 32, 2048, 2048, 128, True, "bf16", 2)
GQA_PREFILL = Prefill("gqa_prefill_b1_h32_hkv8_n8192_d128_causal_k2", 1, 32, 8, 8192, 8192, 128, True,
                      "bf16", 3, k_scale=2.0)
MQA_PREFILL = Prefill("mqa_prefill_b4_h64_hkv1_n4096_d128", 4, 64, 1, 4096, 4096, 128, False, "bf16", 4)
GQA_DECODE = Decode("gqa_decode_b32_h32_hkv8_d128_len8k_32k_s16", 32, 32, 8, 128, 8192, 32768, 32768, 16, 5)

# Next steps on the same path ("Attention variants" §4 sliding window, with the
# window of Mistral-class models; a prompt chunk appended after a cache, the
# bottom-right causal case of "Attention mechanism evolution" KV-cache code).
SWA_PREFILL = Prefill("swa_prefill_b1_h32_hkv8_n16384_w4096_d128", 1, 32, 8, 16384, 16384, 128, True, "bf16", 6,
                      window=4096)
SWA_DECODE = Decode("swa_decode_b32_h32_hkv8_d128_len8k_32k_w4096_s1", 32, 32, 8, 128, 8192, 32768, 32768, 1, 5,
                    window=4096)
PAGED_DECODE = Decode("paged_decode_b32_h32_hkv8_d128_len8k_32k_p16_s16", 32, 32, 8, 128, 8192, 32768, 32768, 16, 5,
                      page_size=16)
FP8_DECODE = Decode("fp8_decode_b32_h32_hkv8_d128_len8k_32k_s16", 32, 32, 8, 128, 8192, 32768, 32768, 16, 5,
                    dtype="e4m3", k_scale=2.0 ** -6, v_scale=2.0 ** -6)
CHUNKED_PREFILL = Prefill("chunked_prefill_b4_h32_hkv8_q512_k8192_d128", 4, 32, 8, 512, 8192, 128, True, "bf16", 7)

PREFILL_WORKLOADS = (SINGLE_HEAD_F32, SINGLE_HEAD_F32_CAUSAL, MHA_PREFILL, GQA_PREFILL, MQA_PREFILL)


@dataclass
class PrefillData:
    spec: Prefill
    q: np.ndarray            # float32 or bf16 bits (uint16)
    k: np.ndarray
    v: np.ndarray
    extras: dict = field(default_factory=dict)


def prefill_inputs(spec: Prefill) -> PrefillData:
    """Q, K, V for a prefill workload, in its storage dtype."""
    qf = _normal_blocks(spec.seed, 0, spec.B, spec.H, (spec.N_q, spec.d))
    kf = _normal_blocks(spec.seed, 1, spec.B, spec.H_kv, (spec.N_k, spec.d))
    vf = _normal_blocks(spec.seed, 2, spec.B, spec.H_kv, (spec.N_k, spec.d))
    if spec.dtype == "f32":
        kf *= np.float32(spec.k_scale)
        return PrefillData(spec, qf, kf, vf)
    if spec.dtype != "bf16":
        raise ValueError(spec.dtype)
    q = f32_to_bf16_bits(qf)
    k = f32_to_bf16_bits(kf)
    v = f32_to_bf16_bits(vf)
    if spec.k_scale != 1.0:
        k = f32_to_bf16_bits(bf16_bits_to_f32(k) * np.float32(spec.k_scale))
    return PrefillData(spec, q, k, v)


@dataclass
class DecodeData:
    spec: Decode
    q: np.ndarray            # [B,H,d] bf16 bits
    k_cache: np.ndarray      # [B,H_kv,N_max,d] bf16 bits
    v_cache: np.ndarray
    seq_lens: np.ndarray     # [B] int32


def decode_seq_lens(spec: Decode) -> np.ndarray:
    rng = np.random.default_rng([spec.seed, 100])
    return rng.integers(spec.len_lo, spec.len_hi, size=spec.B, endpoint=True).astype(np.int32)


def decode_inputs(spec: Decode, pad: int | None = BF16_QNAN, seq_lens=None) -> DecodeData:
    """q, the two caches and seq_lens for a decode workload (bf16 storage).

    ``pad`` is the bf16 bit pattern written to cache rows at or beyond len_b
    (quiet NaN by default; None leaves zeros).  ``seq_lens`` overrides the
    drawn lengths (each in 1..N_max).
    """
    lens = decode_seq_lens(spec) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    if lens.shape != (spec.B,) or lens.min() < 1 or lens.max() > spec.N_max:
        raise ValueError("seq_lens must hold B values in 1..N_max")
    q = f32_to_bf16_bits(np.random.default_rng([spec.seed, 0]).standard_normal((spec.B, spec.H, spec.d),
                                                                              dtype=np.float32))
    caches = []
    for tag in (1, 2):
        f = _normal_blocks(spec.seed, tag, spec.B, spec.H_kv, (spec.N_max, spec.d), rows=lens)
        c = f32_to_bf16_bits(f)
        del f
        if pad is not None:
            for b in range(spec.B):
                c[b, :, int(lens[b]):, :] = pad
        caches.append(c)
    return DecodeData(spec, q, caches[0], caches[1], lens)


def decode_kv_bytes(spec: Decode, seq_lens=None) -> int:
    """Algorithmic KV bytes one decode step reads: sum_b 2*H_kv*len_b*d*2."""
    lens = decode_seq_lens(spec) if seq_lens is None else np.asarray(seq_lens)
    return int(2 * spec.H_kv * spec.d * 2 * int(np.sum(lens.astype(np.int64))))


# ---------------------------------------------------------------- paged caches
def page_table(seq_lens, page_size: int, seed: int, spare: int = 3):
    """A shuffled page assignment: (block_table [B, max_blocks] int32, num_pages).

    Sequence b needs ceil(len_b / page_size) pages; they are dealt from a seeded
    permutation of a pool with `spare` extra pages, so neighbouring logical
    blocks land on unrelated physical pages.  Unused table entries are -1.
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    need = [int((n + page_size - 1) // page_size) for n in lens]
    num_pages = sum(need) + spare
    order = np.random.default_rng([seed, 200]).permutation(num_pages)
    max_blocks = max(1, max(need))
    table = np.full((len(lens), max_blocks), -1, np.int32)
    pos = 0
    for b, nb in enumerate(need):
        table[b, :nb] = order[pos:pos + nb]
        pos += nb
    return table, num_pages


def to_pages(cache: np.ndarray, seq_lens, table: np.ndarray, num_pages: int, page_size: int, pad):
    """Copy rows [0, len_b) of a contiguous cache [B,H_kv,N,d] into a pool
    [num_pages,H_kv,page_size,d] following `table`; everything else is `pad`."""
    B, H_kv, N, d = cache.shape
    pool = np.full((num_pages, H_kv, page_size, d), pad, dtype=cache.dtype)
    for b, n in enumerate(np.asarray(seq_lens)):
        for blk in range((int(n) + page_size - 1) // page_size):
            r0, r1 = blk * page_size, min((blk + 1) * page_size, int(n))
            pool[table[b, blk], :, :r1 - r0] = cache[b, :, r0:r1]
    return pool


# ---------------------------------------------------------------- FP8 caches
E4M3_NAN = 0x7F


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """FP8 E4M3 codes of float32 values: round to nearest even, saturated at
    +-448 (torch's float8_e4m3fn cast does the rounding)."""
    import torch
    x = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def decode_inputs_fp8(spec: Decode, seq_lens=None) -> DecodeData:
    """q (bf16 bits) and FP8 E4M3 caches (codes of value / scale) for a decode
    workload; the same draws as decode_inputs, quantised per tensor.  Rows at or
    past a length hold the NaN code."""
    lens = decode_seq_lens(spec) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    if lens.shape != (spec.B,) or lens.min() < 1 or lens.max() > spec.N_max:
        raise ValueError("seq_lens must hold B values in 1..N_max")
    q = f32_to_bf16_bits(np.random.default_rng([spec.seed, 0]).standard_normal((spec.B, spec.H, spec.d),
                                                                              dtype=np.float32))
    caches = []
    for tag, sc in ((1, spec.k_scale), (2, spec.v_scale)):
        f = _normal_blocks(spec.seed, tag, spec.B, spec.H_kv, (spec.N_max, spec.d), rows=lens)
        f *= np.float32(1.0 / sc)
        c = f32_to_e4m3_codes(f)
        del f
        for b in range(spec.B):
            c[b, :, int(lens[b]):, :] = E4M3_NAN
        caches.append(c)
    return DecodeData(spec, q, caches[0], caches[1], lens)


# ---------------------------------------------------------------- tensors past 4 GiB
# A tensor of billions of elements is too large to draw on the host and to hand
# to the fp64 oracle whole.  Its rows repeat a short seeded table instead: row r
# of a block with shift s is table row (r + s) % period.  The period 8191 is
# 2^13 - 1, so 2^k = 2^(k mod 13) (mod 8191): moving 2^k rows (k >= 13) never
# lands on the same table row.  With 256-byte rows (d = 128, bf16) an address
# that wrapped at 2^31 or 2^32 bytes (2^23 or 2^24 rows) would read a row other
# than the right one, so the check of a sampled row catches it.
LARGE_PERIOD = 8191


def periodic_table(seed: int, tag: int, d: int, period: int = LARGE_PERIOD) -> np.ndarray:
    """bf16 bits [period, d]: the row table, N(0,1) rounded to bf16."""
    rng = np.random.default_rng([seed, tag, period])
    return f32_to_bf16_bits(rng.standard_normal((period, d), dtype=np.float32))


def periodic_rows(start: int, stop: int, shift: int, period: int = LARGE_PERIOD) -> np.ndarray:
    """Table row of each of the rows start .. stop-1 of a block with the given shift."""
    return (np.arange(start, stop, dtype=np.int64) + int(shift)) % period


def scattered_page_table(seq_lens, page_size: int, num_pages: int, seed: int) -> np.ndarray:
    """int32 [B, max_blocks] block table over a pool of num_pages pages, its
    distinct pages drawn (seeded) from the pool's first 64 pages, the 128 around
    page 2^16 and its last 512, so that a large pool is read near its start,
    around 2^16 pages and at its end.  Entries past a sequence's last block are -1."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    blocks = [(int(n) + page_size - 1) // page_size for n in lens]
    mid = 1 << 16
    cand = np.unique(np.concatenate([np.arange(0, 64), np.arange(mid - 64, mid + 64),
                                     np.arange(num_pages - 512, num_pages)]))
    cand = cand[(cand >= 0) & (cand < num_pages)]
    if sum(blocks) > cand.size:
        raise ValueError("pool too small for the sequences")
    pick = np.random.default_rng([seed, 9]).permutation(cand)[:sum(blocks)]
    table = np.full((len(lens), max(blocks)), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(blocks):
        table[b, :n] = pick[at:at + n]
        at += n
    return table
