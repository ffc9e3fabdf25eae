"""Work and byte accounting for the benchmark, and the MI355X peaks it is priced against.

Peaks are AMD's published MI355X figures (not from the pages):
  * dense bf16 MFMA: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz = 2516.6 TFLOP/s (quoted as 2.5 PFLOP/s);
  * HBM3E: 8 TB/s.

Algorithmic work follows the attention cost model of "Attention variants:
GQA/MQA/FlashAttention" (youngju.dev) §1: QK^T and the weighted sum over V
each cost 2*B*H*N_q*N_k*d FLOPs; with the causal block skip of §5.5 about
half of the pairs remain, so the causal figure is halved.  Decode bytes are
the key and value rows a step must read (§7: decode re-reads the cache).
"""
from __future__ import annotations

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12   # 2516.58
PEAK_HBM_GBPS = 8000.0


def attention_flops(B: int, H: int, N_q: int, N_k: int, d: int, causal: bool) -> float:
    """4*B*H*N_q*N_k*d, halved when causal."""
    f = 4.0 * B * H * N_q * N_k * d
    return f / 2 if causal else f


def prefill_bytes(B: int, H: int, H_kv: int, N_q: int, N_k: int, d: int, elem: int = 2) -> int:
    """Read Q, K, V once; write O (elem bytes each) and the fp32 LSE."""
    q_and_o = 2 * B * H * N_q * d
    k_and_v = 2 * B * H_kv * N_k * d
    return (q_and_o + k_and_v) * elem + B * H * N_q * 4


def decode_kv_bytes(H_kv: int, d: int, seq_lens, elem: int = 2) -> int:
    """K and V rows one decode step reads: sum_b 2 * H_kv * len_b * d * elem."""
    return int(sum(2 * H_kv * int(n) * d * elem for n in seq_lens))


# ---- size formulas the pages print worked examples for ----------------------
def score_matrix_bytes(B: int, H: int, N: int, elem: int) -> int:
    """One (B, H, N, N) score tensor ("Attention variants" §1)."""
    return B * H * N * N * elem


def kv_cache_bytes(L: int, N: int, D: int, B: int, elem: int) -> int:
    """2 x L x N x D x B x bytes ("Attention variants" §1; 2 = K and V)."""
    return 2 * L * N * D * B * elem


def kv_cache_bytes_gqa(L: int, N: int, D: int, B: int, elem: int, H: int, G: int) -> float:
    """KV cache with G of H key/value heads kept ("Attention variants" §2, §6)."""
    return kv_cache_bytes(L, N, D, B, elem) * G / H


def layer_kv_bytes(S: int, D: int, elem: int) -> int:
    """2 x S x D x sizeof per layer ("Attention mechanism evolution", MHA box)."""
    return 2 * S * D * elem


def kv_head_fraction(H: int, G: int) -> float:
    return G / H
