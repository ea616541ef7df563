"""Algorithmic work model and MI355X peaks used to express measured rates as roofline fractions.

Counting rules:
  * prefill FLOPs = 4 * d * H_q * (number of valid (query row, key) pairs per
    head): 2*d for the score dot product and 2*d for the weighted sum of V per
    valid pair; softmax work is not counted (the usual attention convention);
    masked-tile waste and K/V re-reads count in the time, never in the work.
  * decode bytes = the valid K and V cache rows (the KV-cache size model of the
    azimuth.plus GQA digest, "KV cache size" formula 2 * L * G * d_k * n, taken
    for one layer, G = H_kv groups and n = each sequence's valid length) plus
    the query and output vectors. Split partials and the combine pass count in
    the time, not in the bytes.
"""
from __future__ import annotations

from typing import Optional, Sequence

# Published MI355X peaks (dense, no sparsity).
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0

ESIZE = {"bf16": 2, "f32": 4}


def kv_cache_bytes(layers: int, groups: int, d_k: int, n_tokens: int, esize: int) -> int:
    """K/V cache size: 2 (K and V) x layers x K/V groups x head size x tokens x element size."""
    return 2 * layers * groups * d_k * n_tokens * esize


def kv_cache_reduction(h_q: int, groups: int) -> float:
    """Cache shrink factor of GQA-G against MHA with H_q K/V heads (= H_q / G)."""
    return h_q / groups


def prefill_valid_pairs(B: int, S: int, causal: bool, seqlens: Optional[Sequence[int]],
                        window: int = 0) -> int:
    """Valid (query row, key) pairs per head summed over the batch.

    Key j is valid for query i iff j < L_b, (not causal or j <= i) and (window == 0 or
    j > i - window); every query row i < S counts.
    """
    total = 0
    for b in range(B):
        L = S if seqlens is None else max(0, min(int(seqlens[b]), S))
        if window > 0:
            for i in range(S):
                hi = min(L, i + 1) if causal else L
                total += max(0, hi - max(0, i - window + 1))
        elif causal:
            # rows i < L see i + 1 keys; rows i >= L see L keys
            total += L * (L + 1) // 2 + (S - L) * L
        else:
            total += S * L
    return total


def prefill_flops(B: int, S: int, Hq: int, d: int, causal: bool,
                  seqlens: Optional[Sequence[int]], window: int = 0) -> int:
    return 4 * d * Hq * prefill_valid_pairs(B, S, causal, seqlens, window)


def decode_bytes(B: int, Hq: int, Hkv: int, d: int, lens: Sequence[int], max_len: int,
                 esize: int, window: int = 0) -> int:
    """Valid K/V rows read (the last `window` of each sequence when window > 0) plus q and o."""
    def keys(x):
        L = max(0, min(int(x), max_len))
        return min(L, window) if window > 0 else L
    total_len = sum(keys(x) for x in lens)
    cache = kv_cache_bytes(1, Hkv, d, total_len, esize)
    return cache + 2 * B * Hq * d * esize


def mean_pool_bytes(H: int, G: int, per_head: int, esize: int) -> int:
    """MHA -> GQA conversion traffic: every input element read once, every output written once."""
    return (H + G) * per_head * esize


def decode_flops(Hq: int, d: int, lens: Sequence[int], max_len: int) -> int:
    total_len = sum(max(0, min(int(x), max_len)) for x in lens)
    return 4 * d * Hq * total_len
