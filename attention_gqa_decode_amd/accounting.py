"""Algorithmic byte and FLOP counts used to express measured times as rooflines.

KV-cache size per token follows the lecture page "추론 최적화" (base.kaita.kr), section 2
(K and V per layer and head: 2 x layers x kv_heads x head_dim x bytes), whose exercises
work it out for a 32-layer model.  Decode bytes are the bytes a decode step must move at
least once: every cached K and V row of every request, the query, and the output.
Prefill FLOPs count the causal (unmasked) half only: 4 x Hsz FLOPs per (query row,
visible key) pair (2 for QK^T, 2 for PV).
"""
from __future__ import annotations


def kv_cache_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def decode_bytes(seqlens, B: int, Hq: int, KH: int, Hsz: int, in_bytes: int = 2, out_bytes: int = 4,
                 kv_bytes: int | None = None) -> int:
    """Bytes a decode step must move: K and V of every cached token (kv_bytes per element,
    default in_bytes), the query (in_bytes) and the output (out_bytes)."""
    kvb = in_bytes if kv_bytes is None else kv_bytes
    kv = sum(2 * KH * int(L) * Hsz * kvb for L in seqlens)
    return kv + B * Hq * Hsz * in_bytes + B * Hq * Hsz * out_bytes


def decode_flops(seqlens, Hq: int, Hsz: int) -> int:
    return sum(4 * Hq * Hsz * int(L) for L in seqlens)


def prefill_causal_flops(B: int, ISL: int, Hq: int, Hsz: int) -> int:
    return 4 * Hsz * Hq * B * ISL * (ISL + 1) // 2


def prefill_bytes(B: int, ISL: int, Hq: int, KH: int, Hsz: int) -> int:
    return 2 * B * ISL * Hsz * (2 * Hq + 2 * KH)  # q and out (bf16), k and v (bf16)
