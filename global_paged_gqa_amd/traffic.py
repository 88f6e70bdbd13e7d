"""Algorithmic work of one call, for roofline figures (counting only, no attention math).

Decode: every visible key's K (and V unless shared) is read once:
    bytes = sum over rows and KV heads of n_visible * head_dim * e B * (1 if K=V else 2),
    e = 2 for bf16 pools, 1 for FP8 (E4M3) pools.
Prefill: flops = sum over visible (query, key) pairs of 4 * head_dim * num_q_heads
    (QK^T and PV, two flops per multiply-add, masked or skipped pairs not counted).
A query at position p sees p + 1 keys (global) or min(p + 1, window) keys (local).
"""
import numpy as np


def kv_bytes_per_token(layers, bytes_per_elem: int = 2) -> int:
    """Cache bytes one token of context occupies: sum over (num_kv_heads, head_dim, kv_shared) layers."""
    return sum(hkv * hd * (1 if shared else 2) * bytes_per_elem for hkv, hd, shared in layers)


def n_visible(is_global: bool, window: int, pos) -> np.ndarray:
    pos = np.asarray(pos, dtype=np.int64)
    return pos + 1 if is_global else np.minimum(pos + 1, window)


def decode_kv_bytes(is_global, window, num_kv_heads, head_dim, kv_shared, ctx_lens, elem_bytes: int = 2) -> int:
    n = int(n_visible(is_global, window, np.asarray(ctx_lens, np.int64) - 1).sum())
    return n * num_kv_heads * head_dim * elem_bytes * (1 if kv_shared else 2)


def prefill_flops(is_global, window, num_q_heads, head_dim, ctx_lens, q_lens) -> int:
    total = 0
    for L, C in zip(np.asarray(ctx_lens, np.int64), np.asarray(q_lens, np.int64)):
        if C > 0:
            total += int(n_visible(is_global, window, np.arange(L - C, L)).sum())
    return total * 4 * head_dim * num_q_heads
