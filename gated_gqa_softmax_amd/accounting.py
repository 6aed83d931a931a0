"""Algorithmic work of the hot path: flops for prefill, HBM bytes for decode.

These are the figures throughput and roofline fractions are computed from.
They count what the method must do, not what a given kernel happens to move.
"""
from __future__ import annotations

import numpy as np


def causal_prefill_flops(batch: int, n_q_heads: int, head_dim: int, seq_len: int) -> float:
    """2*B*H*d*n*(n+1): 2d flops for q.k and 2d for the value mix, per visible
    (i, j <= i) pair per query head. Norm, rotation, exp and gate are excluded."""
    return 2.0 * batch * n_q_heads * head_dim * seq_len * (seq_len + 1)


def causal_backward_flops(batch: int, n_q_heads: int, head_dim: int, seq_len: int) -> float:
    """Backward of the causal prefill: five products per visible (i, j <= i)
    pair per query head (q.k again, dy.v, P^T dy, dS^T q, dS k), 2d flops each:
    2.5 times ``causal_prefill_flops``. Recomputing the forward's softmax
    statistics, the gate, norm and rotation backward are excluded."""
    return 2.5 * causal_prefill_flops(batch, n_q_heads, head_dim, seq_len)


def chunk_prefill_flops(cache_lens, n_q_heads: int, head_dim: int, chunk_len: int) -> float:
    """Chunked prefill: row i of sequence b sees L_b + i + 1 keys, so
    sum_b 2*H*d*(2*n*L_b + n*(n+1)) (the whole-sequence formula when L_b = 0)."""
    n = chunk_len
    return float(sum(2.0 * n_q_heads * head_dim * (2.0 * n * int(L) + n * (n + 1)) for L in cache_lens))


def kv_numbers_per_token(n_kv_heads: int, head_dim: int) -> int:
    """Cached numbers per token per full-attention layer: 2 (K and V) * G * d."""
    return 2 * n_kv_heads * head_dim


def kv_cache_bytes(tokens: int, layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    return tokens * layers * kv_numbers_per_token(n_kv_heads, head_dim) * elem_bytes


def decode_bytes(cache_lens, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 elem_bytes: int = 2, gate_mode: str = "elementwise") -> int:
    """HBM bytes one decode step must move.

    Every cached K-hat row and V row of every sequence is read once
    (sum_b L_b * 2 * G * d elements); per sequence the step also reads q, the
    gate logits, k_new and v_new, writes the gated output and appends one
    K-hat row and one V row to the cache.
    """
    lens = np.asarray(cache_lens, dtype=np.int64)
    B = lens.size
    H, G, d = n_q_heads, n_kv_heads, head_dim
    cache = int(lens.sum()) * 2 * G * d * elem_bytes
    gate = {"elementwise": H * d, "headwise": H, "none": 0}[gate_mode]
    per_seq = (H * d            # q
               + gate           # gate logits
               + 2 * G * d      # k_new, v_new
               + H * d          # out
               + 2 * G * d      # appended K-hat and V slot
               ) * elem_bytes
    return cache + B * per_seq
