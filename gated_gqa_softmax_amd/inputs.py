"""Seeded synthetic inputs for gated GQA causal attention.

This module is the ONLY code shared by the CPU oracle and the HIP path. It
draws random numbers and rounds them to the storage format; it holds none of
the attention arithmetic (no norm, rotation, softmax or gate).

Recipe (every workload uses ``numpy.random.default_rng``, PCG64):

* prefill: ``rng = default_rng(seed)`` draws, in this order, q ``[B,n,H,d]``,
  k ``[B,n,G,d]``, v ``[B,n,G,d]`` (all N(0,1)), the gate logits
  (N(0,1.5): ``[B,n,H,d]`` elementwise, ``[B,n,H]`` headwise), then the
  q-norm and k-norm weight noise (weights = 1 + 0.02 N(0,1), shape ``[d]``).
  Positions are ``arange(n)`` for every sequence.
* decode: ``rng = default_rng(seed)`` draws the cache lengths
  (uniform integers in ``[lo, hi]``), q ``[B,H,d]``, k_new, v_new ``[B,G,d]``,
  the gate logits, then the two weight noises. Each sequence's cache rows are
  drawn from their own stream ``default_rng([seed, b])``: K-hat rows
  ``[L_b,G,d]`` then V rows ``[L_b,G,d]``, all N(0,1), so one sequence can be
  regenerated without drawing the others.

"N(0,s)" means standard deviation s. bf16 workloads round every tensor except
the norm weights to the nearest bf16 value (round-to-nearest-even) and keep it
in a float32 array, so both sides read exactly the same numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

GATE_NONE = "none"
GATE_HEADWISE = "headwise"
GATE_ELEMENTWISE = "elementwise"


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str              # "prefill" or "decode"
    batch: int
    seq_len: int           # prefill tokens per sequence (decode: 1 new token)
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rot_dim: int
    dtype: str             # "bf16" or "f32"
    gate_mode: str
    seed: int
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    gate_std: float = 1.5
    weight_std: float = 0.02
    cache_len_lo: int = 0
    cache_len_hi: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The synthetic workloads (shapes taken from the pages' models: a toy,
# Qwen3.5-0.8B's 8/2/256, Qwen3-0.6B's 16/8/128, the paper's MoE 32/4/128 at
# 32K tokens, a decode batch over a long cache, and chunked prefill of the
# Qwen3.5-0.8B shape: four 1024-token chunks after 0, 1024, 2048 and 3072
# cached tokens).
WORKLOADS = {
    "toy": Workload("toy", "prefill", 1, 16, 2, 1, 8, 2, "f32", GATE_ELEMENTWISE, seed=1),
    "qwen35_0p8b_prefill": Workload("qwen35_0p8b_prefill", "prefill", 1, 4096, 8, 2, 256, 64,
                                    "bf16", GATE_ELEMENTWISE, seed=2),
    "qwen3_0p6b_batched_prefill": Workload("qwen3_0p6b_batched_prefill", "prefill", 4, 2048, 16, 8,
                                           128, 32, "bf16", GATE_HEADWISE, seed=3),
    "moe_long_context_prefill": Workload("moe_long_context_prefill", "prefill", 1, 32768, 32, 4,
                                         128, 32, "bf16", GATE_ELEMENTWISE, seed=4),
    "decode_64seq": Workload("decode_64seq", "decode", 64, 1, 8, 2, 256, 64, "bf16",
                             GATE_ELEMENTWISE, seed=5, cache_len_lo=1024, cache_len_hi=32768),
    "qwen35_0p8b_chunk": Workload("qwen35_0p8b_chunk", "prefill", 4, 1024, 8, 2, 256, 64, "bf16",
                                  GATE_ELEMENTWISE, seed=6, extra={"cache_lens": [0, 1024, 2048, 3072]}),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); float32 out.

    NaN stays NaN; finite values beyond the bf16 range round to infinity.
    """
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    nan = np.isnan(x)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    if nan.any():
        x[nan] = np.float32("nan")
    return x


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x)


def _normal(rng, shape, std=1.0):
    return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)


def gate_shape(w: Workload, lead: tuple) -> Optional[tuple]:
    if w.gate_mode == GATE_ELEMENTWISE:
        return lead + (w.n_q_heads, w.head_dim)
    if w.gate_mode == GATE_HEADWISE:
        return lead + (w.n_q_heads,)
    return None


def make_prefill(w: Workload, q_scale: float = 1.0) -> dict:
    """Draw one prefill workload. ``q_scale`` multiplies q after drawing."""
    B, n, H, G, d = w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim
    rng = np.random.default_rng(w.seed)
    q = _normal(rng, (B, n, H, d)) * np.float32(q_scale)
    k = _normal(rng, (B, n, G, d))
    v = _normal(rng, (B, n, G, d))
    gs = gate_shape(w, (B, n))
    gate = _normal(rng, gs, w.gate_std) if gs is not None else None
    w_q = (1.0 + _normal(rng, (d,), w.weight_std)).astype(np.float32)
    w_k = (1.0 + _normal(rng, (d,), w.weight_std)).astype(np.float32)
    pos = np.broadcast_to(np.arange(n, dtype=np.int32), (B, n)).copy()
    return dict(q=_store(q, w.dtype), k=_store(k, w.dtype), v=_store(v, w.dtype),
                gate=None if gate is None else _store(gate, w.dtype),
                q_norm_w=w_q, k_norm_w=w_k, positions=pos)


def make_decode(w: Workload, cache_lens: Optional[np.ndarray] = None) -> dict:
    """Draw the per-step decode tensors and the cache lengths (not the cache)."""
    B, H, G, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    rng = np.random.default_rng(w.seed)
    lens = rng.integers(w.cache_len_lo, w.cache_len_hi, endpoint=True, size=B).astype(np.int32)
    if cache_lens is not None:
        lens = np.asarray(cache_lens, dtype=np.int32).copy()
    q = _normal(rng, (B, H, d))
    k_new = _normal(rng, (B, G, d))
    v_new = _normal(rng, (B, G, d))
    gs = gate_shape(w, (B,))
    gate = _normal(rng, gs, w.gate_std) if gs is not None else None
    w_q = (1.0 + _normal(rng, (d,), w.weight_std)).astype(np.float32)
    w_k = (1.0 + _normal(rng, (d,), w.weight_std)).astype(np.float32)
    return dict(q=_store(q, w.dtype), k_new=_store(k_new, w.dtype), v_new=_store(v_new, w.dtype),
                gate=None if gate is None else _store(gate, w.dtype),
                q_norm_w=w_q, k_norm_w=w_k, cache_lens=lens)


def decode_cache_rows(w: Workload, b: int, length: int) -> tuple:
    """Cache rows of sequence ``b``: (K-hat [length,G,d], V [length,G,d])."""
    rng = np.random.default_rng([w.seed, b])
    kh = _normal(rng, (length, w.n_kv_heads, w.head_dim))
    vv = _normal(rng, (length, w.n_kv_heads, w.head_dim))
    return _store(kh, w.dtype), _store(vv, w.dtype)


def for_each_cache_rows(w: Workload, cache_lens, fn, threads: int = 8) -> None:
    """Call ``fn(b, k_hat_rows, v_rows)`` for every sequence, drawing the
    sequences' streams on a thread pool (the draws are independent)."""
    from concurrent.futures import ThreadPoolExecutor

    def job(b):
        return b, decode_cache_rows(w, b, int(cache_lens[b]))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        for b, (kh, vv) in ex.map(job, range(w.batch)):
            fn(b, kh, vv)


def sample_row_blocks(w: Workload, count: int = 16, rows: int = 256, seed: int = 7) -> list:
    """Seeded sample of query-row blocks for workloads too large to check or
    time on the CPU whole: ``count`` distinct block starts (multiples of
    ``rows``), sorted, the last block always included."""
    nblk = -(-w.seq_len // rows)
    if count >= nblk:
        return [i * rows for i in range(nblk)]
    pick = np.random.default_rng(seed).choice(nblk - 1, count - 1, replace=False)
    return sorted(int(p) * rows for p in pick) + [(nblk - 1) * rows]
