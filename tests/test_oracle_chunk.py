"""CPU pins of the oracle's chunked prefill against a KV cache.

The chunk function is pinned to the whole-sequence prefill (itself pinned by
the golden examples and the loop oracle): chunk row i of sequence b must equal
row L_b + i of a prefill over the whole sequence, with the cache holding the
K-hat and V of the first L_b tokens. A wrong key offset, mask index or default
position breaks these equalities.
"""
import numpy as np
import pytest

from oracle import attention as oracle

RMS_EPS, BASE = 1e-6, 10000.0


def _inputs(B, T, H, G, d, gate_mode, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, G, d))
    v = rng.standard_normal((B, T, G, d))
    gate = {"elementwise": rng.standard_normal((B, T, H, d)), "headwise": rng.standard_normal((B, T, H)),
            "none": None}[gate_mode]
    wq = 1.0 + 0.1 * rng.standard_normal(d)
    wk = 1.0 + 0.1 * rng.standard_normal(d)
    return q, k, v, gate, wq, wk


@pytest.mark.parametrize("gate_mode", ["elementwise", "headwise", "none"])
def test_chunk_rows_equal_whole_sequence_prefill(gate_mode):
    B, T, H, G, d, rot = 3, 21, 4, 2, 16, 4
    q, k, v, gate, wq, wk = _inputs(B, T, H, G, d, gate_mode, seed=11)
    pos = np.tile(np.arange(T), (B, 1))
    full = oracle.prefill(q, k, v, gate, gate_mode=gate_mode, q_norm_w=wq, k_norm_w=wk, positions=pos,
                          rms_eps=RMS_EPS, rope_base=BASE, rot_dim=rot).reshape(B, T, H, d)
    khat_full = oracle.prefill_keys(k, wk, pos, rms_eps=RMS_EPS, rope_base=BASE, rot_dim=rot)
    L = np.array([8, 0, 20])
    n = int((T - L).max())
    lens = T - L

    def chunk(x):  # rows L_b .. T-1 of each sequence, zero padding after
        if x is None:
            return None
        c = np.zeros((B, n) + x.shape[2:])
        for b in range(B):
            c[b, :lens[b]] = x[b, L[b]:]
        return c

    out, kh = oracle.prefill_chunk(chunk(q), chunk(k), chunk(v), chunk(gate), gate_mode=gate_mode, q_norm_w=wq,
                                   k_norm_w=wk, k_cache_rows=lambda b: (khat_full[b, :L[b]], v[b, :L[b]]),
                                   cache_lens=L, chunk_lens=lens, rms_eps=RMS_EPS, rope_base=BASE, rot_dim=rot)
    out = out.reshape(B, n, H, d)
    for b in range(B):
        np.testing.assert_allclose(out[b, :lens[b]], full[b, L[b]:], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(kh[b, :lens[b]], khat_full[b, L[b]:], rtol=1e-12, atol=1e-12)
        assert np.all(np.isnan(out[b, lens[b]:]))


def test_chunk_with_empty_cache_is_prefill():
    B, n, H, G, d, rot = 2, 13, 4, 1, 8, 2
    q, k, v, gate, wq, wk = _inputs(B, n, H, G, d, "elementwise", seed=12)
    pos = np.tile(np.arange(n), (B, 1))
    want = oracle.prefill(q, k, v, gate, gate_mode="elementwise", q_norm_w=wq, k_norm_w=wk, positions=pos,
                          rms_eps=RMS_EPS, rope_base=BASE, rot_dim=rot)
    empty = (np.zeros((0, G, d)), np.zeros((0, G, d)))
    got, _ = oracle.prefill_chunk(q, k, v, gate, gate_mode="elementwise", q_norm_w=wq, k_norm_w=wk,
                                  k_cache_rows=lambda b: empty, cache_lens=np.zeros(B, np.int64), rms_eps=RMS_EPS,
                                  rope_base=BASE, rot_dim=rot)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_chunk_default_positions_follow_the_cache():
    B, n, H, G, d, rot = 2, 5, 2, 1, 8, 8
    q, k, v, gate, wq, wk = _inputs(B, n, H, G, d, "headwise", seed=13)
    L = np.array([3, 9])
    rng = np.random.default_rng(14)
    cache = [(rng.standard_normal((L[b], G, d)), rng.standard_normal((L[b], G, d))) for b in range(B)]
    kw = dict(gate_mode="headwise", q_norm_w=wq, k_norm_w=wk, k_cache_rows=lambda b: cache[b], cache_lens=L,
              rms_eps=RMS_EPS, rope_base=BASE, rot_dim=rot)
    a, ka = oracle.prefill_chunk(q, k, v, gate, **kw)
    b_, kb = oracle.prefill_chunk(q, k, v, gate, positions=L[:, None] + np.arange(n)[None, :], **kw)
    np.testing.assert_array_equal(a, b_)
    np.testing.assert_array_equal(ka, kb)
    # and positions do matter (rot = d: every dimension is rotated)
    c, _ = oracle.prefill_chunk(q, k, v, gate, positions=np.zeros((B, n), np.int64), **kw)
    assert np.abs(c - a).max() > 1e-3


def test_chunk_skips_invalid_sequences_and_padding():
    B, n, H, G, d = 3, 4, 2, 1, 8
    q, k, v, gate, wq, wk = _inputs(B, n, H, G, d, "none", seed=15)
    L = np.array([2, 7, 1])
    cache = lambda b: (np.ones((L[b], G, d)), np.ones((L[b], G, d)))
    out, kh = oracle.prefill_chunk(q, k, v, None, gate_mode="none", q_norm_w=wq, k_norm_w=wk, k_cache_rows=cache,
                                   cache_lens=L, chunk_lens=np.array([4, 4, 0]), max_cache_len=5, rms_eps=RMS_EPS)
    assert np.all(np.isfinite(out[0]))
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(kh[1]))   # L = 7 > max_cache_len
    assert np.all(np.isnan(out[2]))                                 # no real rows
