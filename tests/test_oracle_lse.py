"""Pins of the oracle's row log-sum-exp (oracle.attention.prefill_row_lse),
the statistic the training forward saves for the backward: a closed form, an
independent brute force over Python floats, and the invariant that ties it
to the already pinned prefill (the probabilities it defines sum to one and
reproduce the attention output)."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import loops as L
from tests.test_oracle_pins import _rand_case


def test_zero_query_gives_log2_of_the_visible_key_count():
    """q = 0: every score is 0, so row i sums exp(0) over its i + 1 keys."""
    q, k, _, _, wq, wk, pos = _rand_case(21, B=2, n=9, H=4, G=2, d=8, rot=4)
    lse = A.prefill_row_lse(np.zeros_like(q), k, q_norm_w=wq, k_norm_w=wk, positions=pos, rot_dim=4)
    want = np.log2(np.arange(1, 10, dtype=np.float64))[None, :, None]
    assert np.allclose(lse, np.broadcast_to(want, lse.shape), atol=1e-12, rtol=0)


def test_identical_keys_add_the_score_to_the_count():
    """Every key equal (no RoPE, so k-hat is the same for all j): s_ij = c_i for
    j <= i and lse_i = c_i / ln 2 + log2(i + 1)."""
    rng = np.random.default_rng(22)
    B, n, H, G, d = 1, 6, 2, 1, 8
    q = rng.standard_normal((B, n, H, d))
    k = np.broadcast_to(rng.standard_normal(d), (B, n, G, d)).copy()
    pos = np.broadcast_to(np.arange(n), (B, n))
    lse = A.prefill_row_lse(q, k, q_norm_w=None, k_norm_w=None, positions=pos, rot_dim=0, scale=0.5)
    for i in range(n):
        for h in range(H):
            c = float(q[0, i, h] @ k[0, 0, 0]) * 0.5
            assert abs(lse[0, i, h] - (c / math.log(2.0) + math.log2(i + 1))) < 1e-12


@pytest.mark.parametrize("seed,B,n,H,G,d,rot", [(23, 1, 5, 2, 1, 4, 4), (24, 2, 7, 4, 2, 8, 2), (25, 1, 6, 6, 3, 8, 0)])
def test_matches_bruteforce_loops(seed, B, n, H, G, d, rot):
    """Scores from the brute force's own norm and rotation (Python floats),
    summed with math.fsum; positions start away from zero."""
    q, k, _, _, wq, wk, pos = _rand_case(seed, B, n, H, G, d, rot)
    pos = pos + 5
    got = A.prefill_row_lse(q, k, q_norm_w=wq, k_norm_w=wk, positions=pos, rot_dim=rot)
    grp = H // G
    sc = 1.0 / math.sqrt(d)
    for b in range(B):
        kh = [[L._rotated(L._normed(k[b, j, g].tolist(), wk.tolist(), 1e-6), int(pos[b, j]), rot, 10000.0)
               for g in range(G)] for j in range(n)]
        for i in range(n):
            for h in range(H):
                qh = L._rotated(L._normed(q[b, i, h].tolist(), wq.tolist(), 1e-6), int(pos[b, i]), rot, 10000.0)
                s = [math.fsum(a * c for a, c in zip(qh, kh[j][h // grp])) * sc for j in range(i + 1)]
                want = math.log2(math.fsum(math.exp(x) for x in s))
                assert abs(got[b, i, h] - want) < 1e-12, (b, i, h)


def test_probabilities_sum_to_one_and_reproduce_the_prefill():
    """P_ij = 2^(s_ij log2 e - lse_i) over j <= i: rows sum to one and P V is
    the ungated prefill output (prefill is pinned to the pages' examples);
    a sampled-rows call returns the same values as the full one."""
    B, n, H, G, d, rot = 2, 11, 4, 2, 8, 4
    q, k, v, _, wq, wk, pos = _rand_case(26, B, n, H, G, d, rot, A.GATE_NONE)
    kw = dict(q_norm_w=wq, k_norm_w=wk, positions=pos, rot_dim=rot)
    lse = A.prefill_row_lse(q, k, **kw)
    y = A.prefill(q, k, v, None, gate_mode=A.GATE_NONE, **kw).reshape(B, n, H, d)
    qh = A.rope(A.rms_norm(q, wq, 1e-6), pos, rot, 10000.0)
    kh = A.prefill_keys(k, wk, pos, rms_eps=1e-6, rope_base=10000.0, rot_dim=rot)
    for b in range(B):
        for h in range(H):
            g = A.kv_group(h, H, G)
            for i in range(n):
                s = kh[b, :i + 1, g] @ qh[b, i, h] / math.sqrt(d)
                p = np.exp2(s * math.log2(math.e) - lse[b, i, h])
                assert abs(p.sum() - 1.0) < 1e-12
                assert np.allclose(p @ v[b, :i + 1, g], y[b, i, h], atol=1e-12, rtol=0)
    rows = [(0, 0, 0), (1, 10, 3), (0, 5, 2)]
    part = A.prefill_row_lse(q, k, rows=rows, **kw)
    assert np.array_equal(part, np.array([lse[r] for r in rows]))
