"""Pins of the CPU oracle against values the pages print and exact special cases.

Each test names the page and section its numbers come from (the fixtures in
tests/golden carry the same citation).
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from tests.conftest import load_golden


def _r(x, nd):
    return np.round(np.asarray(x, dtype=np.float64), nd)


# -- "Transformer by Hand · 6. Gated attention": three tokens by hand --------

def _three_token_prefill(gate=None, gate_mode=A.GATE_NONE, queries=None):
    g = load_golden("three_token_example.json")
    q = np.array(queries if queries is not None else g["queries"])[None, :, None, :]   # [1,3,1,2]
    k = np.array(g["keys"])[None, :, None, :]
    v = np.array(g["values"])[None, :, None, :]
    pos = np.arange(3)[None]
    return g, A.prefill(q, k, v, gate, gate_mode=gate_mode, q_norm_w=None, k_norm_w=None,
                        positions=pos, rot_dim=0)


def test_three_token_scores_weights_output():
    g = load_golden("three_token_example.json")
    q = np.array(g["queries"][2])
    k = np.array(g["keys"])
    scores = k @ q / math.sqrt(2)
    assert list(_r(scores, 2)) == g["row2_scores_2dp"]
    _, a = A.causal_attention(np.array(g["queries"]), k, np.array(g["values"]), 1 / math.sqrt(2),
                              return_weights=True)
    assert list(_r(a[2], 3)) == g["row2_weights_3dp"]
    _, out = _three_token_prefill()
    assert list(_r(out[0, 2], 3)) == g["row2_output_3dp"]
    # fp64 value of the page's rounded (0.277, 1.723)
    assert out[0, 2, 0] == pytest.approx(0.27747, abs=5e-5)


def test_three_token_causal_matrix():
    g = load_golden("three_token_example.json")
    _, a = A.causal_attention(np.array(g["queries"]), np.array(g["keys"]), np.array(g["values"]),
                              1 / math.sqrt(2), return_weights=True)
    assert _r(a, 3).tolist() == g["causal_weights_3dp"]
    assert np.allclose(a.sum(-1), 1.0)


def test_zero_query_uniform_then_gate_minus_six():
    g = load_golden("three_token_example.json")
    # Row 2 sees all three keys; a zero query gives uniform weights.
    zq = [[0.0, 0.0], [0.0, 0.0], [0.0, 0.0]]
    _, out = _three_token_prefill(queries=zq)
    assert list(_r(out[0, 2], 3)) == g["zero_query_output_3dp"]
    _, a = A.causal_attention(np.zeros((3, 2)), np.array(g["keys"]), np.array(g["values"]),
                              1 / math.sqrt(2), return_weights=True)
    assert list(_r(a[2], 3)) == g["zero_query_weights_3dp"]
    gate = np.full((1, 3, 1), g["gate_logit"])      # headwise: one logit per token per head
    _, gout = _three_token_prefill(gate=gate, gate_mode=A.GATE_HEADWISE, queries=zq)
    assert round(float(A.sigmoid(np.array([g["gate_logit"]]))[0]), 4) == g["gate_value_4dp"]
    assert list(_r(gout[0, 2], 4)) == g["gated_zero_query_output_4dp"]


# -- "Attention, worked all the way through": the 2x2 known-answer figure ----

def test_two_by_two_fp32_digits_and_fp64():
    g = load_golden("two_by_two_known_answer.json")
    Q, K, V = (np.array(g[x]) for x in ("Q", "K", "V"))
    o32, a32 = A.causal_attention(Q, K, V, 1 / math.sqrt(2), dtype=np.float32, return_weights=True)
    # The figure prints float32 results with 8 significant digits.
    for got, want in ((a32, g["A"]), (o32, g["O"])):
        for x, y in zip(np.ravel(got), np.ravel(want)):
            assert float(f"{x:.8g}") == y
    o64, a64 = A.causal_attention(Q, K, V, 1 / math.sqrt(2), return_weights=True)
    assert np.allclose(a64, g["A"], atol=2e-8, rtol=0)
    assert np.allclose(o64, g["O"], atol=5e-7, rtol=0)
    # Same numbers through the full prefill path (norm and RoPE off).
    out = A.prefill(Q[None, :, None], K[None, :, None], V[None, :, None], None, gate_mode=A.GATE_NONE,
                    q_norm_w=None, k_norm_w=None, positions=np.arange(2)[None], rot_dim=0)
    assert np.allclose(out[0], o64, atol=0, rtol=0)


# -- gate pins ---------------------------------------------------------------

def test_sigmoid_points():
    g = load_golden("gate_examples.json")["sigmoid_points"]
    assert list(_r(A.sigmoid(np.array(g["z"])), 4)) == g["g_4dp"]
    assert A.sigmoid(np.array([0.0]))[0] == 0.5
    assert A.sigmoid(np.array([100.0]))[0] == 1.0
    # both branches agree with the textbook logistic away from overflow
    z = np.linspace(-30, 30, 61)
    assert np.allclose(A.sigmoid(z), 1 / (1 + np.exp(-z)), rtol=1e-15, atol=0)


def test_gate_toy():
    g = load_golden("gate_examples.json")["gate_toy"]
    W = np.array(g["W_gate"])
    for word in ("book", "she"):
        z = np.array(g["x"][word]) @ W                         # the caller's projection
        assert list(_r(z, 1)) == g["z_1dp"][word]
        zz = z.reshape(2, 2)                                   # 2 heads x 2 dims
        heads = np.array(g["heads"][word])
        gated = A.apply_gate(heads, zz, A.GATE_ELEMENTWISE)
        assert _r(A.sigmoid(zz), 3).tolist() == g["g_3dp"][word]
        assert _r(gated, 3).tolist() == g["out_3dp"][word]


def test_gated_heads_headwise():
    g = load_golden("gate_examples.json")["gated_heads"]
    res = A.apply_gate(np.array(g["head_outputs"]), np.array([math.log(1 / 9), 0.0]), A.GATE_HEADWISE)
    assert math.isclose(res[0][0], g["result_0_0"])
    assert math.isclose(res[1][1], g["result_1_1"])
    z0 = A.apply_gate(np.array(g["zero_logit_heads"]), np.array([0.0]), A.GATE_HEADWISE)
    assert z0.tolist() == g["zero_logit_result_exact"]      # exactly 0.5x


def test_gated_heads_rejects_bad_input():
    with pytest.raises(ValueError):
        A.apply_gate(np.array([[4.0, -2.0]]), np.array([np.nan]), A.GATE_HEADWISE)
    with pytest.raises(ValueError):
        A.apply_gate(np.array([[4.0, -2.0]]), np.array([]), A.GATE_HEADWISE)
    q = np.ones((1, 2, 1, 2))
    q[0, 1, 0, 0] = np.inf
    with pytest.raises(ValueError):
        A.prefill(q, np.ones((1, 2, 1, 2)), np.ones((1, 2, 1, 2)), None, gate_mode=A.GATE_NONE,
                  q_norm_w=None, k_norm_w=None, positions=np.arange(2)[None])


def test_elementwise_concat_example():
    g = load_golden("gate_examples.json")["elementwise_concat"]
    p = np.array(g["gates"])
    logits = np.log(p / (1 - p))
    out = A.apply_gate(np.array(g["Y"]), logits, A.GATE_ELEMENTWISE).reshape(-1)
    assert np.allclose(out, g["concat"], atol=1e-12)


def _rand_case(seed, B=2, n=7, H=4, G=2, d=8, rot=4, gate_mode=A.GATE_ELEMENTWISE):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, n, H, d))
    k = rng.standard_normal((B, n, G, d))
    v = rng.standard_normal((B, n, G, d))
    gate = {A.GATE_ELEMENTWISE: rng.standard_normal((B, n, H, d)) * 1.5,
            A.GATE_HEADWISE: rng.standard_normal((B, n, H)) * 1.5, A.GATE_NONE: None}[gate_mode]
    wq = 1 + 0.02 * rng.standard_normal(d)
    wk = 1 + 0.02 * rng.standard_normal(d)
    pos = np.broadcast_to(np.arange(n), (B, n))
    return q, k, v, gate, wq, wk, pos


def test_gate_one_is_plain_attention_and_zero_logit_is_half():
    q, k, v, _, wq, wk, pos = _rand_case(3)
    kw = dict(q_norm_w=wq, k_norm_w=wk, positions=pos, rot_dim=4)
    plain = A.prefill(q, k, v, None, gate_mode=A.GATE_NONE, **kw)
    ones = A.prefill(q, k, v, np.full(q.shape, 100.0), gate_mode=A.GATE_ELEMENTWISE, **kw)
    assert np.array_equal(plain, ones)                        # sigmoid(100) == 1.0 exactly
    half = A.prefill(q, k, v, np.zeros(q.shape[:3]), gate_mode=A.GATE_HEADWISE, **kw)
    assert np.array_equal(half, plain * 0.5)
    off = A.prefill(q, k, v, np.full(q.shape, -100.0), gate_mode=A.GATE_ELEMENTWISE, **kw)
    assert np.max(np.abs(off)) < 1e-40
