"""Pins of the oracle's gate variants (``GateForm``) against closed forms,
library routines and the plain gate they reduce to.

Sources ("Gated Attention for Large Language Models ... 论文阅读"): section
"五个门控位置与训练结果总览" (multiplicative vs additive Y + sigmoid(X W), sigmoid
vs SiLU), "实验规模与参数预算怎样控制" (the head-shared gate of Table 1),
"第一条机制线索：value 与输出投影之间的非线性" (per-head SDPA-output RMSNorm,
the additive gate without its SiLU, the input-independent gate) and
"第二条机制线索：当前 query 决定的稀疏过滤" (NS-sigmoid = 0.5 + 0.5 sigmoid, scores
kept in [0.5, 1]).
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import attention as A

KW = dict(q_norm_w=None, k_norm_w=None, rms_eps=1e-6, rope_base=10000.0, rot_dim=2)


def _inputs(seed, B=2, n=6, H=4, G=2, d=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, n, H, d))
    k = rng.standard_normal((B, n, G, d))
    v = rng.standard_normal((B, n, G, d))
    return q, k, v, np.tile(np.arange(n), (B, 1))


def test_activations_closed_forms():
    z = np.array([-30.0, -2.5, -0.25, 0.0, 0.25, 2.5, 30.0])
    np.testing.assert_allclose(A.gate_activation(z, "sigmoid"), expit(z), rtol=1e-15, atol=0)
    np.testing.assert_allclose(A.gate_activation(z, "ns_sigmoid"), 0.5 + 0.5 * expit(z), rtol=1e-15, atol=0)
    np.testing.assert_allclose(A.gate_activation(z, "silu"), z * expit(z), rtol=1e-15, atol=1e-300)
    np.testing.assert_array_equal(A.gate_activation(z, "identity"), z)
    assert A.gate_activation(0.0, "ns_sigmoid") == 0.75
    assert A.gate_activation(0.0, "silu") == 0.0
    ns = A.gate_activation(np.linspace(-50, 50, 1001), "ns_sigmoid")
    assert ns.min() >= 0.5 and ns.max() <= 1.0
    with pytest.raises(ValueError):
        A.gate_activation(z, "tanh")


def _plain(q, k, v, pos):
    return A.prefill(q, k, v, None, gate_mode=A.GATE_NONE, positions=pos, **KW)


@pytest.mark.parametrize("act,want", [("sigmoid", 0.5), ("ns_sigmoid", 0.75), ("silu", 0.0), ("identity", 0.0)])
def test_zero_logits_scale_or_shift_by_act0(act, want):
    q, k, v, pos = _inputs(81)
    plain = _plain(q, k, v, pos)
    z = np.zeros(q.shape)
    mul = A.prefill(q, k, v, z, gate_mode=A.GATE_ELEMENTWISE, positions=pos,
                    gate_form=A.GateForm(act=act), **KW)
    add = A.prefill(q, k, v, z, gate_mode=A.GATE_ELEMENTWISE, positions=pos,
                    gate_form=A.GateForm(act=act, combine="add"), **KW)
    np.testing.assert_array_equal(mul, plain * want)
    np.testing.assert_array_equal(add, plain + want)


def test_additive_gate_closed_and_open():
    q, k, v, pos = _inputs(82)
    plain = _plain(q, k, v, pos)
    z = np.full(q.shape[:3], -800.0)                                  # headwise, sigmoid = 0
    out = A.prefill(q, k, v, z, gate_mode=A.GATE_HEADWISE, positions=pos, gate_form=A.GateForm(combine="add"), **KW)
    np.testing.assert_array_equal(out, plain)
    z[:, :, 1] = 800.0                                                # head 1: + 1
    out = A.prefill(q, k, v, z, gate_mode=A.GATE_HEADWISE, positions=pos, gate_form=A.GateForm(combine="add"), **KW)
    d = q.shape[-1]
    np.testing.assert_array_equal(out[..., d:2 * d], plain[..., d:2 * d] + 1.0)
    np.testing.assert_array_equal(out[..., :d], plain[..., :d])


@pytest.mark.parametrize("mode", [A.GATE_ELEMENTWISE, A.GATE_HEADWISE])
def test_shared_gates_equal_the_repeated_gate(mode):
    q, k, v, pos = _inputs(83)
    B, n, H, d = q.shape
    rng = np.random.default_rng(84)
    row = (d,) if mode == A.GATE_ELEMENTWISE else ()
    z_tok = rng.standard_normal((B, n) + row)            # one gate per token, for every head
    z_head = rng.standard_normal((H,) + row)             # one gate per head, for every token
    z_one = rng.standard_normal(row)                     # one gate for everything
    for form, z, full in (
            (A.GateForm(share_heads=True), z_tok, np.repeat(np.expand_dims(z_tok, 2), H, axis=2)),
            (A.GateForm(input_independent=True), z_head, np.broadcast_to(z_head, (B, n, H) + row)),
            (A.GateForm(share_heads=True, input_independent=True, act="silu"), z_one,
             np.broadcast_to(z_one, (B, n, H) + row))):
        got = A.prefill(q, k, v, z, gate_mode=mode, positions=pos, gate_form=form, **KW)
        ref_form = A.GateForm(act=form.act)
        want = A.prefill(q, k, v, np.ascontiguousarray(full), gate_mode=mode, positions=pos, gate_form=ref_form, **KW)
        np.testing.assert_array_equal(got, want)


def test_output_norm_per_head():
    q, k, v, pos = _inputs(85)
    B, n, H, d = q.shape
    one = A.GateForm(out_norm_w=np.ones(d), out_norm_eps=0.0)
    out = A.prefill(q, k, v, None, gate_mode=A.GATE_NONE, positions=pos, gate_form=one, **KW).reshape(B, n, H, d)
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 1.0, rtol=1e-12)
    # scale invariance in v, the weight per column, and the norm comes before the gate
    out2 = A.prefill(q, k, 3.0 * v, None, gate_mode=A.GATE_NONE, positions=pos, gate_form=one, **KW)
    np.testing.assert_allclose(out2.reshape(out.shape), out, rtol=1e-12, atol=1e-14)
    w = np.linspace(0.5, 2.0, d)
    outw = A.prefill(q, k, v, None, gate_mode=A.GATE_NONE, positions=pos,
                     gate_form=A.GateForm(out_norm_w=w, out_norm_eps=0.0), **KW).reshape(out.shape)
    np.testing.assert_allclose(outw, out * w, rtol=1e-12)
    z = np.random.default_rng(86).standard_normal(q.shape)
    gated = A.prefill(q, k, v, z, gate_mode=A.GATE_ELEMENTWISE, positions=pos, gate_form=one, **KW)
    np.testing.assert_allclose(gated.reshape(out.shape), out * expit(z), rtol=1e-12)
    # plain RMSNorm with eps: x / sqrt(mean(x^2) + eps)
    plain = _plain(q, k, v, pos).reshape(out.shape)
    eps = 0.3
    oe = A.prefill(q, k, v, None, gate_mode=A.GATE_NONE, positions=pos,
                   gate_form=A.GateForm(out_norm_w=np.ones(d), out_norm_eps=eps), **KW).reshape(out.shape)
    np.testing.assert_allclose(oe, plain / np.sqrt(np.mean(plain ** 2, -1, keepdims=True) + eps), rtol=1e-12)


def test_default_form_is_the_plain_gate():
    q, k, v, pos = _inputs(87)
    z = np.random.default_rng(88).standard_normal(q.shape)
    a = A.prefill(q, k, v, z, gate_mode=A.GATE_ELEMENTWISE, positions=pos, **KW)
    b = A.prefill(q, k, v, z, gate_mode=A.GATE_ELEMENTWISE, positions=pos, gate_form=A.GateForm(), **KW)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_allclose(a, _plain(q, k, v, pos) * expit(z).reshape(a.shape), rtol=1e-13)


def test_forms_agree_across_prefill_rows_chunk_and_decode():
    q, k, v, pos = _inputs(89, B=1, n=5)
    B, n, H, d = q.shape
    form = A.GateForm(act="ns_sigmoid", combine="add", share_heads=True,
                      out_norm_w=np.linspace(0.9, 1.1, d), out_norm_eps=1e-3)
    z = np.random.default_rng(90).standard_normal((B, n, d))
    full = A.prefill(q, k, v, z, gate_mode=A.GATE_ELEMENTWISE, positions=pos, gate_form=form, **KW)
    rows = A.prefill_rows(q, k, v, z, [(0, 3, 2), (0, 4, 0)], gate_mode=A.GATE_ELEMENTWISE, positions=pos,
                          gate_form=form, **KW)
    np.testing.assert_allclose(rows[0], full[0, 3, 2 * d:3 * d], rtol=1e-12)
    np.testing.assert_allclose(rows[1], full[0, 4, :d], rtol=1e-12)
    khat = A.prefill_keys(k, None, pos, rms_eps=1e-6, rope_base=10000.0, rot_dim=2)
    dec, _ = A.decode(q[:, 4], k[:, 4], v[:, 4], z[:, 4], gate_mode=A.GATE_ELEMENTWISE, q_norm_w=None,
                      k_norm_w=None, k_cache_rows=lambda b: (khat[b, :4], v[b, :4]), cache_lens=np.array([4]),
                      rms_eps=1e-6, rope_base=10000.0, rot_dim=2, gate_form=form)
    np.testing.assert_allclose(dec[0], full[0, 4], rtol=1e-12, atol=1e-13)
    ch, _ = A.prefill_chunk(q[:, 2:], k[:, 2:], v[:, 2:], z[:, 2:], gate_mode=A.GATE_ELEMENTWISE, q_norm_w=None,
                            k_norm_w=None, k_cache_rows=lambda b: (khat[b, :2], v[b, :2]), cache_lens=np.array([2]),
                            rms_eps=1e-6, rope_base=10000.0, rot_dim=2, gate_form=form)
    np.testing.assert_allclose(ch[0], full[0, 2:], rtol=1e-12, atol=1e-13)
