"""Pins of the oracle's reading of a fused q projection (query and gate logits
from one projection, per-head [q | gate] rows).

Sources: "Transformer by Hand · 6. Gated attention", "Why the gate is packed
into q_proj" (each head's outputs are its query followed by its gate) and the
forward code and shape table of "The code: qwen/attention.py" ([B,T,4096]
viewed as [B,T,8,512], first 256 query, last 256 gate; the gate multiplies the
[B,T,2048] head concat). "Gated Attention：算完注意力，再决定用多少",
"怎样做一个有意义的对照？": a gate held at 1 gives plain attention, a gate at 0
silences its branch.
"""
import numpy as np
import pytest

from oracle import attention as A


def test_split_follows_the_per_head_layout_index_by_index():
    # a flat projection row whose every value names its own index
    H, d = 3, 4
    flat = np.arange(H * 2 * d, dtype=np.float64)
    q, gate = A.split_q_proj(flat.reshape(H, 2 * d), d, A.GATE_ELEMENTWISE)
    assert q.shape == (H, d) and gate.shape == (H, d)
    for h in range(H):
        for e in range(d):
            assert q[h, e] == h * 2 * d + e
            assert gate[h, e] == h * 2 * d + d + e


def test_split_matches_the_shape_table():
    B, T, H, d = 2, 3, 8, 256
    x = np.arange(B * T * H * 2 * d, dtype=np.float64).reshape(B, T, H * 2 * d)    # q_proj(x): [B,T,4096]
    q, gate = A.split_q_proj(x.reshape(B, T, H, 2 * d), d, A.GATE_ELEMENTWISE)
    assert q.shape == (B, T, 8, 256)
    g2 = gate.reshape(B, T, -1)                                                       # [B,T,2048]
    assert g2.shape == (B, T, 2048)
    # output column h*d + e of the concat is gated by projection value h*2d + d + e
    for h in (0, 5, 7):
        for e in (0, 17, 255):
            assert g2[1, 2, h * d + e] == x[1, 2, h * 2 * d + d + e]


def test_split_headwise_reading():
    H, d = 2, 3
    flat = np.arange(H * (d + 1), dtype=np.float64)
    q, gate = A.split_q_proj(flat.reshape(H, d + 1), d, A.GATE_HEADWISE)
    assert q.shape == (H, d) and gate.shape == (H,)
    for h in range(H):
        assert list(q[h]) == [h * (d + 1) + e for e in range(d)]
        assert gate[h] == h * (d + 1) + d


@pytest.mark.parametrize("mode,width", [(A.GATE_ELEMENTWISE, 9), (A.GATE_HEADWISE, 8), (A.GATE_NONE, 8)])
def test_split_rejects_other_widths(mode, width):
    with pytest.raises(ValueError):
        A.split_q_proj(np.zeros((2, width)), 4, mode)


def _packed_prefill(gate_half, gate_mode, rng, B=1, n=5, H=4, G=2, d=8):
    q = rng.standard_normal((B, n, H, d))
    k = rng.standard_normal((B, n, G, d))
    v = rng.standard_normal((B, n, G, d))
    qg = np.concatenate([q, gate_half], axis=-1) if gate_mode == A.GATE_ELEMENTWISE else \
        np.concatenate([q, gate_half[..., None]], axis=-1)
    qq, gg = A.split_q_proj(qg, d, gate_mode)
    kw = dict(q_norm_w=None, k_norm_w=None, positions=np.tile(np.arange(n), (B, 1)), rms_eps=1e-6,
              rope_base=10000.0, rot_dim=2)
    gated = A.prefill(qq, k, v, gg, gate_mode=gate_mode, **kw)
    plain = A.prefill(q, k, v, None, gate_mode=A.GATE_NONE, **kw)
    return gated, plain


@pytest.mark.parametrize("mode", [A.GATE_ELEMENTWISE, A.GATE_HEADWISE])
def test_open_gate_half_gives_plain_attention_of_the_query_half(mode):
    rng = np.random.default_rng(71)
    B, n, H, d = 1, 5, 4, 8
    z = np.full((B, n, H, d) if mode == A.GATE_ELEMENTWISE else (B, n, H), 800.0)   # sigmoid = 1 in fp64
    gated, plain = _packed_prefill(z, mode, rng)
    np.testing.assert_array_equal(gated, plain)


@pytest.mark.parametrize("mode", [A.GATE_ELEMENTWISE, A.GATE_HEADWISE])
def test_closed_gate_of_one_head_silences_only_its_columns(mode):
    rng = np.random.default_rng(72)
    B, n, H, d = 1, 5, 4, 8
    z = np.full((B, n, H, d) if mode == A.GATE_ELEMENTWISE else (B, n, H), 800.0)
    z[:, :, 2] = -800.0                                                                 # sigmoid = 0 for head 2
    gated, plain = _packed_prefill(z, mode, rng)
    cols = np.arange(H * d)
    head2 = (cols >= 2 * d) & (cols < 3 * d)
    assert np.all(gated[..., head2] == 0.0)
    np.testing.assert_array_equal(gated[..., ~head2], plain[..., ~head2])
    assert np.all(plain[..., head2] != 0.0)
