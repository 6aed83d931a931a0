"""Pins of the backward oracle (``oracle.backward``): every gradient against
central finite differences of the forward oracle, and the gate gradient
against the worked SGD example that "Transformer by Hand · 6. Gated
attention" prints in "How the gate is learned" (two tokens, a one-number gate
per token, learning rate 1: w, both gates, the loss and the gradient at steps
0, 1, 2, 5, 20, 50 and 200)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import backward as BW


def _setup(seed, gate_mode, B=1, n=4, H=4, G=2, d=4, rot=2, norm=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, n, H, d))
    k = rng.standard_normal((B, n, G, d))
    v = rng.standard_normal((B, n, G, d))
    gate = None
    if gate_mode == A.GATE_ELEMENTWISE:
        gate = rng.standard_normal((B, n, H, d))
    elif gate_mode == A.GATE_HEADWISE:
        gate = rng.standard_normal((B, n, H))
    wq = 1.0 + 0.3 * rng.standard_normal(d) if norm else None
    wk = 1.0 + 0.3 * rng.standard_normal(d) if norm else None
    pos = np.tile(np.arange(3, 3 + n), (B, 1))
    dout = rng.standard_normal((B, n, H * d))
    return dict(q=q, k=k, v=v, gate=gate, wq=wq, wk=wk, pos=pos, dout=dout)


def _loss(x, gate_mode, rot):
    out = A.prefill(x["q"], x["k"], x["v"], x["gate"], gate_mode=gate_mode, q_norm_w=x["wq"], k_norm_w=x["wk"],
                    positions=x["pos"], rms_eps=1e-3, rope_base=100.0, rot_dim=rot)
    return float(np.sum(out * x["dout"]))


@pytest.mark.parametrize("gate_mode", [A.GATE_ELEMENTWISE, A.GATE_HEADWISE, A.GATE_NONE])
@pytest.mark.parametrize("norm", [True, False])
def test_gradients_match_central_differences(gate_mode, norm):
    rot = 2
    x = _setup(61 + (gate_mode == A.GATE_HEADWISE) + 2 * norm, gate_mode, norm=norm)
    got = BW.prefill_backward(x["q"], x["k"], x["v"], x["gate"], x["dout"], gate_mode=gate_mode,
                              q_norm_w=x["wq"], k_norm_w=x["wk"], positions=x["pos"], rms_eps=1e-3,
                              rope_base=100.0, rot_dim=rot)
    h = 1e-6
    pairs = [("q", "dq"), ("k", "dk"), ("v", "dv")]
    if x["gate"] is not None:
        pairs.append(("gate", "dgate"))
    if norm:
        pairs += [("wq", "dq_norm_w"), ("wk", "dk_norm_w")]
    for name, gname in pairs:
        arr = x[name]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _loss(x, gate_mode, rot)
            arr[idx] = keep - h
            lm = _loss(x, gate_mode, rot)
            arr[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(got[gname], fd, rtol=2e-6, atol=2e-7, err_msg=f"{gate_mode} {gname}")


def test_longer_causal_gqa_case_against_differences():
    # more keys per row than the tiny case, group of 3, rot = d
    rng = np.random.default_rng(66)
    x = _setup(67, A.GATE_ELEMENTWISE, B=2, n=7, H=3, G=1, d=6, rot=6)
    got = BW.prefill_backward(x["q"], x["k"], x["v"], x["gate"], x["dout"], gate_mode=A.GATE_ELEMENTWISE,
                              q_norm_w=x["wq"], k_norm_w=x["wk"], positions=x["pos"], rms_eps=1e-3,
                              rope_base=100.0, rot_dim=6)
    h = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        arr = x[name]
        for _ in range(12):                    # a sample of elements
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _loss(x, A.GATE_ELEMENTWISE, 6)
            arr[idx] = keep - h
            lm = _loss(x, A.GATE_ELEMENTWISE, 6)
            arr[idx] = keep
            assert abs(got[gname][idx] - (lp - lm) / (2 * h)) <= 2e-6 * max(1.0, abs(got[gname][idx])), (gname, idx)


# The worked example: x(?) = [1, 0], x(digit) = [0, 1]; y = r + g * o with
# r = [0, 1], o = [1, 0.8], target t = 1, loss sum (y - t)^2 / 2, w0 = [0.01, -0.02].
PRINTED = {   # step: (w, gates, loss, gradient)
    0: ([0.010, -0.020], [0.502, 0.495], 0.2022, [-0.1244, 0.0792]),
    1: ([0.134, -0.099], [0.534, 0.475], 0.1811, [-0.1161, 0.0758]),
    2: ([0.250, -0.175], [0.562, 0.456], 0.1624, [-0.1077, 0.0725]),
    5: ([0.550, -0.382], [0.634, 0.406], 0.1196, [-0.0849, 0.0626]),
    20: ([1.365, -1.065], [0.797, 0.256], 0.0417, [-0.0330, 0.0313]),
    50: ([1.980, -1.678], [0.879, 0.157], 0.0153, [-0.0129, 0.0134]),
    200: ([2.835, -2.568], [0.945, 0.071], 0.0032, [-0.0029, 0.0030]),
}


def test_gate_gradient_reproduces_the_printed_sgd_run():
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    r, o, t = np.array([0.0, 1.0]), np.array([1.0, 0.8]), np.array([1.0, 1.0])
    w = np.array([0.01, -0.02])
    for step in range(201):
        z = x @ w
        g = A.sigmoid(z)
        yout = r + g * o
        loss = float(np.sum((yout - t) ** 2 / 2))
        # the head output o with a headwise gate of one head: dL/dout = y - t
        _, dz = BW.gate_backward(o[:, None, None], z[:, None], (yout - t)[:, None, None], A.GATE_HEADWISE)
        grad = x.T @ dz[:, 0]
        if step in PRINTED:
            pw, pg, pl, pgrad = PRINTED[step]
            assert np.array_equal(np.round(w, 3), pw), (step, w)
            assert np.array_equal(np.round(g, 3), pg), (step, g)
            assert round(loss, 4) == pl, (step, loss)
            assert np.array_equal(np.round(grad, 4), pgrad), (step, grad)
        w = w - 1.0 * grad


def test_norm_and_rope_backward_pieces():
    rng = np.random.default_rng(68)
    x = rng.standard_normal((3, 5, 8))
    w = rng.standard_normal(8)
    g = rng.standard_normal((3, 5, 8))
    dx, dw = BW.rms_norm_backward(x, w, 0.01, g)
    # the norm is invariant to scaling x: its gradient is orthogonal to x (with eps = 0)
    dx0, _ = BW.rms_norm_backward(x, w, 0.0, g)
    np.testing.assert_allclose(np.sum(dx0 * x, axis=-1), 0.0, atol=1e-12)
    # RoPE is a rotation: the backward is the inverse rotation and keeps pair norms
    pos = np.arange(5)[None].repeat(3, 0)
    gb = BW.rope_backward(g[:, :, None, :], pos, 8, 10000.0)
    np.testing.assert_allclose(A.rope(gb, pos, 8, 10000.0), g[:, :, None, :], atol=1e-13)
    assert dw.shape == (8,) and dx.shape == x.shape


@pytest.mark.parametrize("gate_mode", [A.GATE_ELEMENTWISE, A.GATE_HEADWISE])
def test_backward_rows_equal_the_whole_backward(gate_mode):
    x = _setup(69, gate_mode, B=2, n=9, H=4, G=2, d=8, rot=4)
    kw = dict(gate_mode=gate_mode, q_norm_w=x["wq"], k_norm_w=x["wk"], positions=x["pos"], rms_eps=1e-3,
              rope_base=100.0, rot_dim=4)
    full = BW.prefill_backward(x["q"], x["k"], x["v"], x["gate"], x["dout"], **kw)
    qr = [(0, 0, 0), (1, 8, 3), (0, 5, 2)]
    kr = [(1, 8, 1), (0, 6, 0), (1, 0, 1)]
    rows = BW.backward_rows(x["q"], x["k"], x["v"], x["gate"], x["dout"], q_rows=qr, k_rows=kr, **kw)
    for r, (b, i, h) in enumerate(qr):
        np.testing.assert_allclose(rows["dq"][r], full["dq"][b, i, h], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rows["dgate"][r], full["dgate"][b, i, h], rtol=1e-10, atol=1e-12)
    for r, (b, j, g) in enumerate(kr):
        np.testing.assert_allclose(rows["dk"][r], full["dk"][b, j, g], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rows["dv"][r], full["dv"][b, j, g], rtol=1e-10, atol=1e-12)
