"""NumPy oracle of the backward pass of gated GQA causal attention.

TEST INFRASTRUCTURE: only tests, the smoke check and the bench's CPU-baseline
leg may use this module (as for ``oracle.attention``).

The chain rule written out step by step through the forward definition of
``oracle.attention`` (fp64 by default):

    out = y * sigmoid(z)                        gate ("门放在哪里？"; the gradient
                                                (y - t) * o * g(1 - g) * x of the
                                                toy in "How the gate is learned")
    y   = softmax(q_hat k_hat^T * scale) V      causal, GQA
    q_hat = RoPE(RMSNorm(q, w_q)), k_hat = RoPE(RMSNorm(k, w_k))

Given dout = dL/dout [B,n,H*d]:

    dy = dout * sigmoid(z);  dz = dout * y * sigmoid(z) (1 - sigmoid(z))
         (headwise: dz_h = sum_e dout_e y_e * sigma'(z_h); no gate: dy = dout)
    dP = dy V^T;  dS = P * (dP - rowsum(P * dP))
    dq_hat = dS k_hat * scale;  dk_hat = sum over the group's heads of dS^T q_hat * scale
    dV = sum over the group's heads of P^T dy
    RoPE^-1 on the gradients (rotation by -angle), then the RMSNorm backward
    dx = (w*g - x_hat * mean(w*g*x_hat)) / r,  dw = sum over rows of g * x_hat
    with r = sqrt(mean(x^2) + eps) and x_hat = x / r.

Sources: the forward is that of ``oracle.attention`` ("Transformer by Hand ·
6. Gated attention", "The formula", "Four things Qwen3.5 adds to the
textbook", "The code: qwen/attention.py"); the gate's gradient is the one
"Transformer by Hand · 6. Gated attention" prints in "How the gate is
learned". The rest is calculus on that definition, pinned by central finite
differences of the forward oracle in the tests.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import (GATE_ELEMENTWISE, GATE_HEADWISE, GATE_NONE, _check_finite, _default_scale, kv_group,
                        rms_norm, rope, rope_angles, sigmoid, softmax_rows)


def rms_norm_backward(x, w, eps: float, g, dtype=np.float64):
    """(dx, dw) of n = x / sqrt(mean(x^2) + eps) * w over the last axis, for
    the upstream gradient g = dL/dn. dw sums over every leading axis; w=None
    (no norm) passes g through and returns dw=None."""
    x = np.asarray(x, dtype=dtype)
    g = np.asarray(g, dtype=dtype)
    if w is None:
        return g, None
    w = np.asarray(w, dtype=dtype)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + dtype(eps))
    xh = x / r
    gw = g * w
    dx = (gw - xh * np.mean(gw * xh, axis=-1, keepdims=True)) / r
    dw = np.sum((g * xh).reshape(-1, x.shape[-1]), axis=0)
    return dx, dw


def rope_backward(g, positions, rot_dim: int, base: float, dtype=np.float64):
    """Gradient through ``oracle.attention.rope``: the rotation's transpose
    (each pair turned back by its angle); dims >= rot_dim pass through."""
    g = np.asarray(g, dtype=dtype)
    if rot_dim == 0:
        return g
    half = rot_dim // 2
    th = rope_angles(positions, rot_dim, base, dtype=np.float64)[..., None, :]
    c = np.cos(th).astype(dtype)
    s = np.sin(th).astype(dtype)
    out = g.copy()
    ga = g[..., :half]
    gb = g[..., half:rot_dim]
    out[..., :half] = ga * c + gb * s
    out[..., half:rot_dim] = gb * c - ga * s
    return out


def gate_backward(y, z, dout, gate_mode: str, dtype=np.float64):
    """(dy, dz) of out = y * sigmoid(z) for per-head outputs y [..., H, d]
    and dout of the same shape; z [..., H, d] (elementwise) or [..., H]
    (headwise). The gate's slope is g(1 - g), as on "Transformer by Hand ·
    6. Gated attention", "How the gate is learned"."""
    y = np.asarray(y, dtype=dtype)
    dout = np.asarray(dout, dtype=dtype)
    if gate_mode == GATE_NONE:
        return dout, None
    g = sigmoid(z, dtype=dtype)
    slope = g * (1.0 - g)
    if gate_mode == GATE_ELEMENTWISE:
        return dout * g, dout * y * slope
    if gate_mode == GATE_HEADWISE:
        return dout * g[..., None], np.sum(dout * y, axis=-1) * slope
    raise ValueError(f"unknown gate mode {gate_mode!r}")


def attention_backward(qh, kh, v, dy, scale: float, dtype=np.float64):
    """One head's causal attention backward: qh [n,d] (normed, rotated), kh
    [n,d], v [n,d], dy [n,d] = dL/dy. Returns (dqh, dkh, dv)."""
    n = qh.shape[0]
    s = (qh @ kh.T) * dtype(scale)
    s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = softmax_rows(s, dtype)
    dp = dy @ v.T
    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    return (ds @ kh) * dtype(scale), (ds.T @ qh) * dtype(scale), p.T @ dy


def prefill_backward(q, k, v, gate, dout, *, gate_mode: str, q_norm_w, k_norm_w, positions,
                     rms_eps: float = 1e-6, rope_base: float = 10000.0, rot_dim: int = 0,
                     scale: Optional[float] = None, dtype=np.float64) -> dict:
    """Gradients of sum(dout * prefill(...)) with respect to every input.

    q [B,n,H,d], k/v [B,n,G,d], gate [B,n,H,d] | [B,n,H] | None, dout
    [B,n,H*d]. Returns dq, dk, dv, dgate (None without a gate), dq_norm_w,
    dk_norm_w (None without a norm), in the inputs' shapes.
    """
    for name, x in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_finite(name, x)
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    B, n, H, d = q.shape
    G = k.shape[2]
    sc = _default_scale(d, scale)
    pos = np.asarray(positions)
    qn = rms_norm(q, q_norm_w, rms_eps, dtype)
    kn = rms_norm(k, k_norm_w, rms_eps, dtype)
    qh = rope(qn, pos, rot_dim, rope_base, dtype)
    kh = rope(kn, pos, rot_dim, rope_base, dtype)
    # forward attention output y (ungated), per head
    y = np.empty((B, n, H, d), dtype=dtype)
    for b in range(B):
        for h in range(H):
            g = kv_group(h, H, G)
            s = (qh[b, :, h] @ kh[b, :, g].T) * dtype(sc)
            s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
            y[b, :, h] = softmax_rows(s, dtype) @ v[b, :, g]
    dy, dgate = gate_backward(y, gate, np.asarray(dout, dtype=dtype).reshape(B, n, H, d), gate_mode, dtype)
    dqh = np.zeros_like(qh)
    dkh = np.zeros_like(kh)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = kv_group(h, H, G)
            a, bk, bv = attention_backward(qh[b, :, h], kh[b, :, g], v[b, :, g], dy[b, :, h], sc, dtype)
            dqh[b, :, h] = a
            dkh[b, :, g] += bk
            dv[b, :, g] += bv
    dqn = rope_backward(dqh, pos, rot_dim, rope_base, dtype)
    dkn = rope_backward(dkh, pos, rot_dim, rope_base, dtype)
    dq, dwq = rms_norm_backward(q, q_norm_w, rms_eps, dqn, dtype)
    dk, dwk = rms_norm_backward(k, k_norm_w, rms_eps, dkn, dtype)
    return dict(dq=dq, dk=dk, dv=dv, dgate=dgate, dq_norm_w=dwq, dk_norm_w=dwk, y=y)


def backward_rows(q, k, v, gate, dout, *, q_rows, k_rows, gate_mode: str, q_norm_w, k_norm_w, positions,
                  rms_eps: float = 1e-6, rope_base: float = 10000.0, rot_dim: int = 0,
                  scale: Optional[float] = None, dtype=np.float64) -> dict:
    """The gradients of selected rows only, for sizes where the whole
    backward is too expensive on the CPU (the same definition, row by row).

    q_rows: (b, i, h) -> dq[b, i, h] and dgate[b, i, h] (elementwise: [d],
    headwise: a scalar); k_rows: (b, j, g) -> dk[b, j, g] and dv[b, j, g],
    which need every query row i >= j of the group's heads (cheap for keys
    near the end of the sequence)."""
    q = np.asarray(q)
    B, n, H, d = q.shape
    G = np.asarray(k).shape[2]
    grp = H // G
    sc = dtype(_default_scale(d, scale))
    pos = np.asarray(positions)
    z_all = None if gate is None else np.asarray(gate)
    dout = np.asarray(dout, dtype=dtype).reshape(B, n, H, d)
    cache = {}

    def khat(b, g):
        if ("k", b, g) not in cache:
            kn = rms_norm(np.asarray(k)[b, :, g][:, None, :], k_norm_w, rms_eps, dtype)
            cache[("k", b, g)] = rope(kn, pos[b], rot_dim, rope_base, dtype)[:, 0, :]
        return cache[("k", b, g)]

    def qhat_row(b, i, h):
        qn = rms_norm(q[b, i, h][None, None, :], q_norm_w, rms_eps, dtype)
        return rope(qn, pos[b, i:i + 1], rot_dim, rope_base, dtype)[0, 0]

    def row(b, i, h):
        """P row, y, dy, dP row and dS row of query (b, i, h)."""
        g = h // grp
        kh = khat(b, g)[: i + 1]
        vv = np.asarray(v, dtype=dtype)[b, : i + 1, g]
        qv = qhat_row(b, i, h)
        p = softmax_rows(((kh @ qv) * sc)[None, :], dtype)[0]
        y = p @ vv
        if gate_mode == GATE_ELEMENTWISE:
            dy = dout[b, i, h] * sigmoid(z_all[b, i, h], dtype)
        elif gate_mode == GATE_HEADWISE:
            dy = dout[b, i, h] * sigmoid(z_all[b, i, h], dtype)
        else:
            dy = dout[b, i, h]
        dp = vv @ dy
        ds = p * (dp - np.sum(p * dp))
        return qv, kh, p, y, dy, ds

    out = {"dq": [], "dgate": [], "dk": [], "dv": []}
    for (b, i, h) in q_rows:
        qv, kh, p, y, dy, ds = row(b, i, h)
        dqh = (ds @ kh) * sc
        dqn = rope_backward(dqh[None, None, :], pos[b, i:i + 1], rot_dim, rope_base, dtype)[0, 0]
        dq, _ = rms_norm_backward(q[b, i, h][None, :], q_norm_w, rms_eps, dqn[None, :], dtype)
        out["dq"].append(dq[0])
        if gate_mode != GATE_NONE:
            _, dz = gate_backward(y[None, None, :], np.asarray(z_all[b, i, h])[None, None],
                                  dout[b, i, h][None, None, :], gate_mode, dtype)
            out["dgate"].append(dz[0, 0])
    for (b, j, g) in k_rows:
        dkh = np.zeros(d, dtype=dtype)
        dvj = np.zeros(d, dtype=dtype)
        for h in range(g * grp, (g + 1) * grp):
            for i in range(j, n):
                qv, kh, p, y, dy, ds = row(b, i, h)
                dvj += p[j] * dy
                dkh += ds[j] * qv * sc
        dkn = rope_backward(dkh[None, None, :], pos[b, j:j + 1], rot_dim, rope_base, dtype)[0, 0]
        dk, _ = rms_norm_backward(np.asarray(k)[b, j, g][None, :], k_norm_w, rms_eps, dkn[None, :], dtype)
        out["dk"].append(dk[0])
        out["dv"].append(dvj)
    return {key: np.array(val) for key, val in out.items()}
