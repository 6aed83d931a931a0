"""Brute-force pure-Python gated GQA causal attention, for tiny shapes.

TEST INFRASTRUCTURE (see the package docstring). Written independently of
``oracle.attention`` (no NumPy, no shared helpers): explicit loops over
batch, token, head, key and dimension, so that the two can check each other.
It follows the same definition, step by step, in the order the pages give
("Attention, worked all the way through", section "Qwen3's exact order":
RMSNorm q and k per head, RoPE q and k, per-query-head causal attention with
GQA sharing, concatenate; then the output gate of "Gated Attention：算完注意力，
再决定用多少", section "门放在哪里？").

Inputs are nested Python lists: q[b][i][h][e], k/v[b][j][g][e],
gate[b][i][h][e] (elementwise) or gate[b][i][h] (headwise) or None.
"""
from __future__ import annotations

import math


def _normed(vec, w, eps):
    if w is None:
        return list(vec)
    d = len(vec)
    ss = 0.0
    for x in vec:
        ss += x * x
    inv = 1.0 / math.sqrt(ss / d + eps)
    return [vec[e] * inv * w[e] for e in range(d)]


def _rotated(vec, pos, rot_dim, base):
    out = list(vec)
    half = rot_dim // 2
    for t in range(half):
        theta = pos * base ** (-2.0 * t / rot_dim)
        c, s = math.cos(theta), math.sin(theta)
        a, b = vec[t], vec[t + half]
        out[t] = a * c - b * s
        out[t + half] = b * c + a * s
    return out


def _sig(z):
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    e = math.exp(z)
    return e / (1.0 + e)


def gated_attention(q, k, v, gate, gate_mode, w_q, w_k, positions, eps, base, rot_dim, scale=None):
    """Returns out[b][i][h*d + e] as nested lists."""
    B = len(q)
    n = len(q[0])
    H = len(q[0][0])
    d = len(q[0][0][0])
    G = len(k[0][0])
    group = H // G
    sc = scale if scale else 1.0 / math.sqrt(d)
    out = []
    for b in range(B):
        rows = []
        khat = [[_rotated(_normed(k[b][j][g], w_k, eps), positions[b][j], rot_dim, base)
                 for g in range(G)] for j in range(n)]
        for i in range(n):
            row = []
            for h in range(H):
                g = h // group
                qh = _rotated(_normed(q[b][i][h], w_q, eps), positions[b][i], rot_dim, base)
                scores = []
                for j in range(i + 1):
                    dot = 0.0
                    for e in range(d):
                        dot += qh[e] * khat[j][g][e]
                    scores.append(dot * sc)
                m = max(scores)
                ex = [math.exp(s - m) for s in scores]
                tot = sum(ex)
                for e in range(d):
                    acc = 0.0
                    for j in range(i + 1):
                        acc += ex[j] / tot * v[b][j][g][e]
                    if gate_mode == "elementwise":
                        acc *= _sig(gate[b][i][h][e])
                    elif gate_mode == "headwise":
                        acc *= _sig(gate[b][i][h])
                    row.append(acc)
            rows.append(row)
        out.append(rows)
    return out
