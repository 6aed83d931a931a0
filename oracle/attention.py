"""NumPy oracle: gated GQA causal attention written out as its definition.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the bench's CPU-baseline leg may use this module.

Notation follows the pages. For batch b, query token i, query head h, with
group = H/G query heads per key/value head and g = floor(h / group):

    q_hat = RoPE(RMSNorm(q[b,i,h], w_q), pos[b,i])
    k_hat_j = RoPE(RMSNorm(k[b,j,g], w_k), pos[b,j])          for j <= i
    s_j = (q_hat . k_hat_j) * scale,   scale = 1/sqrt(d)
    a_j = exp(s_j - max s) / sum_j exp(s_j - max s)           (causal: j <= i)
    y = sum_j a_j v[b,j,g]
    out[b,i,h*d:(h+1)*d] = y * sigmoid(z)                      (z: gate logits)

Sources:
* "Transformer by Hand · 6. Gated attention": section "The formula"
  (softmax(QK^T/sqrt(d) + M) V with the causal mask M); section "Four things
  Qwen3.5 adds to the textbook" (GQA sharing, QK-Norm before RoPE, RoPE on the
  first quarter of the head, the output gate); the forward code and its shape
  table in "The code: qwen/attention.py" (norm then RoPE, repeat_interleave
  for GQA, mask above the diagonal, gate multiplied after the head concat).
* "Gated Attention：算完注意力，再决定用多少", section "门放在哪里？"
  (Y = Concat_h(G_h ⊙ O_h) W_O, headwise vs elementwise gate) and the
  two-branch sigmoid in "两个 head，手算一次".
* "多头注意力与 GQA", section "分组查询注意力（GQA）" (head h reads KV group
  floor(h / group_size)).
* "Attention, worked all the way through": "Why scaling and stable softmax
  matter" (subtract the row max before exp; a masked -inf gets weight 0) and
  "Qwen3's exact order" (norm q and k, not v; then RoPE; then attention).
* "Gated Attention for Large Language Models ... 论文阅读", section
  "从标准注意力走到门控，计算流程有什么变化" (S, Y, g = sigmoid(X W_theta),
  Y~ = Y ⊙ g, concat then W_O).

Readings where the pages are silent (each is also listed in the design notes):
* RMSNorm: x / sqrt(mean(x^2) + eps) * w, eps inside the root, w the
  effective multiplier (parity with a real checkpoint's norm: unpinned).
* RoPE: rotate-half pairs (t, t + r/2) inside the first r = rot_dim dims, angle
  pos * base^(-2t/r); dims >= r untouched (checkpoint convention: unpinned).
* The causal mask is by token index inside the call (j <= i); positions only
  feed RoPE.
* Decode: the new token at position L attends to the L cached keys and to
  itself; cached K-hat is used as stored (already normed and rotated).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable, Optional, Sequence

import numpy as np

GATE_NONE = "none"
GATE_HEADWISE = "headwise"
GATE_ELEMENTWISE = "elementwise"


def _check_finite(name: str, x) -> None:
    # The headwise gate helper on "Gated Attention：算完注意力，再决定用多少"
    # rejects empty and non-finite inputs with ValueError; the oracle keeps
    # that convention for every input it is given.
    if x is None:
        return
    a = np.asarray(x)
    if a.size == 0:
        raise ValueError(f"{name}: expected a nonempty array")
    if a.dtype.kind == "f" and not np.all(np.isfinite(a)):
        raise ValueError(f"{name}: expected finite values")


def rms_norm(x: np.ndarray, w: Optional[np.ndarray], eps: float, dtype=np.float64) -> np.ndarray:
    """Per-vector RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w.

    QK-Norm of "Transformer by Hand · 6. Gated attention" (section "Four
    things Qwen3.5 adds to the textbook": q and k each pass an RMSNorm, one
    shared [d] weight per projection, before RoPE). ``w=None`` skips the norm.
    Pinned by closed forms and scale invariance in the tests.
    """
    x = np.asarray(x, dtype=dtype)
    if w is None:
        return x
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + dtype(eps)) * np.asarray(w, dtype=dtype)


def rope_angles(positions: np.ndarray, rot_dim: int, base: float, dtype=np.float64) -> np.ndarray:
    """Angles theta[..., t] = pos * base^(-2t/rot_dim) for t < rot_dim/2."""
    half = rot_dim // 2
    t = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(base), -2.0 * t / rot_dim)
    return (np.asarray(positions, dtype=np.float64)[..., None] * inv_freq).astype(dtype)


def rope(x: np.ndarray, positions: np.ndarray, rot_dim: int, base: float, dtype=np.float64) -> np.ndarray:
    """Rotate the first ``rot_dim`` dims of x [..., T, heads, d] by position.

    Partial RoPE of "Transformer by Hand · 6. Gated attention" (only the first
    quarter of each head rotates; the rest stays position-free). Pair
    convention (rotate-half within the rotated block) is a reading.
    ``positions`` has shape [..., T]; ``rot_dim == 0`` returns x unchanged.
    """
    x = np.asarray(x, dtype=dtype)
    if rot_dim == 0:
        return x
    half = rot_dim // 2
    th = rope_angles(positions, rot_dim, base, dtype=np.float64)[..., None, :]  # [..., T, 1, half]
    c = np.cos(th).astype(dtype)
    s = np.sin(th).astype(dtype)
    out = x.copy()
    a = x[..., :half]
    b = x[..., half:rot_dim]
    out[..., :half] = a * c - b * s
    out[..., half:rot_dim] = b * c + a * s
    return out


def sigmoid(z, dtype=np.float64):
    """Two-branch stable logistic sigmoid.

    As written on "Gated Attention：算完注意力，再决定用多少" (section
    "两个 head，手算一次"): z >= 0 uses 1/(1+e^-z), z < 0 uses e^z/(1+e^z).
    """
    z = np.asarray(z, dtype=dtype)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def apply_gate(y: np.ndarray, z: Optional[np.ndarray], gate_mode: str, dtype=np.float64,
               form: Optional[GateForm] = None) -> np.ndarray:
    """Output gate on per-head attention outputs y [..., H, d].

    Elementwise: y * sigmoid(z) with z [..., H, d]; headwise: one logit per
    token per head, z [..., H]; none: y. Source: "Gated Attention：算完注意力，
    再决定用多少", section "门放在哪里？" (G_h ⊙ O_h, headwise vs elementwise),
    and "Transformer by Hand · 6. Gated attention", "How the gate is computed:
    three steps" (g = sigmoid(z), multiplied dimension by dimension).
    ``form`` (already expanded z) selects the variants of ``GateForm``: the
    per-head output norm first, then combine(y, act(z)).
    """
    form = DEFAULT_GATE if form is None else form
    y = np.asarray(y, dtype=dtype)
    if form.out_norm_w is not None:
        y = rms_norm(y, form.out_norm_w, form.out_norm_eps, dtype)
    if gate_mode == GATE_NONE:
        return y
    _check_finite("gate logits", z)
    g = gate_activation(z, form.act, dtype=dtype)
    if gate_mode == GATE_HEADWISE:
        g = g[..., None]
    elif gate_mode != GATE_ELEMENTWISE:
        raise ValueError(f"unknown gate mode {gate_mode!r}")
    if form.combine == "mul":
        return y * g
    if form.combine == "add":
        return y + g
    raise ValueError(f"unknown gate combine {form.combine!r}")


@dataclass(frozen=True)
class GateForm:
    """Variants of the output gate, from "Gated Attention for Large Language
    Models ... 论文阅读":

    * act -- function of the gate logits: "sigmoid" (the default), "ns_sigmoid"
      0.5 + 0.5 sigmoid(z) (section "第二条机制线索：当前 query 决定的稀疏过滤"),
      "silu" z sigmoid(z) (SiLU against sigmoid, section "五个门控位置与训练结果
      总览"), "identity" z (the additive gate with its SiLU removed, section
      "第一条机制线索：value 与输出投影之间的非线性").
    * combine -- "mul" Y * act(z) (the default) or "add" Y + act(z) (the
      additive version, "五个门控位置与训练结果总览").
    * share_heads -- one gate for every head of a token (the head-shared vector
      of Table 1, "实验规模与参数预算怎样控制"): the gate has no head dim.
    * input_independent -- one gate for every token (the input-independent
      control of "第一条机制线索"): the gate has no batch or token dims.
    * out_norm_w -- per-head RMSNorm of the attention output before the gate
      (the per-head SDPA-output RMSNorm control of "第一条机制线索"), weight
      [d], epsilon out_norm_eps; None = no norm.
    """
    act: str = "sigmoid"
    combine: str = "mul"
    share_heads: bool = False
    input_independent: bool = False
    out_norm_w: Optional[np.ndarray] = None
    out_norm_eps: float = 1e-6


DEFAULT_GATE = GateForm()


def gate_activation(z, act: str, dtype=np.float64) -> np.ndarray:
    """act(z) for the gate forms above."""
    z = np.asarray(z, dtype=dtype)
    if act == "sigmoid":
        return sigmoid(z, dtype)
    if act == "ns_sigmoid":
        return 0.5 + 0.5 * sigmoid(z, dtype)
    if act == "silu":
        return z * sigmoid(z, dtype)
    if act == "identity":
        return z
    raise ValueError(f"unknown gate activation {act!r}")


def expand_gate(z, gate_mode: str, form: GateForm, lead: tuple, n_heads: int):
    """Gate logits as given for ``form`` -> the per-(token, head) shape
    [*lead, H, d] (elementwise) or [*lead, H] (headwise) by repeating them
    over the dims the form leaves out."""
    if gate_mode == GATE_NONE or z is None:
        return None
    z = np.asarray(z)
    row = z.shape[-1:] if gate_mode == GATE_ELEMENTWISE else ()
    if form.input_independent:
        z = z.reshape((1,) * len(lead) + z.shape)
    if form.share_heads:
        z = np.expand_dims(z, axis=z.ndim - len(row))
    return np.broadcast_to(z, tuple(lead) + (n_heads,) + tuple(row))


def softmax_rows(s: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Stable row softmax: exp(x - max) / sum exp(x - max); -inf maps to 0.

    "Attention, worked all the way through", section "Why scaling and stable
    softmax matter".
    """
    s = np.asarray(s, dtype=dtype)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     dtype=np.float64, return_weights: bool = False):
    """One head: softmax(Q K^T * scale + M) V with M = -inf above the diagonal.

    q [T,d], k [T,d], v [T,dv]. "Transformer by Hand · 6. Gated attention",
    section "The formula"; "Attention, worked all the way through", section
    "One head · explicit axes" (score, mask, row softmax, weighted read).
    """
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    T = q.shape[0]
    s = (q @ k.T) * dtype(scale)
    mask = np.triu(np.ones((T, k.shape[0]), dtype=bool), k=1)
    s = np.where(mask, -np.inf, s)
    a = softmax_rows(s, dtype=dtype)
    o = a @ v
    return (o, a) if return_weights else o


def kv_group(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Query head h reads KV head floor(h / (H/G)) ("多头注意力与 GQA", GQA section)."""
    return h // (n_q_heads // n_kv_heads)


def split_q_proj(qg: np.ndarray, head_dim: int, gate_mode: str):
    """(q, gate) from the output of a q projection that also makes the gate.

    "Transformer by Hand · 6. Gated attention", "Why the gate is packed into
    q_proj" and the forward code and shape table of "The code:
    qwen/attention.py": the projection's [.., H*2d] output, viewed per head as
    [.., H, 2d], holds each head's d query values followed by its d gate
    logits. ``qg`` is that per-head view. The pages pack only the elementwise
    gate; for a headwise gate this reads the same layout with one logit per
    head, [.., H, d+1] (query values, then the logit). Returns
    q [.., H, d] and gate [.., H, d] (elementwise) or [.., H] (headwise).
    """
    qg = np.asarray(qg)
    d = int(head_dim)
    if gate_mode == GATE_ELEMENTWISE:
        if qg.shape[-1] != 2 * d:
            raise ValueError(f"fused q/gate rows have {qg.shape[-1]} values, expected {2 * d}")
        return qg[..., :d], qg[..., d:]
    if gate_mode == GATE_HEADWISE:
        if qg.shape[-1] != d + 1:
            raise ValueError(f"fused q/gate rows have {qg.shape[-1]} values, expected {d + 1}")
        return qg[..., :d], qg[..., d]
    raise ValueError(f"a fused q/gate projection needs a gate, got gate_mode {gate_mode!r}")


def _default_scale(d: int, scale: Optional[float]) -> float:
    # 1/sqrt(head_dim): "The formula" on "Transformer by Hand · 6. Gated attention".
    return 1.0 / math.sqrt(d) if not scale else float(scale)


def prefill_keys(k, k_norm_w, positions, *, rms_eps: float, rope_base: float, rot_dim: int,
                 dtype=np.float64) -> np.ndarray:
    """K-hat = RoPE(RMSNorm(k)) for k [B,n,G,d]: what a prefill writes to a KV cache."""
    kn = rms_norm(k, k_norm_w, rms_eps, dtype=dtype)
    return rope(kn, positions, rot_dim, rope_base, dtype=dtype)


def prefill(q, k, v, gate, *, gate_mode: str, q_norm_w, k_norm_w, positions,
            rms_eps: float = 1e-6, rope_base: float = 10000.0, rot_dim: int = 0,
            scale: Optional[float] = None, dtype=np.float64, block: int = 256,
            gate_form: Optional[GateForm] = None) -> np.ndarray:
    """Gated GQA causal attention over whole sequences.

    q [B,n,H,d], k/v [B,n,G,d], gate [B,n,H,d] | [B,n,H] | None, norm weights
    [d] or None, positions [B,n] int. Returns out [B,n,H*d] (the gated head
    concat that W_O would consume). Query rows are processed in blocks of
    ``block`` rows against all keys up to the block's last row; the blocking
    does not change the result.
    """
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_finite(name, x)
    q = np.asarray(q)
    B, n, H, d = q.shape
    G = np.asarray(k).shape[2]
    if H % G:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    sc = _default_scale(d, scale)
    qh = rope(rms_norm(q, q_norm_w, rms_eps, dtype), positions, rot_dim, rope_base, dtype)
    kh = prefill_keys(k, k_norm_w, positions, rms_eps=rms_eps, rope_base=rope_base,
                      rot_dim=rot_dim, dtype=dtype)
    vv = np.asarray(v, dtype=dtype)
    y = np.empty((B, n, H, d), dtype=dtype)
    for b in range(B):
        for h in range(H):
            g = kv_group(h, H, G)
            for r0 in range(0, n, block):
                r1 = min(n, r0 + block)
                s = (qh[b, r0:r1, h] @ kh[b, :r1, g].T) * dtype(sc)       # [rows, r1]
                rows = np.arange(r0, r1)[:, None]
                s = np.where(np.arange(r1)[None, :] > rows, -np.inf, s)   # causal: j <= i
                y[b, r0:r1, h] = softmax_rows(s, dtype) @ vv[b, :r1, g]
    form = DEFAULT_GATE if gate_form is None else gate_form
    out = apply_gate(y, expand_gate(gate, gate_mode, form, (B, n), H), gate_mode, dtype=dtype, form=form)
    return out.reshape(B, n, H * d)


def prefill_row_lse(q, k, *, q_norm_w, k_norm_w, positions, rms_eps: float = 1e-6,
                    rope_base: float = 10000.0, rot_dim: int = 0, scale: Optional[float] = None,
                    rows: Optional[Sequence[tuple]] = None, dtype=np.float64) -> np.ndarray:
    """Log2 of the normalising sum of each causal softmax row.

    lse[b,i,h] = log2 sum_{j <= i} exp(s_ij), s_ij = (q_hat_i . k_hat_j) * scale,
    the denominator of softmax(QK^T/sqrt(d) + M) ("Transformer by Hand · 6.
    Gated attention", "The formula"), so a_ij = exp(s_ij) / 2^lse[b,i,h].
    Evaluated in the stable form m + log sum exp(s - m) with m the row max
    ("Attention, worked all the way through", "Why scaling and stable softmax
    matter"), then divided by ln 2. Returns [B,n,H], or with ``rows`` (a list
    of (b, i, h)) the values of those rows only.
    """
    for name, x in (("q", q), ("k", k)):
        _check_finite(name, x)
    q = np.asarray(q)
    B, n, H, d = q.shape
    G = np.asarray(k).shape[2]
    if H % G:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    sc = _default_scale(d, scale)
    kh = prefill_keys(k, k_norm_w, positions, rms_eps=rms_eps, rope_base=rope_base,
                      rot_dim=rot_dim, dtype=dtype)
    want = [(b, i, h) for b in range(B) for i in range(n) for h in range(H)] if rows is None else list(rows)
    out = np.empty(len(want), dtype=dtype)
    for t, (b, i, h) in enumerate(want):
        qh = rope(rms_norm(q[b, i:i + 1, h:h + 1], q_norm_w, rms_eps, dtype),
                  np.asarray(positions)[b, i:i + 1], rot_dim, rope_base, dtype)[0, 0]   # [T=1, 1 head, d]
        s = (kh[b, :i + 1, kv_group(h, H, G)] @ qh) * dtype(sc)       # keys j <= i
        m = np.max(s)
        out[t] = (m + np.log(np.sum(np.exp(s - m)))) / math.log(2.0)
    return out.reshape(B, n, H) if rows is None else out


def prefill_rows(q, k, v, gate, rows: Sequence[tuple], *, gate_mode: str, q_norm_w, k_norm_w,
                 positions, rms_eps: float = 1e-6, rope_base: float = 10000.0, rot_dim: int = 0,
                 scale: Optional[float] = None, dtype=np.float64,
                 gate_form: Optional[GateForm] = None) -> np.ndarray:
    """The same computation for selected (b, i, h) rows only; returns [len(rows), d].

    Used at sizes where the whole output is too expensive on the CPU.
    """
    q = np.asarray(q)
    B, n, H, d = q.shape
    G = np.asarray(k).shape[2]
    sc = _default_scale(d, scale)
    form = DEFAULT_GATE if gate_form is None else gate_form
    gate = expand_gate(gate, gate_mode, form, (B, n), H)
    out = np.empty((len(rows), d), dtype=dtype)
    khat_cache = {}
    for r, (b, i, h) in enumerate(rows):
        g = kv_group(h, H, G)
        if (b, g) not in khat_cache:
            khat_cache[(b, g)] = rope(rms_norm(np.asarray(k)[b, :, g][:, None, :], k_norm_w, rms_eps, dtype),
                                      np.asarray(positions)[b], rot_dim, rope_base, dtype)[:, 0, :]
        kh = khat_cache[(b, g)]
        qv = rope(rms_norm(q[b, i, h][None, None, :], q_norm_w, rms_eps, dtype),
                  np.asarray(positions)[b, i:i + 1], rot_dim, rope_base, dtype)[0, 0]
        s = (kh[: i + 1] @ qv) * dtype(sc)
        a = softmax_rows(s[None, :], dtype)[0]
        y = a @ np.asarray(v, dtype=dtype)[b, : i + 1, g]
        if gate_mode == GATE_ELEMENTWISE:
            zz = np.asarray(gate)[b, i, h][None, :]          # [1 head, d]
        elif gate_mode == GATE_HEADWISE:
            zz = np.asarray(gate)[b, i, h:h + 1]             # [1 head]
        else:
            zz = None
        out[r] = apply_gate(y[None, :], zz, gate_mode, dtype, form)[0]
    return out


def prefill_blocks(q, k, v, gate, blocks: Sequence[tuple], *, gate_mode: str, q_norm_w, k_norm_w,
                   positions, block_rows: int = 256, rms_eps: float = 1e-6, rope_base: float = 10000.0,
                   rot_dim: int = 0, scale: Optional[float] = None, dtype=np.float64) -> np.ndarray:
    """The definition for whole query-row blocks: for each (b, r0) in
    ``blocks``, rows r0 .. r0 + block_rows - 1 (clipped to n) of every head,
    each against keys [0, i] ("The formula": causal softmax(QK^T/sqrt(d)) V,
    GQA head h reading KV head floor(h / group)). Returns [len(blocks),
    block_rows, H*d]; rows past n are NaN. Used at sizes where the whole
    output is too expensive on the CPU; equals the matching rows of
    ``prefill``."""
    q = np.asarray(q)
    B, n, H, d = q.shape
    G = np.asarray(k).shape[2]
    sc = _default_scale(d, scale)
    pos = np.asarray(positions)
    out = np.full((len(blocks), block_rows, H * d), np.nan, dtype=dtype)
    khat = {}
    for o, (b, r0) in enumerate(blocks):
        r1 = min(n, r0 + block_rows)
        if r0 >= r1:
            continue
        if b not in khat:
            khat[b] = rope(rms_norm(np.asarray(k)[b][None], k_norm_w, rms_eps, dtype), pos[b][None], rot_dim,
                           rope_base, dtype)[0]                                   # [n, G, d]
        kh = khat[b]
        qh = rope(rms_norm(q[b, r0:r1][None], q_norm_w, rms_eps, dtype), pos[b, r0:r1][None], rot_dim,
                  rope_base, dtype)[0]                                          # [rows, H, d]
        vv = np.asarray(v)[b, :r1]
        y = np.empty((r1 - r0, H, d), dtype=dtype)
        rows = np.arange(r0, r1)[:, None]
        for h in range(H):
            g = kv_group(h, H, G)
            s = (qh[:, h] @ kh[:r1, g].T) * dtype(sc)                          # [rows, r1]
            s = np.where(np.arange(r1)[None, :] > rows, -np.inf, s)             # causal: j <= i
            y[:, h] = softmax_rows(s, dtype) @ vv[:, g].astype(dtype)
        z = None if gate is None else np.asarray(gate)[b, r0:r1][None]
        out[o, : r1 - r0] = apply_gate(y[None], z, gate_mode, dtype=dtype).reshape(r1 - r0, H * d)
    return out


def prefill_chunk(q, k, v, gate, *, gate_mode: str, q_norm_w, k_norm_w, k_cache_rows, cache_lens,
                  chunk_lens=None, positions=None, max_cache_len: Optional[int] = None, rms_eps: float = 1e-6,
                  rope_base: float = 10000.0, rot_dim: int = 0, scale: Optional[float] = None, dtype=np.float64,
                  gate_form: Optional[GateForm] = None):
    """A chunk of new tokens per sequence after the tokens already in a KV cache.

    q [B,n,H,d], k/v [B,n,G,d] (raw), gate as for ``prefill``.
    ``k_cache_rows(b)`` returns (K-hat [L_b,G,d], V [L_b,G,d]) for sequence b,
    the L_b = cache_lens[b] cached rows, used as stored. Chunk row i < n_b
    (n_b = chunk_lens[b], default n) is token L_b + i: its K-hat is
    RoPE(RMSNorm(k)) at position positions[b,i] (default L_b + i), and its
    query attends to the cached rows and to chunk rows 0..i, i.e. to cache
    slots [0, L_b + i]. Rows i >= n_b (padding), and every row of a sequence
    whose L_b lies outside [0, max_cache_len], are not computed: NaN.
    Returns (out [B,n,H*d], k_hat [B,n,G,d] of the chunk rows).

    Sources: the mask M of "Gated Attention：算完注意力，再决定用多少", section
    "门放在哪里？" (causal / padding mask), with the cache of "多头注意力与 GQA",
    section "标准多头注意力（MHA）" (history K and V kept and re-read); for one
    sequence this is rows L_b.. of ``prefill`` over the whole sequence.
    """
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_finite(name, x)
    q = np.asarray(q)
    B, n, H, d = q.shape
    G = np.asarray(k).shape[2]
    sc = _default_scale(d, scale)
    lens = np.asarray(cache_lens)
    form = DEFAULT_GATE if gate_form is None else gate_form
    gate = expand_gate(gate, gate_mode, form, (B, n), H)
    out = np.full((B, n, H, d), np.nan, dtype=dtype)
    khat = np.full((B, n, G, d), np.nan, dtype=dtype)
    for b in range(B):
        L = int(lens[b])
        nb = n if chunk_lens is None else max(0, min(n, int(np.asarray(chunk_lens)[b])))
        if L < 0 or (max_cache_len is not None and L > max_cache_len) or nb == 0:
            continue
        pos = (np.arange(L, L + nb) if positions is None else np.asarray(positions)[b, :nb])
        qh = rope(rms_norm(q[b, :nb], q_norm_w, rms_eps, dtype), pos, rot_dim, rope_base, dtype)       # [nb,H,d]
        kh = rope(rms_norm(np.asarray(k)[b, :nb], k_norm_w, rms_eps, dtype), pos, rot_dim, rope_base, dtype)
        khat[b, :nb] = kh
        kc, vc = k_cache_rows(b)
        keys = np.concatenate([np.asarray(kc, dtype=dtype)[:L], kh], axis=0)                          # [L+nb,G,d]
        vals = np.concatenate([np.asarray(vc, dtype=dtype)[:L], np.asarray(v, dtype=dtype)[b, :nb]], axis=0)
        rows = L + np.arange(nb)[:, None]                          # cache slot of each chunk row
        hidden = np.arange(L + nb)[None, :] > rows                 # causal in cache slots
        for h in range(H):
            g = kv_group(h, H, G)
            s = (qh[:, h] @ keys[:, g].T) * dtype(sc)
            s = np.where(hidden, -np.inf, s)
            out[b, :nb, h] = softmax_rows(s, dtype) @ vals[:, g]
        z = None if gate_mode == GATE_NONE else np.asarray(gate)[b, :nb]   # [nb,H,d] or [nb,H]
        out[b, :nb] = apply_gate(out[b, :nb], z, gate_mode, dtype, form)
    return out.reshape(B, n, H * d), khat


def decode(q, k_new, v_new, gate, *, gate_mode: str, q_norm_w, k_norm_w, k_cache_rows: Iterable,
           cache_lens, rms_eps: float = 1e-6, rope_base: float = 10000.0, rot_dim: int = 0,
           scale: Optional[float] = None, dtype=np.float64, seqs: Optional[Sequence[int]] = None,
           gate_form: Optional[GateForm] = None):
    """One decode step per sequence.

    q [B,H,d], k_new/v_new [B,G,d] (raw, before norm), gate [B,H,d] | [B,H].
    ``k_cache_rows(b)`` returns (K-hat [L_b,G,d], V [L_b,G,d]) for sequence b:
    the cached rows, used as stored. The new token sits at position L_b and
    attends to the L_b cached keys and to itself (causal: a row sees j <= i).
    Returns (out [len(seqs),H*d], k_hat_new [len(seqs),G,d]).

    Source: "多头注意力与 GQA", section "标准多头注意力（MHA）" (a decode step
    dots the new query with every cached key and mixes every cached value; Q
    is never cached), with the prefill definition above for one row.
    """
    q = np.asarray(q)
    B, H, d = q.shape
    G = np.asarray(k_new).shape[1]
    sc = _default_scale(d, scale)
    lens = np.asarray(cache_lens)
    seqs = list(range(B)) if seqs is None else list(seqs)
    form = DEFAULT_GATE if gate_form is None else gate_form
    gate = expand_gate(gate, gate_mode, form, (B,), H)
    out = np.empty((len(seqs), H * d), dtype=dtype)
    khn = np.empty((len(seqs), G, d), dtype=dtype)
    for r, b in enumerate(seqs):
        L = int(lens[b])
        pos = np.array([L])
        qh = rope(rms_norm(q[b][None], q_norm_w, rms_eps, dtype), pos, rot_dim, rope_base, dtype)[0]  # [H,d]
        kn = rope(rms_norm(np.asarray(k_new)[b][None], k_norm_w, rms_eps, dtype), pos, rot_dim,
                  rope_base, dtype)[0]                                                              # [G,d]
        khn[r] = kn
        kc, vc = k_cache_rows(b)
        kc = np.asarray(kc, dtype=dtype)[:L]
        vc = np.asarray(vc, dtype=dtype)[:L]
        y = np.empty((H, d), dtype=dtype)
        for h in range(H):
            g = kv_group(h, H, G)
            keys = np.concatenate([kc[:, g], kn[g][None]], axis=0)
            vals = np.concatenate([vc[:, g], np.asarray(v_new, dtype=dtype)[b, g][None]], axis=0)
            s = (keys @ qh[h]) * dtype(sc)
            y[h] = softmax_rows(s[None], dtype)[0] @ vals
        z = None if gate is None else np.asarray(gate)[b]
        out[r] = apply_gate(y, z, gate_mode, dtype, form).reshape(H * d)
    return out, khn
