"""GPU parity of the training pair through the C ABI: ga_prefill_lse (the
output and each softmax row's log2 log-sum-exp) and ga_prefill_backward_lse
(the gradients from that output and those statistics), against the fp64
oracle: prefill, prefill_row_lse and the backward oracle.

Tolerances. out: the bf16 bars of the other prefill tests. Gradients: the
relative bars of the backward tests. lse: the kernels compute the scores from
q-hat and k-hat rounded to bf16 (unit roundoff u = 2^-8), so by
Cauchy-Schwarz each score is off by at most (2u + u^2) * scale * |q_hat| *
|k_hat|, and a log-sum-exp (a smooth maximum) moves by no more than its
largest score does; times log2 e for the log2 form, times 1.01 for the fp32
norm and rotation, plus 1e-4 for the fp32 sum and exp2/log2."""
import math

import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import attention as A
from oracle import backward as BW
from tests.gpu_helpers import assert_close, dev, desc_for, host, tdt
from tests.test_gpu_backward import _assert_rel, _case

pytestmark = pytest.mark.gpu

CASES = [
    _case("d256_g4_elem", 1, 100, 8, 2, 256, 64, "elementwise", seed=701),
    _case("d128_g1_head", 2, 70, 4, 4, 128, 32, "headwise", seed=702),
    _case("d64_g3_none_nonorm", 2, 45, 6, 2, 64, 16, "none", norm=False, seed=703),
    _case("d256_g3_elem", 1, 90, 6, 2, 256, 64, "elementwise", seed=704),
    _case("d128_g8_head", 1, 200, 8, 1, 128, 32, "headwise", seed=706),
    _case("d128_g2_elem_long", 1, 300, 4, 2, 128, 32, "elementwise", seed=707),
    # RoPE widths neither fused kernel serves (rot % 16 != 0): q-hat is prepared in the workspace
    _case("d128_rot24_elem_prepared_q", 1, 50, 4, 2, 128, 24, "elementwise", seed=708),
    _case("d64_rot8_head_prepared_q", 2, 37, 4, 2, 64, 8, "headwise", seed=709),
]


def _lse_bound(w, x, wq, wk):
    """Largest score error bf16 operands allow, in log2 units (module docstring)."""
    qh = A.rope(A.rms_norm(x["q"], wq, w.rms_eps), x["positions"], w.rot_dim, w.rope_base)
    kh = A.prefill_keys(x["k"], wk, x["positions"], rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    u = 2.0 ** -8
    qn = float(np.sqrt((qh ** 2).sum(-1)).max())
    kn = float(np.sqrt((kh ** 2).sum(-1)).max())
    return (2 * u + u * u) * qn * kn / math.sqrt(w.head_dim) * math.log2(math.e) * 1.01 + 1e-4


def _run_pair(w, x, dout, wq, wk):
    et = tdt(w)
    d = desc_for(w)
    args = (d, dev(x["q"], et), dev(x["k"], et), dev(x["v"], et))
    kw = dict(gate=dev(x["gate"], et), q_norm_w=dev(wq), k_norm_w=dev(wk), positions=dev(x["positions"]))
    out, lse = api.ga_prefill_lse(*args, **kw)
    grads = api.ga_prefill_backward(*args, dev(dout, et), out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return out, lse, grads


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_training_pair_small(w):
    print(f"[train-lse] {w.name}", flush=True)
    x = inputs.make_prefill(w)
    rng = np.random.default_rng(w.seed + 50)
    dout = inputs.round_bf16(rng.standard_normal((w.batch, w.seq_len, w.n_q_heads * w.head_dim)).astype(np.float32))
    wq = x["q_norm_w"] if w.extra["norm"] else None
    wk = x["k_norm_w"] if w.extra["norm"] else None
    out, lse, got = _run_pair(w, x, dout, wq, wk)
    kw = dict(q_norm_w=wq, k_norm_w=wk, positions=x["positions"], rms_eps=w.rms_eps, rope_base=w.rope_base,
              rot_dim=w.rot_dim)
    assert_close(host(out), A.prefill(x["q"], x["k"], x["v"], x["gate"], gate_mode=w.gate_mode, **kw), w,
                 f"{w.name} out")
    err = np.abs(host(lse) - A.prefill_row_lse(x["q"], x["k"], **kw))
    bound = _lse_bound(w, x, wq, wk)
    print(f"  lse: max err {err.max():.2e} (bound {bound:.2e}), mean {err.mean():.2e}", flush=True)
    assert err.max() <= bound
    want = BW.prefill_backward(x["q"], x["k"], x["v"], x["gate"], dout, gate_mode=w.gate_mode, **kw)
    names = ["dq", "dk", "dv"] + (["dgate"] if w.gate_mode != "none" else []) + \
        (["dq_norm_w", "dk_norm_w"] if w.extra["norm"] else [])
    for name in names:
        r = _assert_rel(host(got[name]), want[name], f"{w.name} {name}")
        print(f"  {name}: rel max {r[0]:.2e} rel mean {r[1]:.2e}", flush=True)


def test_training_pair_one_token_rows():
    """One token per sequence: the softmax has one key, so by definition
    dS = dP - rowsum(dy * y) = 0 and dq = dk = 0 (and the norm weights'
    gradients). ga_prefill_backward_lse takes the row sum from the stored
    out = bf16(y g) and dP from bf16(dy) = bf16(dout g), so per row
    |dS| <= 2^-7 sum_t |dout_t g_t v_t| (two bf16 roundings, u = 2^-8). dq,
    dk and the weight gradients are linear in dS with directions the oracle's
    norm and RoPE backward give, so each is bounded by that |dS| times those
    directions (x 1.01 for their bf16 and fp32 roundings). out, lse, dv and
    dgate are compared with the oracle at the usual bars."""
    w = _case("d256_one_token", 3, 1, 8, 2, 256, 64, "elementwise", seed=705)
    print(f"[train-lse] {w.name}", flush=True)
    x = inputs.make_prefill(w)
    dout = inputs.round_bf16(np.random.default_rng(w.seed + 50).standard_normal(
        (w.batch, 1, w.n_q_heads * w.head_dim)).astype(np.float32))
    wq, wk, pos = x["q_norm_w"], x["k_norm_w"], x["positions"]
    out, lse, got = _run_pair(w, x, dout, wq, wk)
    kw = dict(q_norm_w=wq, k_norm_w=wk, positions=pos, rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    assert_close(host(out), A.prefill(x["q"], x["k"], x["v"], x["gate"], gate_mode=w.gate_mode, **kw), w, "out")
    assert np.abs(host(lse) - A.prefill_row_lse(x["q"], x["k"], **kw)).max() <= _lse_bound(w, x, wq, wk)
    want = BW.prefill_backward(x["q"], x["k"], x["v"], x["gate"], dout, gate_mode=w.gate_mode, **kw)
    for name in ("dv", "dgate"):
        _assert_rel(host(got[name]), want[name], f"{w.name} {name}")
    B, H, G, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    grp, sc = H // G, 1.0 / math.sqrt(d)
    qh = A.rope(A.rms_norm(x["q"], wq, w.rms_eps), pos, w.rot_dim, w.rope_base)          # [B,1,H,d]
    kh = A.prefill_keys(x["k"], wk, pos, rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    g = 1.0 / (1.0 + np.exp(-x["gate"].astype(np.float64)))                               # [B,1,H,d]
    dv_ = dout.reshape(B, 1, H, d).astype(np.float64)
    bound_dq = np.zeros((B, 1, H, d))
    bound_dk = np.zeros((B, 1, G, d))
    bound_wq = np.zeros(d)
    bound_wk = np.zeros(d)
    for b in range(B):
        for h in range(H):
            kv = h // grp
            beta = 2.0 ** -7 * np.abs(dv_[b, 0, h] * g[b, 0, h] * x["v"][b, 0, kv]).sum()
            back = lambda up, xin, wgt: BW.rms_norm_backward(
                xin[None, None], wgt, w.rms_eps, BW.rope_backward(up[None, None], pos[b, :1], w.rot_dim, w.rope_base))
            uq, wq_dir = back(kh[b, 0, kv] * sc, x["q"][b, 0, h], wq)
            uk, wk_dir = back(qh[b, 0, h] * sc, x["k"][b, 0, kv], wk)
            bound_dq[b, 0, h] += beta * np.abs(uq[0, 0])
            bound_dk[b, 0, kv] += beta * np.abs(uk[0, 0])
            bound_wq += beta * np.abs(wq_dir)
            bound_wk += beta * np.abs(wk_dir)
    for name, bound in (("dq", bound_dq), ("dk", bound_dk), ("dq_norm_w", bound_wq), ("dk_norm_w", bound_wk)):
        val = np.abs(host(got[name]))
        assert np.all(val <= bound * 1.01 + 1e-7), f"{name}: {val.max():.3e} vs bound {bound.max():.3e}"
        print(f"  {name}: max {val.max():.2e}, bound max {bound.max():.2e}", flush=True)


def test_training_pair_is_deterministic_and_matches_the_recomputing_backward():
    """Two runs of the pair agree bit for bit; the gradients equal those of
    ga_prefill_backward (which recomputes the statistics) up to the bf16
    roundings of out versus y."""
    w = CASES[0]
    x = inputs.make_prefill(w)
    dout = inputs.round_bf16(np.random.default_rng(9).standard_normal(
        (w.batch, w.seq_len, w.n_q_heads * w.head_dim)).astype(np.float32))
    a = _run_pair(w, x, dout, x["q_norm_w"], x["k_norm_w"])
    b = _run_pair(w, x, dout, x["q_norm_w"], x["k_norm_w"])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for name in a[2]:
        assert torch.equal(a[2][name], b[2][name]), name
    et = tdt(w)
    ref = api.ga_prefill_backward(desc_for(w), dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), dev(dout, et),
                                  gate=dev(x["gate"], et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]),
                                  positions=dev(x["positions"]))
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dgate", "dq_norm_w", "dk_norm_w"):
        _assert_rel(host(a[2][name]), host(ref[name]), f"{name} against the recomputing backward")


def test_training_pair_full_workload_sampled():
    """The 4096-token d = 256 workload the bench times: sampled rows of out,
    lse, dq and dgate, dk / dv rows of keys near the end, and the column sums
    of dV (the sums of dy over each group's heads at any size)."""
    w = inputs.WORKLOADS["qwen35_0p8b_prefill"]
    print(f"[train-lse] {w.name} full size", flush=True)
    x = inputs.make_prefill(w)
    dout = inputs.round_bf16(np.random.default_rng(w.seed + 72).standard_normal(
        (w.batch, w.seq_len, w.n_q_heads * w.head_dim)).astype(np.float32))
    out, lse, got = _run_pair(w, x, dout, x["q_norm_w"], x["k_norm_w"])
    kw = dict(q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], positions=x["positions"], rms_eps=w.rms_eps,
              rope_base=w.rope_base, rot_dim=w.rot_dim)
    q_rows = [(0, 0, 0), (0, 1, 7), (0, 1000, 3), (0, 2049, 4), (0, 4095, 5), (0, 3333, 1)]
    k_rows = [(0, 4095, 0), (0, 4090, 1), (0, 4064, 0)]
    d = w.head_dim
    o = host(out).reshape(w.batch, w.seq_len, w.n_q_heads, d)
    assert_close(np.stack([o[b, i, h] for b, i, h in q_rows]),
                 A.prefill_rows(x["q"], x["k"], x["v"], x["gate"], q_rows, gate_mode=w.gate_mode, **kw), w, "out rows")
    got_lse = host(lse)
    err = np.abs(np.array([got_lse[r] for r in q_rows]) - A.prefill_row_lse(x["q"], x["k"], rows=q_rows, **kw))
    assert err.max() <= _lse_bound(w, x, x["q_norm_w"], x["k_norm_w"]), err
    want = BW.backward_rows(x["q"], x["k"], x["v"], x["gate"], dout, q_rows=q_rows, k_rows=k_rows,
                            gate_mode=w.gate_mode, **kw)
    dq, dgate, dk, dv = (host(got[k_]) for k_ in ("dq", "dgate", "dk", "dv"))
    _assert_rel(np.stack([dq[b, i, h] for b, i, h in q_rows]), want["dq"], "dq rows")
    _assert_rel(np.stack([dgate[b, i, h] for b, i, h in q_rows]), want["dgate"], "dgate rows")
    _assert_rel(np.stack([dk[b, j, g] for b, j, g in k_rows]), want["dk"], "dk rows")
    _assert_rel(np.stack([dv[b, j, g] for b, j, g in k_rows]), want["dv"], "dv rows")
    sig = 1.0 / (1.0 + np.exp(-x["gate"].astype(np.float64)))
    dy = dout.reshape(x["gate"].shape).astype(np.float64) * sig
    grp = w.n_q_heads // w.n_kv_heads
    for g in range(w.n_kv_heads):
        _assert_rel(dv[0, :, g].sum(axis=0), dy[0, :, g * grp:(g + 1) * grp].sum(axis=(0, 1)),
                    f"column sums of dv, group {g}")
