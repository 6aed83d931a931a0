"""Shared helpers of the GPU parity tests (no test functions here)."""
from __future__ import annotations

import numpy as np
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import attention as oracle

BF16_MAX_ABS = 2e-2     # bf16 I/O, fp32 accumulation
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-4      # fp32 path


def tdt(w: inputs.Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def dev(x, dtype=None):
    """numpy -> GPU tensor. bf16 inputs are already bf16-representable, so the
    conversion is exact."""
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=dtype if dtype is not None else t.dtype)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def desc_for(w: inputs.Workload, batch=None, softmax_scale=0.0, kernel="auto", bwd_kernel="auto"):
    return api.make_desc(w.batch if batch is None else batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim,
                         w.rope_base, w.rms_eps, softmax_scale, tdt(w), w.gate_mode, kernel=kernel,
                         bwd_kernel=bwd_kernel)


def tol(w: inputs.Workload):
    return (BF16_MAX_ABS, BF16_MEAN_ABS) if w.dtype == "bf16" else (F32_MAX_ABS, F32_MAX_ABS)


def assert_close(got, want, w: inputs.Workload, label=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite GPU output"
    err = np.abs(got - want)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    max_tol, mean_tol = tol(w)
    assert mx <= max_tol and mean <= mean_tol, f"{label}: max-abs {mx:.3e} (tol {max_tol}), mean-abs {mean:.3e} (tol {mean_tol})"
    return mx, mean


def gpu_prefill(w: inputs.Workload, x: dict, with_cache=False, cap=None, softmax_scale=0.0, kernel="auto"):
    et = tdt(w)
    d = desc_for(w, softmax_scale=softmax_scale, kernel=kernel)
    q, k, v = dev(x["q"], et), dev(x["k"], et), dev(x["v"], et)
    gate = dev(x["gate"], et) if x["gate"] is not None else None
    wq = dev(x["q_norm_w"]) if x.get("q_norm_w") is not None else None
    wk = dev(x["k_norm_w"]) if x.get("k_norm_w") is not None else None
    pos = dev(x["positions"]) if x.get("positions") is not None else None
    kc = vc = None
    if with_cache:
        cap = cap or w.seq_len
        kc = torch.zeros((w.batch, cap, w.n_kv_heads, w.head_dim), dtype=et, device="cuda")
        vc = torch.zeros_like(kc)
    out = api.ga_prefill(d, q, k, v, gate, wq, wk, pos, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    return (out, kc, vc) if with_cache else out


def oracle_prefill(w: inputs.Workload, x: dict, softmax_scale=None):
    return oracle.prefill(x["q"], x["k"], x["v"], x["gate"], gate_mode=w.gate_mode, q_norm_w=x.get("q_norm_w"),
                          k_norm_w=x.get("k_norm_w"), positions=x["positions"], rms_eps=w.rms_eps,
                          rope_base=w.rope_base, rot_dim=w.rot_dim, scale=softmax_scale)
