"""GPU parity of ga_prefill_backward with the fp64 backward oracle, through
the C ABI: d in {64, 128, 256}, GQA groups 1, 3, 4 and 8, the three gate
modes, with and without the norms, ragged token counts (not multiples of the
32-row blocks).

Tolerance. The backward products read bf16 operands (q-hat, k-hat, dy, P,
dS) and accumulate in fp32; each gradient is stored in bf16. The gradients
have no fixed scale, so the bar is relative to each gradient tensor:
max|err| <= 2e-2 * max|want| and mean|err| <= 1e-2 * mean|want|."""
import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import backward as BW
from tests.gpu_helpers import dev, desc_for, host, tdt

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 2e-2, 1e-2


def _case(name, B, n, H, G, d, rot, gate, norm=True, seed=600):
    return inputs.Workload(name, "prefill", B, n, H, G, d, rot, "bf16", gate, seed=seed, extra={"norm": norm})


CASES = [
    _case("d256_g4_elem", 1, 100, 8, 2, 256, 64, "elementwise", seed=601),
    _case("d128_g1_head", 2, 70, 4, 4, 128, 32, "headwise", seed=602),
    _case("d64_g3_none_nonorm", 2, 45, 6, 2, 64, 16, "none", norm=False, seed=603),
    _case("d256_g8_elem", 1, 33, 8, 1, 256, 64, "elementwise", seed=604),
    _case("d128_g2_elem_long", 1, 300, 4, 2, 128, 32, "elementwise", seed=605),
]


def _assert_rel(got, want, label):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (label, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= REL_MAX * float(np.abs(want).max()), f"{label}: max err {mx:.3e} vs max|want| {np.abs(want).max():.3e}"
    assert mean <= REL_MEAN * float(np.abs(want).mean()), \
        f"{label}: mean err {mean:.3e} vs mean|want| {np.abs(want).mean():.3e}"
    return mx / float(np.abs(want).max()), mean / float(np.abs(want).mean())


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_small(w):
    print(f"[backward] {w.name}", flush=True)
    et = tdt(w)
    x = inputs.make_prefill(w)
    rng = np.random.default_rng(w.seed + 50)
    dout = inputs.round_bf16(rng.standard_normal((w.batch, w.seq_len, w.n_q_heads * w.head_dim)).astype(np.float32))
    wq = x["q_norm_w"] if w.extra["norm"] else None
    wk = x["k_norm_w"] if w.extra["norm"] else None
    got = api.ga_prefill_backward(desc_for(w), dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), dev(dout, et),
                                  gate=dev(x["gate"], et), q_norm_w=dev(wq), k_norm_w=dev(wk),
                                  positions=dev(x["positions"]))
    torch.cuda.synchronize()
    want = BW.prefill_backward(x["q"], x["k"], x["v"], x["gate"], dout, gate_mode=w.gate_mode, q_norm_w=wq,
                               k_norm_w=wk, positions=x["positions"], rms_eps=w.rms_eps, rope_base=w.rope_base,
                               rot_dim=w.rot_dim)
    names = ["dq", "dk", "dv"] + (["dgate"] if w.gate_mode != "none" else []) + \
        (["dq_norm_w", "dk_norm_w"] if w.extra["norm"] else [])
    for name in names:
        r = _assert_rel(host(got[name]), want[name], f"{w.name} {name}")
        print(f"  {name}: rel max {r[0]:.2e} rel mean {r[1]:.2e}", flush=True)


def test_backward_is_deterministic():
    w = CASES[0]
    et = tdt(w)
    x = inputs.make_prefill(w)
    dout = dev(inputs.round_bf16(np.random.default_rng(7).standard_normal(
        (w.batch, w.seq_len, w.n_q_heads * w.head_dim)).astype(np.float32)), et)
    args = (desc_for(w), dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), dout)
    kw = dict(gate=dev(x["gate"], et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]),
              positions=dev(x["positions"]))
    a = api.ga_prefill_backward(*args, **kw)
    b = api.ga_prefill_backward(*args, **kw)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name
