"""GPU parity of ga_prefill_backward with the fp64 backward oracle, through
the C ABI: d in {64, 128, 256}, GQA groups 1, 2, 3, 4, 8 and 16, the three
gate modes, with and without the norms, ragged token counts (not multiples of
the 32-row blocks), the LDS-staged attention kernels (d = 128, 256) and the
register-operand ones (d = 64, odd groups at d = 256, or forced by
desc.bwd_kernel = plain).

Tolerance. The backward products read bf16 operands (q-hat, k-hat, dy, P,
dS) and accumulate in fp32; each gradient is stored in bf16. The gradients
have no fixed scale, so the bar is relative to each gradient tensor:
max|err| <= 2e-2 * max|want| and mean|err| <= 1e-2 * mean|want|, with the
scales floored at 1e-3 for gradients that vanish (a one-token sequence has
dq = dk = 0 exactly; the kernels give rounding residue there)."""
import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import backward as BW
from tests.gpu_helpers import dev, desc_for, host, tdt

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 2e-2, 1e-2
FLOOR = 1e-3


def _case(name, B, n, H, G, d, rot, gate, norm=True, seed=600):
    return inputs.Workload(name, "prefill", B, n, H, G, d, rot, "bf16", gate, seed=seed, extra={"norm": norm})


CASES = [
    _case("d256_g4_elem", 1, 100, 8, 2, 256, 64, "elementwise", seed=601),
    _case("d128_g1_head", 2, 70, 4, 4, 128, 32, "headwise", seed=602),
    _case("d64_g3_none_nonorm", 2, 45, 6, 2, 64, 16, "none", norm=False, seed=603),
    _case("d256_g8_elem", 1, 33, 8, 1, 256, 64, "elementwise", seed=604),
    _case("d128_g2_elem_long", 1, 300, 4, 2, 128, 32, "elementwise", seed=605),
    _case("d256_one_token", 3, 1, 8, 2, 256, 64, "elementwise", seed=606),
    _case("d128_g1_one_block_plus_one", 2, 65, 2, 2, 128, 32, "headwise", seed=607),
    _case("d64_g16_none", 1, 80, 16, 1, 64, 16, "none", seed=608),
    # the LDS-staged dq kernel: d = 128 with groups of 4 and 8, d = 256 with group 2
    _case("d128_g4_elem_staged", 2, 97, 8, 2, 128, 32, "elementwise", seed=609),
    _case("d128_g8_head_staged", 1, 200, 8, 1, 128, 32, "headwise", seed=610),
    _case("d256_g2_head_staged", 1, 130, 4, 2, 256, 64, "headwise", seed=611),
    # group 3 at d = 256: the staged dq cannot pair its dim slices, so the register-operand dq runs
    _case("d256_g3_elem_plain_dq", 1, 90, 6, 2, 256, 64, "elementwise", seed=612),
    # a RoPE width that is not a multiple of 16
    _case("d128_rot24_elem", 1, 50, 4, 2, 128, 24, "elementwise", seed=615),
]

# The register-operand kernels, forced everywhere by their switches
PLAIN_CASES = [
    _case("d256_g4_elem_plain", 1, 100, 8, 2, 256, 64, "elementwise", seed=613),
    _case("d128_g4_head_plain", 2, 77, 8, 2, 128, 32, "headwise", seed=614),
]


def _assert_rel(got, want, label):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (label, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    smax, smean = max(float(np.abs(want).max()), FLOOR), max(float(np.abs(want).mean()), FLOOR)
    assert mx <= REL_MAX * smax, f"{label}: max err {mx:.3e} vs max|want| {np.abs(want).max():.3e}"
    assert mean <= REL_MEAN * smean, f"{label}: mean err {mean:.3e} vs mean|want| {np.abs(want).mean():.3e}"
    return mx / smax, mean / smean


@pytest.mark.parametrize("w", PLAIN_CASES, ids=lambda w: w.name)
def test_backward_plain_kernels(w):
    _backward_case(w, bwd_kernel="plain")


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_small(w):
    _backward_case(w)


def _backward_case(w, bwd_kernel="auto"):
    print(f"[backward] {w.name}", flush=True)
    et = tdt(w)
    x = inputs.make_prefill(w)
    rng = np.random.default_rng(w.seed + 50)
    dout = inputs.round_bf16(rng.standard_normal((w.batch, w.seq_len, w.n_q_heads * w.head_dim)).astype(np.float32))
    wq = x["q_norm_w"] if w.extra["norm"] else None
    wk = x["k_norm_w"] if w.extra["norm"] else None
    got = api.ga_prefill_backward(desc_for(w, bwd_kernel=bwd_kernel), dev(x["q"], et), dev(x["k"], et),
                                  dev(x["v"], et), dev(dout, et), gate=dev(x["gate"], et), q_norm_w=dev(wq),
                                  k_norm_w=dev(wk), positions=dev(x["positions"]))
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


def test_backward_full_workload_sampled():
    """The 4096-token workload the bench times: sampled dq / dgate rows, dk /
    dv rows of keys near the end (every query row they need), and the column
    sums of dV, which equal the sums of dy over each group's heads whatever
    the size (each softmax row sums to one)."""
    w = inputs.WORKLOADS["qwen35_0p8b_prefill"]
    print(f"[backward] {w.name} full size", flush=True)
    et = tdt(w)
    x = inputs.make_prefill(w)
    dout = inputs.round_bf16(np.random.default_rng(w.seed + 70).standard_normal(
        (w.batch, w.seq_len, w.n_q_heads * w.head_dim)).astype(np.float32))
    got = api.ga_prefill_backward(desc_for(w), dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), dev(dout, et),
                                  gate=dev(x["gate"], et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]),
                                  positions=dev(x["positions"]))
    torch.cuda.synchronize()
    q_rows = [(0, 0, 0), (0, 1, 7), (0, 1000, 3), (0, 2049, 4), (0, 4095, 5)]
    k_rows = [(0, 4095, 0), (0, 4090, 1), (0, 4064, 0)]
    want = BW.backward_rows(x["q"], x["k"], x["v"], x["gate"], dout, q_rows=q_rows, k_rows=k_rows,
                            gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"],
                            positions=x["positions"], rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    dq, dgate, dk, dv = (host(got[k_]) for k_ in ("dq", "dgate", "dk", "dv"))
    _assert_rel(np.stack([dq[b, i, h] for b, i, h in q_rows]), want["dq"], "dq rows")
    _assert_rel(np.stack([dgate[b, i, h] for b, i, h in q_rows]), want["dgate"], "dgate rows")
    _assert_rel(np.stack([dk[b, j, g] for b, j, g in k_rows]), want["dk"], "dk rows")
    _assert_rel(np.stack([dv[b, j, g] for b, j, g in k_rows]), want["dv"], "dv rows")
    # sum over keys of dV = sum over queries and the group's heads of dy = dout * sigmoid(z)
    sig = 1.0 / (1.0 + np.exp(-x["gate"].astype(np.float64)))
    dy = dout.reshape(x["gate"].shape).astype(np.float64) * sig
    grp = w.n_q_heads // w.n_kv_heads
    for g in range(w.n_kv_heads):
        want_sum = dy[0, :, g * grp:(g + 1) * grp].sum(axis=(0, 1))
        _assert_rel(dv[0, :, g].sum(axis=0), want_sum, f"column sums of dv, group {g}")


def test_backward_batched_headwise_workload_sampled():
    """The 4 x 2048-token, d = 128, headwise-gate workload: sampled rows of
    dq, the headwise dgate, dk and dv, and the column sums of dv."""
    w = inputs.WORKLOADS["qwen3_0p6b_batched_prefill"]
    print(f"[backward] {w.name} full size", flush=True)
    et = tdt(w)
    x = inputs.make_prefill(w)
    dout = inputs.round_bf16(np.random.default_rng(w.seed + 71).standard_normal(
        (w.batch, w.seq_len, w.n_q_heads * w.head_dim)).astype(np.float32))
    got = api.ga_prefill_backward(desc_for(w), dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), dev(dout, et),
                                  gate=dev(x["gate"], et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]),
                                  positions=dev(x["positions"]))
    torch.cuda.synchronize()
    n = w.seq_len
    q_rows = [(0, 0, 0), (1, 1, 15), (2, 1000, 6), (3, 2047, 9), (3, 512, 1)]
    k_rows = [(0, n - 1, 0), (1, n - 5, 7), (3, n - 40, 3)]
    want = BW.backward_rows(x["q"], x["k"], x["v"], x["gate"], dout, q_rows=q_rows, k_rows=k_rows,
                            gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"],
                            positions=x["positions"], rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    dq, dgate, dk, dv = (host(got[k_]) for k_ in ("dq", "dgate", "dk", "dv"))
    _assert_rel(np.stack([dq[b, i, h] for b, i, h in q_rows]), want["dq"], "dq rows")
    _assert_rel(np.array([dgate[b, i, h] for b, i, h in q_rows]), want["dgate"], "dgate rows (headwise)")
    _assert_rel(np.stack([dk[b, j, g] for b, j, g in k_rows]), want["dk"], "dk rows")
    _assert_rel(np.stack([dv[b, j, g] for b, j, g in k_rows]), want["dv"], "dv rows")
    sig = 1.0 / (1.0 + np.exp(-x["gate"].astype(np.float64)))                  # [B, n, H]
    dy = dout.reshape(w.batch, n, w.n_q_heads, w.head_dim).astype(np.float64) * sig[..., None]
    grp = w.n_q_heads // w.n_kv_heads
    for b in (0, 3):
        for g in (0, w.n_kv_heads - 1):
            _assert_rel(dv[b, :, g].sum(axis=0), dy[b, :, g * grp:(g + 1) * grp].sum(axis=(0, 1)),
                        f"column sums of dv, seq {b} group {g}")
