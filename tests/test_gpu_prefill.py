"""GPU parity of ga_prefill against the fp64 CPU oracle (element by element),
at sizes spanning several key tiles with ragged tails, at the full workload
sizes, and on the method's special cases. Every call goes through the C ABI."""
import math

import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import attention as oracle
from tests.conftest import load_golden
from tests.gpu_helpers import (assert_close, dev, desc_for, gpu_prefill, host, oracle_prefill, tdt)

pytestmark = pytest.mark.gpu

W = inputs.Workload


def _case(name, B, n, H, G, d, rot, gate, dtype="bf16", seed=100):
    return W(name, "prefill", B, n, H, G, d, rot, dtype, gate, seed=seed)


SMALL_CASES = [
    # fused MFMA kernel, every head_dim it serves, groups 1..16, ragged n
    _case("d256_g4_n300", 1, 300, 8, 2, 256, 64, "elementwise", seed=101),
    _case("d128_g2_b2_n130", 2, 130, 16, 8, 128, 32, "headwise", seed=102),
    _case("d128_g8_n200", 1, 200, 32, 4, 128, 32, "elementwise", seed=103),
    _case("d64_g1_n77_nogate", 1, 77, 4, 4, 64, 16, "none", seed=104),
    _case("d256_g4_n1", 1, 1, 8, 2, 256, 64, "elementwise", seed=105),
    _case("d128_g3_n17", 1, 17, 6, 2, 128, 32, "elementwise", seed=106),        # 128 % group != 0
    _case("d128_g16_full_rope", 1, 65, 16, 1, 128, 128, "elementwise", seed=107),
    _case("d128_g1_full_rope_no_table", 1, 150, 2, 2, 128, 128, "headwise", seed=108),
    _case("d256_g2_b3_n97", 3, 97, 4, 2, 256, 0, "headwise", seed=109),          # no RoPE
    _case("d128_g128", 1, 20, 128, 1, 128, 32, "elementwise", seed=113),         # group > 64: first design
    _case("d256_g64_n40", 1, 40, 64, 1, 256, 64, "headwise", seed=114),
    # generic kernel (fp32, or bf16 shapes without a fused kernel)
    _case("f32_d24_g2", 2, 33, 4, 2, 24, 8, "headwise", dtype="f32", seed=110),
    _case("bf16_d96_g2", 1, 40, 4, 2, 96, 24, "elementwise", seed=111),
    _case("bf16_d128_rot8", 1, 50, 4, 1, 128, 8, "elementwise", seed=112),
]


@pytest.mark.parametrize("w", SMALL_CASES, ids=lambda w: w.name)
def test_prefill_small_shapes(w):
    print(f"[prefill] {w.name}", flush=True)
    x = inputs.make_prefill(w)
    got = host(gpu_prefill(w, x))
    want = oracle_prefill(w, x)
    assert_close(got, want, w, w.name)


# Each fused kernel forced (the descriptor's kernel field) on the shapes it
# serves, so the kernels that the automatic choice keeps for large grids are
# also checked on small ragged ones: several blocks, partial last blocks and
# stages, groups that do not divide the block, full-width RoPE, single tokens.
KERNEL_CASES = [
    ("wide", _case("d128_g2_b2_n130", 2, 130, 16, 8, 128, 32, "headwise", seed=102)),
    ("wide", _case("d128_g8_n200", 1, 200, 32, 4, 128, 32, "elementwise", seed=103)),
    ("wide", _case("d128_g3_n17", 1, 17, 6, 2, 128, 32, "elementwise", seed=106)),
    ("wide", _case("d128_g16_full_rope", 1, 65, 16, 1, 128, 128, "elementwise", seed=107)),
    ("wide", _case("d128_g1_n300_full_rope", 1, 300, 2, 2, 128, 128, "headwise", seed=108)),
    ("wide", _case("d128_g128_n3", 1, 3, 128, 1, 128, 32, "elementwise", seed=113)),
    ("wide", _case("d128_g4_n700", 1, 700, 8, 2, 128, 32, "elementwise", seed=115)),
    ("wide", _case("d128_g2_n1_nogate", 2, 1, 4, 2, 128, 0, "none", seed=116)),
    ("mirror", _case("d256_g4_n300", 1, 300, 8, 2, 256, 64, "elementwise", seed=101)),
    ("mirror", _case("d256_g4_b2_n1000", 2, 1000, 8, 2, 256, 64, "headwise", seed=122)),
    ("mirror", _case("d256_g4_n129_nogate", 1, 129, 8, 2, 256, 64, "none", seed=123)),
    ("mirror", _case("d256_g2_n37", 1, 37, 4, 2, 256, 64, "elementwise", seed=124)),
    # d = 256 with rot < 64 takes the tabled RoPE path of the q prologue
    ("mirror", _case("d256_g4_n200_rot32", 1, 200, 8, 2, 256, 32, "elementwise", seed=127)),
    ("mirror", _case("d256_g2_b2_n150_rot48", 2, 150, 4, 2, 256, 48, "headwise", seed=128)),
    ("mirror", _case("d128_g8_n200", 1, 200, 32, 4, 128, 32, "elementwise", seed=103)),
    ("mirror", _case("d128_g4_n700", 1, 700, 8, 2, 128, 32, "elementwise", seed=115)),
    ("simple", _case("d128_g2_b2_n130", 2, 130, 16, 8, 128, 32, "headwise", seed=102)),
    ("simple", _case("d256_g4_n300", 1, 300, 8, 2, 256, 64, "elementwise", seed=101)),
    ("generic", _case("d128_g4_n150_generic", 1, 150, 8, 2, 128, 32, "elementwise", seed=129)),
]


@pytest.mark.parametrize("kernel,w", KERNEL_CASES, ids=lambda v: v if isinstance(v, str) else v.name)
def test_prefill_forced_kernel(kernel, w):
    print(f"[prefill:{kernel}] {w.name}", flush=True)
    assert api.ga_prefill_attention_kernel(desc_for(w, kernel=kernel), w.seq_len) == kernel
    x = inputs.make_prefill(w)
    got = host(gpu_prefill(w, x, kernel=kernel))
    assert_close(got, oracle_prefill(w, x), w, f"{kernel}:{w.name}")


def test_forced_kernel_that_does_not_serve_the_shape_is_an_error():
    w = _case("d256_wide", 1, 64, 8, 2, 256, 64, "elementwise", seed=133)
    x = inputs.make_prefill(w)
    with pytest.raises(api.GaError, match="UNSUPPORTED"):
        gpu_prefill(w, x, kernel="wide")


def test_prefill_peaky_rows():
    """Norm weight x4 makes softmax rows peaky, stressing the running-max rescale.

    Not one of the workloads: its bound is derived, not quoted. The kernel
    rounds q-hat to bf16 (relative error <= 2^-9 per element) for the MFMA, so
    the score error grows with |q-hat|; scaling q-hat by 4 scales the score
    error, and the output error it causes, by about 4. The max-abs bound is
    therefore 4x the workloads' 2e-2; mean-abs keeps the workloads' 2e-3. A
    wrong rescale of the running max gives errors of order 1.
    """
    w = _case("peaky", 1, 257, 8, 2, 256, 64, "elementwise", seed=120)
    x = inputs.make_prefill(w)
    x["q_norm_w"] = x["q_norm_w"] * np.float32(4.0)
    err = np.abs(host(gpu_prefill(w, x)) - oracle_prefill(w, x))
    assert err.max() <= 4 * 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())


def test_prefill_positions_offset():
    """Positions feed RoPE only: a sequence placed at positions 1000.. differs
    from 0.. and matches the oracle at those positions."""
    w = _case("posoff", 2, 70, 8, 2, 128, 32, "elementwise", seed=121)
    x = inputs.make_prefill(w)
    x["positions"] = (x["positions"] + np.array([[1000], [5]], dtype=np.int32)).astype(np.int32)
    assert_close(host(gpu_prefill(w, x)), oracle_prefill(w, x), w, "posoff")


@pytest.mark.parametrize("name", ["toy", "qwen35_0p8b_prefill", "qwen3_0p6b_batched_prefill"])
def test_prefill_full_workloads(name):
    w = inputs.WORKLOADS[name]
    print(f"[prefill] {name} full", flush=True)
    x = inputs.make_prefill(w)
    got = host(gpu_prefill(w, x))
    want = oracle_prefill(w, x)
    mx, mean = assert_close(got, want, w, name)
    print(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_prefill_long_context_sampled_blocks():
    """32K-token workload (B=1, n=32768, 32/4 heads, d=128): the whole output
    on the GPU, in the launch configuration the bench times; 16 seeded blocks
    of 256 query rows (the last block included) x all 32 heads re-derived by
    the oracle's blocked call and compared element by element."""
    w = inputs.WORKLOADS["moe_long_context_prefill"]
    print("[prefill] moe_long_context_prefill: GPU", flush=True)
    x = inputs.make_prefill(w)
    assert api.ga_prefill_attention_kernel(desc_for(w), w.seq_len) == "wide"
    out = gpu_prefill(w, x)
    assert bool(torch.isfinite(out).all()), "non-finite output"
    starts = inputs.sample_row_blocks(w, 16, 256)
    got = np.stack([host(out[0, r0:r0 + 256]) for r0 in starts])
    del out
    print(f"[prefill] moe_long_context_prefill: oracle on blocks {starts}", flush=True)
    want = oracle.prefill_blocks(x["q"], x["k"], x["v"], x["gate"], [(0, r0) for r0 in starts],
                                 gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"],
                                 positions=x["positions"], rms_eps=w.rms_eps, rope_base=w.rope_base,
                                 rot_dim=w.rot_dim)
    mx, mean = assert_close(got, want, w, "long-context blocks")
    print(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_three_token_page_example_on_gpu():
    """The pages' three-token example (d = 2), zero-padded to d = 8 in fp32 with
    the page's 1/sqrt(2) scale: padding q and k with zeros leaves every dot
    product unchanged, padding v adds zero output columns."""
    g = load_golden("three_token_example.json")
    pad = lambda a: np.pad(np.array(a, dtype=np.float32), ((0, 0), (0, 6)))
    w = _case("three_token", 1, 3, 1, 1, 8, 0, "none", dtype="f32")
    x = dict(q=pad(g["queries"])[None, :, None], k=pad(g["keys"])[None, :, None], v=pad(g["values"])[None, :, None],
             gate=None, q_norm_w=None, k_norm_w=None, positions=np.arange(3, dtype=np.int32)[None])
    out = host(gpu_prefill(w, x, softmax_scale=1 / math.sqrt(2)))
    assert list(np.round(out[0, 2, :2], 3)) == g["row2_output_3dp"]
    assert np.all(out[0, :, 2:] == 0)


def test_two_by_two_page_example_on_gpu():
    g = load_golden("two_by_two_known_answer.json")
    pad = lambda a: np.pad(np.array(a, dtype=np.float32), ((0, 0), (0, 6)))
    w = _case("two_by_two", 1, 2, 1, 1, 8, 0, "none", dtype="f32")
    x = dict(q=pad(g["Q"])[None, :, None], k=pad(g["K"])[None, :, None], v=pad(g["V"])[None, :, None], gate=None,
             q_norm_w=None, k_norm_w=None, positions=None)
    x["positions"] = np.arange(2, dtype=np.int32)[None]
    out = host(gpu_prefill(w, x, softmax_scale=1 / math.sqrt(2)))
    assert np.allclose(out[0, :, :2], g["O"], atol=2e-6, rtol=0)


def test_gate_special_cases_are_exact():
    """Zero logits give exactly half of the ungated output; logits of +100
    reproduce it exactly (sigmoid is 1.0 in fp32); -100 silences the head."""
    base = _case("gate_special", 1, 160, 8, 2, 128, 32, "none", seed=130)
    x = inputs.make_prefill(base)
    plain = gpu_prefill(base, x)
    we = base.with_(gate_mode="elementwise")
    wh = base.with_(gate_mode="headwise")
    shape_e = x["q"].shape
    xe = dict(x, gate=np.zeros(shape_e, np.float32))
    half = gpu_prefill(we, xe)
    assert torch.equal(half, plain * 0.5)
    xh = dict(x, gate=np.full(shape_e[:3], 100.0, np.float32))
    assert torch.equal(gpu_prefill(wh, xh), plain)
    xo = dict(x, gate=np.full(shape_e, -100.0, np.float32))
    assert float(gpu_prefill(we, xo).abs().max()) == 0.0


def test_prefill_is_deterministic():
    w = _case("det", 1, 513, 8, 2, 256, 64, "elementwise", seed=131)
    x = inputs.make_prefill(w)
    a = gpu_prefill(w, x)
    b = gpu_prefill(w, x)
    assert torch.equal(a, b)


def test_prefill_cache_write_and_stages():
    """With a cache, slots [0, n) hold K-hat (within one bf16 rounding of the
    oracle's) and V exactly; the two stage calls give the same output as the
    fused call."""
    w = _case("cache", 2, 90, 8, 2, 256, 64, "elementwise", seed=132)
    x = inputs.make_prefill(w)
    out, kc, vc = gpu_prefill(w, x, with_cache=True, cap=100)
    kh = oracle.prefill_keys(x["k"], x["k_norm_w"], x["positions"], rms_eps=w.rms_eps, rope_base=w.rope_base,
                             rot_dim=w.rot_dim)
    got_k = host(kc[:, :90])
    ulp = np.abs(kh) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(got_k - kh) <= ulp)
    assert np.array_equal(host(vc[:, :90]), x["v"].astype(np.float64))
    assert float(kc[:, 90:].abs().max()) == 0.0
    # same result as the no-cache call and as the two stages
    assert torch.equal(out, gpu_prefill(w, x))
    et = tdt(w)
    d = desc_for(w)
    khat = api.ga_prefill_keys(d, dev(x["k"], et), None, dev(x["k_norm_w"]), dev(x["positions"]))
    o2 = api.ga_prefill_attention(d, dev(x["q"], et), khat, dev(x["v"], et), dev(x["gate"], et), dev(x["q_norm_w"]),
                                  dev(x["positions"]), k_norm_w=dev(x["k_norm_w"]))
    torch.cuda.synchronize()
    assert torch.equal(o2, out)
