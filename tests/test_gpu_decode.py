"""GPU parity of ga_decode against the fp64 CPU oracle, through the C ABI:
small ragged caches (empty, one key, several chunks), the full 64-sequence
workload, the appended cache slot, invalid lengths, and decode == the last
row of prefill."""
import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import attention as oracle
from tests.gpu_helpers import assert_close, dev, desc_for, host, tdt

pytestmark = pytest.mark.gpu


def _decode_case(name, lens, H, G, d, rot, gate, dtype="bf16", seed=200):
    return inputs.Workload(name, "decode", len(lens), 1, H, G, d, rot, dtype, gate, seed=seed,
                           extra={"lens": list(lens)})


def _run(w, lens=None, cap_extra=3):
    """Build caches on the GPU, run ga_decode, compare every sequence with the oracle."""
    et = tdt(w)
    x = inputs.make_decode(w, cache_lens=lens)
    L = x["cache_lens"]
    max_len = int(L.max())
    cap = max_len + cap_extra
    kc = torch.zeros((w.batch, cap, w.n_kv_heads, w.head_dim), dtype=et, device="cuda")
    vc = torch.zeros_like(kc)
    rows = {}

    def put(b, kh, vv):
        rows[b] = (kh, vv)
        if len(kh):
            kc[b, :len(kh)] = dev(kh, et)
            vc[b, :len(vv)] = dev(vv, et)

    inputs.for_each_cache_rows(w, L, put)
    d = desc_for(w)
    out = api.ga_decode(d, dev(x["q"], et), dev(x["k_new"], et), dev(x["v_new"], et), kc, vc,
                        dev(x["cache_lens"]), max_len, gate=dev(x["gate"], et) if x["gate"] is not None else None,
                        q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]))
    torch.cuda.synchronize()
    want, khn = oracle.decode(x["q"], x["k_new"], x["v_new"], x["gate"], gate_mode=w.gate_mode,
                              q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], k_cache_rows=lambda b: rows[b],
                              cache_lens=L, rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    return x, out, want, khn, kc, vc


@pytest.mark.parametrize("w", [
    _decode_case("fused_d256_g4", [0, 1, 700, 1536], 8, 2, 256, 64, "elementwise", seed=201),
    _decode_case("fused_d128_g2_headwise", [5, 511, 512, 513], 16, 8, 128, 32, "headwise", seed=202),
    _decode_case("fused_d64_g8_nogate", [1000, 3], 16, 2, 64, 16, "none", seed=203),
    _decode_case("fused_d128_g16", [77, 2049], 16, 1, 128, 32, "elementwise", seed=204),
    _decode_case("fused_d256_g1", [300], 2, 2, 256, 256, "elementwise", seed=205),
    _decode_case("generic_g3", [0, 40, 300], 6, 2, 128, 32, "elementwise", seed=206),
    _decode_case("generic_f32", [7, 130], 4, 2, 24, 8, "headwise", dtype="f32", seed=207),
], ids=lambda w: w.name)
def test_decode_small(w):
    print(f"[decode] {w.name}", flush=True)
    x, out, want, khn, kc, vc = _run(w, lens=np.array(w.extra["lens"], dtype=np.int32))
    assert_close(host(out), want, w, w.name)
    # appended slot L_b: new K-hat (one rounding of the oracle's) and V exactly
    for b, L in enumerate(x["cache_lens"]):
        got_k = host(kc[b, L])
        assert np.all(np.abs(got_k - khn[b]) <= np.abs(khn[b]) * 2.0 ** -8 + 1e-6)
        assert np.array_equal(host(vc[b, L]), x["v_new"][b].astype(np.float64))


def test_decode_split_boundaries():
    """Cache lengths on both sides of one, two and three key chunks of the split."""
    from gated_gqa_softmax_amd import _lib
    ck = int(_lib.load().ga_decode_split_keys())
    lens = [ck - 1, ck, ck + 1, 2 * ck, 2 * ck + 1, 3 * ck - 1]
    w = _decode_case("split_boundaries", lens, 8, 2, 256, 64, "elementwise", seed=208)
    print(f"[decode] split boundaries at {ck}-key chunks: {lens}", flush=True)
    x, out, want, khn, kc, vc = _run(w, lens=np.array(lens, dtype=np.int32))
    assert_close(host(out), want, w, w.name)


def test_decode_full_workload():
    w = inputs.WORKLOADS["decode_64seq"]
    print("[decode] decode_64seq full", flush=True)
    x, out, want, khn, kc, vc = _run(w, cap_extra=1)
    mx, mean = assert_close(host(out), want, w, "decode_64seq")
    print(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_decode_invalid_length_gives_nan_and_no_write():
    w = _decode_case("bad_len", [10, 10], 8, 2, 256, 64, "elementwise", seed=210)
    et = tdt(w)
    x = inputs.make_decode(w, cache_lens=np.array([10, 10], np.int32))
    kc = torch.zeros((2, 20, 2, 256), dtype=et, device="cuda")
    vc = torch.zeros_like(kc)
    lens = dev(np.array([10, 19], np.int32))          # 19 > max_cache_len = 12
    out = api.ga_decode(desc_for(w), dev(x["q"], et), dev(x["k_new"], et), dev(x["v_new"], et), kc, vc, lens, 12,
                        gate=dev(x["gate"], et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]))
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all()
    assert torch.isfinite(out[0].float()).all()
    assert float(kc[1].abs().max()) == 0.0 and float(vc[1].abs().max()) == 0.0


def test_decode_matches_last_prefill_row():
    """Prefill n tokens into a cache, decode token n: the output equals row n of
    a prefill over n + 1 tokens (GPU against GPU, both against the oracle)."""
    n = 1100
    w = inputs.Workload("pd", "prefill", 2, n + 1, 8, 2, 256, 64, "bf16", "elementwise", seed=220)
    et = tdt(w)
    x = inputs.make_prefill(w)
    d = desc_for(w)
    cap = n + 5
    kc = torch.zeros((2, cap, 2, 256), dtype=et, device="cuda")
    vc = torch.zeros_like(kc)
    q, k, v, g = (dev(x[t], et) for t in ("q", "k", "v", "gate"))
    wq, wk = dev(x["q_norm_w"]), dev(x["k_norm_w"])
    pos = dev(x["positions"])
    full = api.ga_prefill(d, q, k, v, g, wq, wk, pos)
    api.ga_prefill(d, q[:, :n].contiguous(), k[:, :n].contiguous(), v[:, :n].contiguous(), g[:, :n].contiguous(),
                   wq, wk, pos[:, :n].contiguous(), k_cache=kc, v_cache=vc)
    lens = dev(np.array([n, n], np.int32))
    dec = api.ga_decode(d, q[:, n].contiguous(), k[:, n].contiguous(), v[:, n].contiguous(), kc, vc, lens, n,
                        gate=g[:, n].contiguous(), q_norm_w=wq, k_norm_w=wk)
    torch.cuda.synchronize()
    want = oracle_last = oracle.prefill_rows(x["q"], x["k"], x["v"], x["gate"], [(0, n, h) for h in range(8)] +
                                            [(1, n, h) for h in range(8)], gate_mode="elementwise",
                                            q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], positions=x["positions"],
                                            rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    want = oracle_last.reshape(2, 8 * 256)
    assert_close(host(dec), want, w, "decode")
    assert_close(host(full[:, n]), want, w, "prefill last row")
    assert_close(host(dec), host(full[:, n]), w, "decode vs prefill")
    # the decode appended exactly what a prefill over n + 1 tokens would cache
    kc2 = torch.zeros_like(kc)
    vc2 = torch.zeros_like(vc)
    api.ga_prefill(d, q, k, v, g, wq, wk, pos, k_cache=kc2, v_cache=vc2)
    torch.cuda.synchronize()
    assert torch.equal(kc[:, :n], kc2[:, :n])
    assert torch.equal(vc[:, : n + 1], vc2[:, : n + 1])
    a, b = host(kc[:, n]), host(kc2[:, n])             # two kernels, one bf16 rounding apart at most
    assert np.all(np.abs(a - b) <= np.abs(b) * 2.0 ** -7 + 1e-6)


def test_decode_stages_match_fused_call():
    w = _decode_case("stages", [900, 31], 8, 2, 256, 64, "elementwise", seed=230)
    et = tdt(w)
    x = inputs.make_decode(w, cache_lens=np.array([900, 31], np.int32))
    cap = 901
    kc = torch.randn((2, cap, 2, 256), device="cuda").to(et)
    vc = torch.randn((2, cap, 2, 256), device="cuda").to(et)
    kc2, vc2 = kc.clone(), vc.clone()
    d = desc_for(w)
    args = (dev(x["q"], et), dev(x["k_new"], et), dev(x["v_new"], et))
    lens = dev(x["cache_lens"])
    gate, wq, wk = dev(x["gate"], et), dev(x["q_norm_w"]), dev(x["k_norm_w"])
    a = api.ga_decode(d, *args, kc, vc, lens, 900, gate=gate, q_norm_w=wq, k_norm_w=wk)
    ws = torch.empty(api.ga_decode_workspace_bytes(d, 900), dtype=torch.uint8, device="cuda")
    api.ga_decode_partials(d, args[0], kc2, vc2, lens, 900, ws, q_norm_w=wq)
    b = api.ga_decode_merge(d, *args, kc2, vc2, lens, 900, ws, gate=gate, q_norm_w=wq, k_norm_w=wk)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2)


def test_decode_is_deterministic():
    """Repeated ga_decode calls over the same caches give the same bits (fixed
    split and merge orders, no atomics); the appended slot is rewritten with
    the same values each time."""
    w = _decode_case("det", [3000, 17, 1025, 512], 8, 2, 256, 64, "elementwise", seed=240)
    et = tdt(w)
    lens_np = np.array(w.extra["lens"], np.int32)
    x = inputs.make_decode(w, cache_lens=lens_np)
    cap = int(lens_np.max()) + 1
    gen = torch.Generator(device="cuda").manual_seed(241)
    kc = torch.randn((4, cap, 2, 256), generator=gen, device="cuda").to(et)
    vc = torch.randn((4, cap, 2, 256), generator=gen, device="cuda").to(et)
    d = desc_for(w)
    args = (dev(x["q"], et), dev(x["k_new"], et), dev(x["v_new"], et), kc, vc, dev(lens_np), int(lens_np.max()))
    kw = dict(gate=dev(x["gate"], et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]))
    first = api.ga_decode(d, *args, **kw).clone()
    k0, v0 = kc.clone(), vc.clone()
    for _ in range(4):
        again = api.ga_decode(d, *args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(again, first)
        assert torch.equal(kc, k0) and torch.equal(vc, v0)
