"""GPU parity of the chunked prefill against a KV cache (ga_prefill_chunk and
its two stages) with the fp64 CPU oracle, through the C ABI: per-sequence
cache lengths (empty, short, several stages), padding rows, skipped
sequences, both kernels (mirrored with key offsets, generic), the cache slots
written and those left alone, chunk rows == rows of a whole-sequence prefill,
and sampled rows at the full size the bench times."""
import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import attention as oracle
from tests.gpu_helpers import assert_close, dev, desc_for, host, tdt

pytestmark = pytest.mark.gpu

SENT_OUT, SENT_CACHE = 5.0, 3.0   # values the call must leave where it writes nothing


def _case(name, B, n, H, G, d, rot, gate, lens, chunk_lens=None, max_len=None, dtype="bf16", seed=300):
    return inputs.Workload(name, "prefill", B, n, H, G, d, rot, dtype, gate, seed=seed,
                           extra={"lens": list(lens), "chunk_lens": chunk_lens,
                                  "max_len": max(lens) if max_len is None else max_len})


def _run(w, stages=False, kernel="auto", bound=True):
    et = tdt(w)
    x = inputs.make_prefill(w)
    B, n, G, d = w.batch, w.seq_len, w.n_kv_heads, w.head_dim
    L = np.array(w.extra["lens"], dtype=np.int32)
    cl = None if w.extra["chunk_lens"] is None else np.array(w.extra["chunk_lens"], dtype=np.int32)
    max_len = w.extra["max_len"]
    cap = max(max_len, int(L.max())) + n + 2
    gen = torch.Generator().manual_seed(w.seed + 1)
    # cached prefix rows (K-hat and V as stored: storage-dtype values), seeded
    kc = torch.full((B, cap, G, d), SENT_CACHE, dtype=et, device="cuda")
    vc = torch.full_like(kc, SENT_CACHE)
    prefix = {}
    for b in range(B):
        kp = torch.randn((int(L[b]), G, d), generator=gen).to(et)
        vp = torch.randn((int(L[b]), G, d), generator=gen).to(et)
        if L[b] > 0 and L[b] <= max_len:
            kc[b, :L[b]] = kp.cuda()
            vc[b, :L[b]] = vp.cuda()
        prefix[b] = (kp.double().numpy(), vp.double().numpy())
    kc0, vc0 = kc.clone(), vc.clone()
    out = torch.full((B, n, w.n_q_heads * d), SENT_OUT, dtype=et, device="cuda")
    d_ = desc_for(w, kernel=kernel)
    q, k, v = dev(x["q"], et), dev(x["k"], et), dev(x["v"], et)
    gate = dev(x["gate"], et) if x["gate"] is not None else None
    wq, wk = dev(x["q_norm_w"]), dev(x["k_norm_w"])
    lens_d, cl_d = dev(L), (dev(cl) if cl is not None else None)
    if stages:
        api.ga_prefill_chunk_keys(d_, k, v, kc, vc, lens_d, max_len, k_norm_w=wk, chunk_lens=cl_d)
        # without k_norm_w the kernel has no score bound and keeps a running max
        api.ga_prefill_chunk_attention(d_, q, kc, vc, lens_d, max_len, gate=gate, q_norm_w=wq,
                                       k_norm_w=wk if bound else None, chunk_lens=cl_d, out=out)
    else:
        api.ga_prefill_chunk(d_, q, k, v, kc, vc, lens_d, max_len, gate=gate, q_norm_w=wq, k_norm_w=wk,
                             chunk_lens=cl_d, out=out)
    torch.cuda.synchronize()
    want, khat = oracle.prefill_chunk(x["q"], x["k"], x["v"], x["gate"], gate_mode=w.gate_mode,
                                      q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"],
                                      k_cache_rows=lambda b: prefix[b], cache_lens=L, chunk_lens=cl,
                                      max_cache_len=max_len, rms_eps=w.rms_eps, rope_base=w.rope_base,
                                      rot_dim=w.rot_dim)
    got = host(out)
    for b in range(B):
        nb = n if cl is None else max(0, min(n, int(cl[b])))
        skipped = L[b] < 0 or L[b] > max_len
        if skipped:
            nb = 0
        if nb:
            assert_close(got[b, :nb], want[b, :nb], w, f"{w.name} seq {b}")
            # cache slots [L, L + nb): K-hat (one rounding of the oracle's) and V exactly
            gk = host(kc[b, L[b]:L[b] + nb])
            assert np.all(np.abs(gk - khat[b, :nb]) <= np.abs(khat[b, :nb]) * 2.0 ** -7 + 1e-5), f"{w.name} K-hat {b}"
            assert np.array_equal(host(vc[b, L[b]:L[b] + nb]), x["v"][b, :nb].astype(np.float64))
        assert np.all(got[b, nb:] == SENT_OUT), f"{w.name} seq {b}: rows past {nb} were written"
        lo = L[b] + nb if not skipped else 0
        assert torch.equal(kc[b, lo:], kc0[b, lo:]) and torch.equal(vc[b, lo:], vc0[b, lo:]), f"{w.name} cache {b}"
        if not skipped:
            assert torch.equal(kc[b, :L[b]], kc0[b, :L[b]]), f"{w.name} prefix {b} changed"
    return got, want


CASES = [
    _case("mirror_d256_rot64_elem_ragged", 3, 100, 8, 2, 256, 64, "elementwise", [0, 37, 130], [100, 64, 1],
          seed=301),
    _case("mirror_d128_rot32_head", 2, 70, 16, 8, 128, 32, "headwise", [5, 300], seed=302),
    _case("mirror_d256_rot32_nogate_stages", 1, 129, 8, 2, 256, 32, "none", [257], seed=303),
    _case("mirror_d256_g4_skip", 3, 40, 8, 2, 256, 64, "elementwise", [10, 999, 0], [40, 40, 0], max_len=64,
          seed=304),
    _case("generic_f32_d8", 2, 9, 2, 1, 8, 2, "elementwise", [3, 0], [9, 4], dtype="f32", seed=305),
    _case("generic_bf16_d64_head", 2, 33, 4, 2, 64, 16, "headwise", [100, 1], seed=306),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_chunk_small(w):
    print(f"[chunk] {w.name}", flush=True)
    want_kernel = "generic" if w.name.startswith("generic") else "mirror"
    cap = max(w.extra["max_len"], max(w.extra["lens"])) + w.seq_len + 2
    assert api.ga_prefill_chunk_kernel(desc_for(w), w.seq_len, cap) == want_kernel
    _run(w, stages=w.name.endswith("stages"))


def test_chunk_running_max_form():
    """The attention stage without k_norm_w: the mirrored kernel's running-max
    softmax instead of the bounded one, same results."""
    w = CASES[0]
    print(f"[chunk] {w.name} without the score bound", flush=True)
    _run(w, stages=True, bound=False)


def test_chunk_forced_generic_kernel():
    w = CASES[0]
    print(f"[chunk] {w.name} on the generic kernel", flush=True)
    assert api.ga_prefill_chunk_kernel(desc_for(w, kernel="generic"), w.seq_len, 400) == "generic"
    _run(w, kernel="generic")


def _whole_vs_chunk(B, T, L, H, G, d, rot, gate, seed, sample_rows=None):
    """Prefill the first L tokens into a cache, then the rest as a chunk; the
    chunk rows must equal rows L.. of a prefill over all T tokens."""
    w = inputs.Workload("whole", "prefill", B, T, H, G, d, rot, "bf16", gate, seed=seed)
    et = tdt(w)
    x = inputs.make_prefill(w)
    dsc = desc_for(w)
    q, k, v = (dev(x[t], et) for t in ("q", "k", "v"))
    g = dev(x["gate"], et) if x["gate"] is not None else None
    wq, wk, pos = dev(x["q_norm_w"]), dev(x["k_norm_w"]), dev(x["positions"])
    cap = T + 8
    kc = torch.zeros((B, cap, G, d), dtype=et, device="cuda")
    vc = torch.zeros_like(kc)
    cut = lambda t, a, b_: t[:, a:b_].contiguous() if t is not None else None
    api.ga_prefill(dsc, cut(q, 0, L), cut(k, 0, L), cut(v, 0, L), cut(g, 0, L), wq, wk, cut(pos, 0, L),
                   k_cache=kc, v_cache=vc)
    lens = dev(np.full(B, L, np.int32))
    part = api.ga_prefill_chunk(dsc, cut(q, L, T), cut(k, L, T), cut(v, L, T), kc, vc, lens, L, gate=cut(g, L, T),
                                q_norm_w=wq, k_norm_w=wk)
    torch.cuda.synchronize()
    return w, x, host(part), kc


def test_chunk_rows_equal_whole_prefill_rows():
    B, T, L, H, G, d = 2, 1500, 1000, 8, 2, 256
    print(f"[chunk] whole vs chunk T={T} L={L}", flush=True)
    w, x, part, _ = _whole_vs_chunk(B, T, L, H, G, d, 64, "elementwise", seed=310)
    et = tdt(w)
    full = api.ga_prefill(desc_for(w), *(dev(x[t], et) for t in ("q", "k", "v", "gate")), dev(x["q_norm_w"]),
                          dev(x["k_norm_w"]), dev(x["positions"]))
    torch.cuda.synchronize()
    assert_close(part, host(full[:, L:]), w, "chunk vs whole prefill")
    rows = [(b, i, h) for b in range(B) for i in (L, L + 1, L + 255, T - 1) for h in (0, 5)]
    want = oracle.prefill_rows(x["q"], x["k"], x["v"], x["gate"], rows, gate_mode="elementwise",
                               q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], positions=x["positions"],
                               rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    got = np.stack([part[b, i - L, h * d:(h + 1) * d] for b, i, h in rows])
    assert_close(got, want, w, "chunk rows vs oracle")


def test_chunk_full_size_sampled_rows():
    """The size the bench times: 3072 cached tokens + a 1024-token chunk of the
    Qwen3.5-0.8B attention shape (H8 G2 d256 rot64, elementwise gate)."""
    B, T, L, H, G, d = 1, 4096, 3072, 8, 2, 256
    print(f"[chunk] full size T={T} L={L}", flush=True)
    w, x, part, _ = _whole_vs_chunk(B, T, L, H, G, d, 64, "elementwise", seed=311)
    rows = [(0, i, h) for i in (L, L + 1, L + 63, L + 64, L + 511, T - 2, T - 1) for h in (0, 3, 7)]
    want = oracle.prefill_rows(x["q"], x["k"], x["v"], x["gate"], rows, gate_mode="elementwise",
                               q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], positions=x["positions"],
                               rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    got = np.stack([part[0, i - L, h * d:(h + 1) * d] for _, i, h in rows])
    assert np.all(np.isfinite(part))
    assert_close(got, want, w, "full-size chunk rows")


def test_chunk_bench_workload_in_full():
    """The mixed-length chunk workload the bench times (four 1024-token chunks
    of the Qwen3.5-0.8B attention shape after 0, 1024, 2048 and 3072 cached
    tokens, elementwise gate), in its launch configuration, compared with the
    oracle on every row of every sequence (and the cache slots written)."""
    wb = inputs.WORKLOADS["qwen35_0p8b_chunk"]
    w = wb.with_(extra={"lens": list(wb.extra["cache_lens"]), "chunk_lens": None,
                        "max_len": max(wb.extra["cache_lens"])})
    print(f"[chunk] {wb.name} in full", flush=True)
    d = desc_for(w)
    assert api.ga_prefill_chunk_kernel(d, w.seq_len, max(w.extra["lens"]) + w.seq_len + 2) == "mirror"
    got, want = _run(w)
    assert np.all(np.isfinite(got))


# Cached prefixes of very different lengths in one call (one sequence with a
# prefix 25x the chunk), ragged chunk lengths, three gate forms.
SKEW_CASES = [
    _case("skew_d256_elementwise", 3, 256, 8, 2, 256, 64, "elementwise", [0, 6000, 100], [256, 200, 17], seed=320),
    _case("skew_d128_headwise", 4, 128, 16, 8, 128, 32, "headwise", [4000, 0, 2500, 64], seed=321),
    _case("skew_d256_nogate", 2, 64, 8, 2, 256, 32, "none", [3000, 1], seed=322),
    # more workgroups than compute units: the plan's second-round estimate
    _case("many_items_d128", 8, 512, 16, 8, 128, 32, "headwise", [4000, 0, 1000, 3000, 200, 2500, 50, 3500],
          [512, 512, 300, 512, 1, 512, 512, 77], seed=324),
    # more sequences than the plan takes (one per lane): the plain mirrored mapping
    _case("many_seqs_d128", 70, 40, 4, 2, 128, 32, "elementwise", [(37 * b) % 300 for b in range(70)],
          [40 - (b % 7) * 6 for b in range(70)], seed=325),
]


@pytest.mark.parametrize("w", SKEW_CASES, ids=lambda w: w.name)
def test_chunk_skewed_prefixes(w):
    print(f"[chunk] {w.name}", flush=True)
    _run(w)


def test_chunk_repeat_bits():
    """Repeated chunk attention calls over the same cache give the same bits."""
    w = SKEW_CASES[0]
    print(f"[chunk] {w.name}: repeats", flush=True)
    et = tdt(w)
    x = inputs.make_prefill(w)
    B, n, G, d = w.batch, w.seq_len, w.n_kv_heads, w.head_dim
    L = np.array(w.extra["lens"], np.int32)
    cl = np.array(w.extra["chunk_lens"], np.int32)
    max_len = int(L.max())
    cap = max_len + n + 2
    gen = torch.Generator(device="cuda").manual_seed(323)
    kc = torch.randn((B, cap, G, d), generator=gen, device="cuda").to(et)
    vc = torch.randn((B, cap, G, d), generator=gen, device="cuda").to(et)
    dsc = desc_for(w)
    args = (dsc, dev(x["q"], et), kc, vc, dev(L), max_len)
    kw = dict(gate=dev(x["gate"], et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]),
              chunk_lens=dev(cl))
    first = api.ga_prefill_chunk_attention(*args, **kw).clone()
    for _ in range(3):
        again = api.ga_prefill_chunk_attention(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(again, first)
