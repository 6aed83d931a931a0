"""GPU parity of the fused q-projection layout (per-head [q | gate] rows, q and
the gate read in place through head strides) through the C ABI: every
prefill kernel (mirrored, wide, simple, generic), the chunked
prefill, decode (fused and generic, whole and in stages) and the full
4096-token workload. Packed calls must give the same bits as the dense
layout on the same kernel, and match the fp64 oracle, which reads the packed
rows through its own split of the projection output."""
import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import attention as oracle
from tests.gpu_helpers import assert_close, dev, desc_for, host, tdt

pytestmark = pytest.mark.gpu


def _pack(q, gate, mode, width):
    """Host arrays [.., H, d] (+ gate) -> per-head rows of ``width`` values:
    the query, then the gate logits (elementwise: d, headwise: 1), then zeros."""
    d = q.shape[-1]
    qg = np.zeros(q.shape[:-1] + (width,), dtype=q.dtype)
    qg[..., :d] = q
    if mode == "elementwise":
        qg[..., d:2 * d] = gate
    else:
        qg[..., d] = gate
    return qg


def _views(qg_t, d, mode):
    return qg_t[..., :d], (qg_t[..., d:2 * d] if mode == "elementwise" else qg_t[..., d])


def _oracle_split(qg, d, mode):
    width = 2 * d if mode == "elementwise" else d + 1
    return oracle.split_q_proj(qg[..., :width], d, mode)


def _width(w, pad):
    d = w.head_dim
    return (2 * d if w.gate_mode == "elementwise" else d + 1) + pad


def _prefill_pair(w, x, qg_np, kernel="auto"):
    """(packed output, dense output) of ga_prefill on the same inputs."""
    et = tdt(w)
    d = w.head_dim
    k, v = dev(x["k"], et), dev(x["v"], et)
    wq, wk = dev(x["q_norm_w"]), dev(x["k_norm_w"])
    pos = dev(x["positions"]) if x.get("positions") is not None else None
    qg = dev(qg_np, et)
    qv, gv = _views(qg, d, w.gate_mode)
    assert not qv.is_contiguous()
    packed = api.ga_prefill(desc_for(w, kernel=kernel), qv, k, v, gv, wq, wk, pos)
    dense = api.ga_prefill(desc_for(w, kernel=kernel), dev(x["q"], et), k, v, dev(x["gate"], et), wq, wk, pos)
    torch.cuda.synchronize()
    return packed, dense


def _prefill_case(name, B, n, H, G, d, rot, gate, pad=0, dtype="bf16", seed=400, kernel=None):
    return inputs.Workload(name, "prefill", B, n, H, G, d, rot, dtype, gate, seed=seed,
                           extra={"pad": pad, "kernel": kernel})


PREFILL = [
    _prefill_case("mirror_d256_elem", 2, 200, 8, 2, 256, 64, "elementwise", seed=401, kernel="mirror"),
    _prefill_case("mirror_d128_head_pad7", 1, 150, 16, 8, 128, 32, "headwise", pad=7, seed=402, kernel="mirror"),
    _prefill_case("simple_d64_elem", 2, 100, 4, 2, 64, 16, "elementwise", seed=403, kernel="simple"),
    _prefill_case("generic_d128_head_qz", 2, 60, 4, 2, 128, 32, "headwise", seed=404, kernel="generic"),
    _prefill_case("generic_f32_elem", 2, 20, 4, 2, 16, 4, "elementwise", dtype="f32", seed=405, kernel="generic"),
]


@pytest.mark.parametrize("w", PREFILL, ids=lambda w: w.name)
def test_packed_prefill_small(w):
    print(f"[packed] {w.name}", flush=True)
    d, width = w.head_dim, _width(w, w.extra["pad"])
    assert api.ga_prefill_attention_kernel(
        api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, d, w.rot_dim, dtype=tdt(w), gate_mode=w.gate_mode,
                      q_head_stride=width, gate_head_stride=width), w.seq_len) == w.extra["kernel"]
    # the dense layout of a generic-kernel shape may have a fused kernel: compare on the same one
    kernel = "generic" if w.extra["kernel"] == "generic" else "auto"
    x = inputs.make_prefill(w)
    qg = _pack(x["q"], x["gate"], w.gate_mode, width)
    packed, dense = _prefill_pair(w, x, qg, kernel=kernel)
    assert torch.equal(packed, dense), f"{w.name}: packed and dense layouts differ"
    q, gate = _oracle_split(qg, d, w.gate_mode)
    want = oracle.prefill(q, x["k"], x["v"], gate, gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"],
                          k_norm_w=x["k_norm_w"], positions=x["positions"], rms_eps=w.rms_eps,
                          rope_base=w.rope_base, rot_dim=w.rot_dim)
    assert_close(host(packed), want, w, w.name)


def _sampled_rows(w, x, qg, packed, rows):
    q, gate = _oracle_split(qg, w.head_dim, w.gate_mode)
    want = oracle.prefill_rows(q, x["k"], x["v"], gate, rows, gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"],
                               k_norm_w=x["k_norm_w"], positions=x["positions"], rms_eps=w.rms_eps,
                               rope_base=w.rope_base, rot_dim=w.rot_dim)
    got = host(packed)
    d = w.head_dim
    got_rows = np.stack([got[b, i, h * d:(h + 1) * d] for b, i, h in rows])
    assert_close(got_rows, want, w, f"{w.name} sampled rows")


def test_packed_prefill_wide_kernel():
    w = _prefill_case("wide_d128_elem", 4, 2048, 16, 8, 128, 32, "elementwise", seed=407)
    print(f"[packed] {w.name}", flush=True)
    d = w.head_dim
    assert api.ga_prefill_attention_kernel(
        api.make_desc(4, 16, 8, 128, 32, gate_mode="elementwise", q_head_stride=2 * d, gate_head_stride=2 * d),
        w.seq_len) == "wide"
    x = inputs.make_prefill(w)
    qg = _pack(x["q"], x["gate"], w.gate_mode, 2 * d)
    packed, dense = _prefill_pair(w, x, qg)
    assert torch.equal(packed, dense)
    _sampled_rows(w, x, qg, packed, [(0, 0, 0), (1, 777, 5), (2, 2047, 15), (3, 1024, 8), (3, 255, 1)])


def test_packed_prefill_full_workload():
    w = inputs.WORKLOADS["qwen35_0p8b_prefill"]
    print(f"[packed] {w.name} full size", flush=True)
    x = inputs.make_prefill(w)
    qg = _pack(x["q"], x["gate"], w.gate_mode, 2 * w.head_dim)
    packed, dense = _prefill_pair(w, x, qg)
    assert torch.equal(packed, dense)
    _sampled_rows(w, x, qg, packed, [(0, 0, 0), (0, 1, 7), (0, 2049, 3), (0, 4095, 4), (0, 4095, 0)])


# -- chunked prefill ------------------------------------------------------------

def test_packed_chunk():
    w = inputs.Workload("chunk_mirror_d256_elem", "prefill", 3, 100, 8, 2, 256, 64, "bf16", "elementwise",
                        seed=408)
    print(f"[packed] {w.name}", flush=True)
    et, d, G = tdt(w), w.head_dim, w.n_kv_heads
    x = inputs.make_prefill(w)
    L = np.array([0, 37, 130], dtype=np.int32)
    cl = np.array([100, 64, 1], dtype=np.int32)
    max_len, cap = 130, 130 + w.seq_len + 2
    gen = torch.Generator().manual_seed(409)
    kc = torch.zeros((w.batch, cap, G, d), dtype=et, device="cuda")
    vc = torch.zeros_like(kc)
    prefix = {}
    for b in range(w.batch):
        kp = torch.randn((int(L[b]), G, d), generator=gen).to(et)
        vp = torch.randn((int(L[b]), G, d), generator=gen).to(et)
        kc[b, :L[b]], vc[b, :L[b]] = kp.cuda(), vp.cuda()
        prefix[b] = (kp.double().numpy(), vp.double().numpy())
    qg = _pack(x["q"], x["gate"], w.gate_mode, 2 * d)
    qv, gv = _views(dev(qg, et), d, w.gate_mode)
    outs = []
    for q_, g_ in ((qv, gv), (dev(x["q"], et), dev(x["gate"], et))):
        kc2, vc2 = kc.clone(), vc.clone()
        outs.append(api.ga_prefill_chunk(desc_for(w), q_, dev(x["k"], et), dev(x["v"], et), kc2, vc2, dev(L),
                                         max_len, gate=g_, q_norm_w=dev(x["q_norm_w"]),
                                         k_norm_w=dev(x["k_norm_w"]), chunk_lens=dev(cl)))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    q, gate = _oracle_split(qg, d, w.gate_mode)
    want, _ = oracle.prefill_chunk(q, x["k"], x["v"], gate, gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"],
                                   k_norm_w=x["k_norm_w"], k_cache_rows=lambda b: prefix[b], cache_lens=L,
                                   chunk_lens=cl, max_cache_len=max_len, rms_eps=w.rms_eps,
                                   rope_base=w.rope_base, rot_dim=w.rot_dim)
    got = host(outs[0])
    for b in range(w.batch):
        assert_close(got[b, :cl[b]], want[b, :cl[b]], w, f"{w.name} seq {b}")


# -- decode -----------------------------------------------------------------------

def _decode_case(name, lens, H, G, d, rot, gate, pad=0, seed=410, fused=True):
    return inputs.Workload(name, "decode", len(lens), 1, H, G, d, rot, "bf16", gate, seed=seed,
                           extra={"lens": list(lens), "pad": pad, "fused": fused})


DECODE = [
    _decode_case("fused_d256_elem", [0, 1, 700, 1536], 8, 2, 256, 64, "elementwise", seed=411),
    _decode_case("fused_d128_head_pad7", [5, 511, 513], 16, 8, 128, 32, "headwise", pad=7, seed=412),
    _decode_case("generic_d128_head_qz", [0, 40, 300], 8, 2, 128, 32, "headwise", seed=413, fused=False),
]


@pytest.mark.parametrize("w", DECODE, ids=lambda w: w.name)
def test_packed_decode(w):
    print(f"[packed] decode {w.name}", flush=True)
    et, d = tdt(w), w.head_dim
    width = _width(w, w.extra["pad"])
    x = inputs.make_decode(w, cache_lens=np.array(w.extra["lens"], dtype=np.int32))
    L = x["cache_lens"]
    max_len = int(L.max())
    cap = max_len + 2
    kc = torch.zeros((w.batch, cap, w.n_kv_heads, d), dtype=et, device="cuda")
    vc = torch.zeros_like(kc)
    rows = {}

    def put(b, kh, vv):
        rows[b] = (kh, vv)
        if len(kh):
            kc[b, :len(kh)] = dev(kh, et)
            vc[b, :len(vv)] = dev(vv, et)

    inputs.for_each_cache_rows(w, L, put)
    qg = _pack(x["q"], x["gate"], w.gate_mode, width)
    qv, gv = _views(dev(qg, et), d, w.gate_mode)
    args = (dev(x["k_new"], et), dev(x["v_new"], et))
    wq, wk, lens = dev(x["q_norm_w"]), dev(x["k_norm_w"]), dev(L)
    d_ = desc_for(w)
    kc1, vc1 = kc.clone(), vc.clone()
    packed = api.ga_decode(d_, qv, *args, kc1, vc1, lens, max_len, gate=gv, q_norm_w=wq, k_norm_w=wk)
    torch.cuda.synchronize()
    q, gate = _oracle_split(qg, d, w.gate_mode)
    want, _ = oracle.decode(q, x["k_new"], x["v_new"], gate, gate_mode=w.gate_mode, q_norm_w=x["q_norm_w"],
                            k_norm_w=x["k_norm_w"], k_cache_rows=lambda b: rows[b], cache_lens=L,
                            rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    assert_close(host(packed), want, w, w.name)
    if not w.extra["fused"]:
        return
    # same bits as the dense layout, whole and in stages
    kc2, vc2 = kc.clone(), vc.clone()
    dense = api.ga_decode(d_, dev(x["q"], et), *args, kc2, vc2, lens, max_len, gate=dev(x["gate"], et),
                          q_norm_w=wq, k_norm_w=wk)
    kc3, vc3 = kc.clone(), vc.clone()
    ws = torch.empty(api.ga_decode_workspace_bytes(d_, max_len), dtype=torch.uint8, device="cuda")
    api.ga_decode_partials(d_, qv, kc3, vc3, lens, max_len, ws, q_norm_w=wq)
    staged = api.ga_decode_merge(d_, qv, *args, kc3, vc3, lens, max_len, ws, gate=gv, q_norm_w=wq, k_norm_w=wk)
    torch.cuda.synchronize()
    assert torch.equal(packed, dense) and torch.equal(staged, dense)
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2) and torch.equal(kc3, kc2)
