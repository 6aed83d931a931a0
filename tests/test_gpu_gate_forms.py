"""GPU parity of the gate variants and the per-head output norm (the
kernels' extended epilogue) with the fp64 oracle's ``GateForm``, through the
C ABI: every prefill kernel (mirrored, chunked, wide, simple, generic) and
decode (fused, generic), each activation, both combines, head-shared and
input-independent gates, and the output norm alone and with a gate.

Tolerance. The bf16 bars (max-abs 2e-2, mean-abs 2e-3) hold for the gated
attention output, whose gate lies in (0, 1). A variant scales an error of
the attention output y by S: max(1, |act(z)|) for a multiplicative gate (an
additive gate passes it through: 1), times |w_e| / rms(y_row) for the output
norm; and its output, larger than y, carries its own final bf16 rounding of
up to half an ulp (2^-9 relative). Each element must satisfy
|got - want| <= 2e-2 * S + 2^-8 * |want|, and the mean error
<= 2e-3 * mean(S) + 2^-9 * mean(|want|) (fp32: 1e-4 bars, 2^-20 rounding)."""
import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import api, inputs
from oracle import attention as oracle
from tests.gpu_helpers import dev, host, tdt, tol

pytestmark = pytest.mark.gpu


def _form(act="sigmoid", combine="mul", heads=False, tokens=False, norm=False):
    return dict(act=act, combine=combine, heads=heads, tokens=tokens, norm=norm)


def _label(f):
    parts = [f["act"], f["combine"]] + [k for k in ("heads", "tokens", "norm") if f[k]]
    return "-".join(parts)


def _gate_logits(w, lead, f, seed):
    """Seeded logits in the shape the form asks for (bf16-representable)."""
    if w.gate_mode == "none":
        return None
    rng = np.random.default_rng(seed)
    row = (w.head_dim,) if w.gate_mode == "elementwise" else ()
    heads = () if f["heads"] else (w.n_q_heads,)
    shape = (() if f["tokens"] else tuple(lead)) + heads + row
    if not shape:
        shape = (1,)
    z = rng.standard_normal(shape).astype(np.float32) * np.float32(1.5)
    return inputs.round_bf16(z) if w.dtype == "bf16" else z


def _norm_w(w, seed):
    rng = np.random.default_rng(seed)
    return (1.0 + 0.1 * rng.standard_normal(w.head_dim)).astype(np.float32)


def _descs(w, f, nw, kernel="auto"):
    wt = dev(nw) if f["norm"] else None
    d = api.make_desc(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.rot_dim, w.rope_base, w.rms_eps, 0.0,
                      tdt(w), w.gate_mode, gate_act=f["act"], gate_combine=f["combine"], share_heads=f["heads"],
                      share_tokens=f["tokens"], out_norm_w=wt, out_norm_eps=1e-6, kernel=kernel)
    of = oracle.GateForm(act=f["act"], combine=f["combine"], share_heads=f["heads"],
                         input_independent=f["tokens"], out_norm_w=nw if f["norm"] else None, out_norm_eps=1e-6)
    return d, of


def _oracle_z(z, f):
    # a gate shared by everything is passed to the oracle without its dummy dim
    if z is not None and f["heads"] and f["tokens"] and z.shape == (1,):
        return z.reshape(())
    return z


def _assert_variant(got, want, y_plain, w, f, z_full, nw, label):
    """got/want [.., H*d]; y_plain the oracle's ungated attention output (same
    shape); z_full the logits expanded to [.., H, d] | [.., H] (or None)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite GPU output"
    shp = want.shape[:-1] + (w.n_q_heads, w.head_dim)
    S = np.ones(shp)
    if z_full is not None and f["combine"] == "mul":
        g = np.abs(oracle.gate_activation(z_full, f["act"]))
        S = S * np.maximum(1.0, g[..., None] if w.gate_mode == "headwise" else g)
    if f["norm"]:
        yp = np.asarray(y_plain, dtype=np.float64).reshape(shp)
        S = S * np.abs(nw) / np.sqrt(np.mean(yp ** 2, axis=-1, keepdims=True) + 1e-6)
    S = S.reshape(want.shape)
    max_tol, mean_tol = tol(w)
    rnd = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -20
    err = np.abs(got - want)
    bound = max_tol * S + rnd * np.abs(want)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{label}: error {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst}"
    mean_bound = mean_tol * S.mean() + 0.5 * rnd * np.abs(want).mean()
    assert err.mean() <= mean_bound, f"{label}: mean error {err.mean():.3e} > {mean_bound:.3e}"
    return float(err.max()), float(err.mean()), float(S.max())


def _prefill_case(name, B, n, H, G, d, rot, gate, dtype="bf16", seed=500, kernel=None):
    return inputs.Workload(name, "prefill", B, n, H, G, d, rot, dtype, gate, seed=seed, extra={"kernel": kernel})


PREFILL = [
    (_prefill_case("mirror_d256_elem", 2, 150, 8, 2, 256, 64, "elementwise", seed=501, kernel="mirror"),
     [_form("silu"), _form("ns_sigmoid", "add", norm=True), _form("identity", "add"), _form(heads=True),
      _form("silu", tokens=True, norm=True), _form("ns_sigmoid", heads=True, tokens=True)]),
    (_prefill_case("mirror_d128_head", 1, 130, 16, 8, 128, 32, "headwise", seed=502, kernel="mirror"),
     [_form("silu", "add"), _form(heads=True, norm=True), _form("identity", tokens=True)]),
    (_prefill_case("mirror_d256_nogate", 1, 100, 8, 2, 256, 64, "none", seed=503, kernel="mirror"),
     [_form(norm=True)]),
    (_prefill_case("simple_d64_elem", 2, 90, 4, 2, 64, 16, "elementwise", seed=504, kernel="simple"),
     [_form("silu", norm=True), _form("ns_sigmoid", "add", tokens=True)]),
    (_prefill_case("simple_d128_head", 1, 70, 4, 4, 128, 32, "headwise", seed=505, kernel="simple"),
     [_form("identity", "add", heads=True, norm=True)]),
    (_prefill_case("generic_f32_elem", 2, 20, 4, 2, 16, 4, "elementwise", dtype="f32", seed=506, kernel="generic"),
     [_form("identity", "add", heads=True, norm=True), _form("silu", tokens=True)]),
    (_prefill_case("generic_bf16_d96_head", 1, 40, 6, 2, 96, 16, "headwise", seed=507, kernel="generic"),
     [_form("ns_sigmoid", "add", norm=True)]),
]

PREFILL_CASES = [(w, f) for w, forms in PREFILL for f in forms]


@pytest.mark.parametrize("w,f", PREFILL_CASES, ids=[f"{w.name}-{_label(f)}" for w, f in PREFILL_CASES])
def test_gate_forms_prefill(w, f):
    print(f"[gate forms] {w.name} {_label(f)}", flush=True)
    x = inputs.make_prefill(w)
    et = tdt(w)
    z = _gate_logits(w, (w.batch, w.seq_len), f, w.seed + 10)
    nw = _norm_w(w, w.seed + 11)
    d, of = _descs(w, f, nw, kernel="simple" if w.extra["kernel"] == "simple" else "auto")
    assert api.ga_prefill_attention_kernel(d, w.seq_len) == w.extra["kernel"]
    out = api.ga_prefill(d, dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), dev(z, et), dev(x["q_norm_w"]),
                         dev(x["k_norm_w"]), dev(x["positions"]))
    torch.cuda.synchronize()
    kw = dict(q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], positions=x["positions"], rms_eps=w.rms_eps,
              rope_base=w.rope_base, rot_dim=w.rot_dim)
    want = oracle.prefill(x["q"], x["k"], x["v"], _oracle_z(z, f), gate_mode=w.gate_mode, gate_form=of, **kw)
    plain = oracle.prefill(x["q"], x["k"], x["v"], None, gate_mode="none", **kw)
    zf = oracle.expand_gate(_oracle_z(z, f), w.gate_mode, of, (w.batch, w.seq_len), w.n_q_heads)
    mx, mean, smax = _assert_variant(host(out), want, plain, w, f, zf, nw, f"{w.name} {_label(f)}")
    print(f"  max-abs {mx:.2e} mean-abs {mean:.2e} (max S {smax:.1f})", flush=True)


def test_gate_forms_wide_kernel():
    w = _prefill_case("wide_d128_elem", 4, 2048, 16, 8, 128, 32, "elementwise", seed=508)
    f = _form("ns_sigmoid", "add", heads=True, norm=True)
    print(f"[gate forms] {w.name} {_label(f)}", flush=True)
    x = inputs.make_prefill(w)
    et = tdt(w)
    z = _gate_logits(w, (w.batch, w.seq_len), f, 518)
    nw = _norm_w(w, 519)
    d, of = _descs(w, f, nw)
    assert api.ga_prefill_attention_kernel(d, w.seq_len) == "wide"
    out = api.ga_prefill(d, dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), dev(z, et), dev(x["q_norm_w"]),
                         dev(x["k_norm_w"]), dev(x["positions"]))
    torch.cuda.synchronize()
    rows = [(0, 0, 0), (1, 777, 5), (2, 2047, 15), (3, 1024, 8), (3, 255, 1)]
    kw = dict(q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], positions=x["positions"], rms_eps=w.rms_eps,
              rope_base=w.rope_base, rot_dim=w.rot_dim)
    want = oracle.prefill_rows(x["q"], x["k"], x["v"], z, rows, gate_mode=w.gate_mode, gate_form=of, **kw)
    plain = oracle.prefill_rows(x["q"], x["k"], x["v"], None, rows, gate_mode="none", **kw)
    zf = oracle.expand_gate(z, w.gate_mode, of, (w.batch, w.seq_len), w.n_q_heads)
    got = host(out)
    dd = w.head_dim
    # one row per "token" with a single head: check row r as a [1, d] output
    w1 = w.with_(batch=1, seq_len=len(rows), n_q_heads=1, n_kv_heads=1)
    z1 = np.stack([zf[b, i, h] for b, i, h in rows])[:, None]
    _assert_variant(np.stack([got[b, i, h * dd:(h + 1) * dd] for b, i, h in rows]), want, plain, w1, f, z1, nw,
                    w.name)


def test_gate_forms_chunk():
    w = _prefill_case("chunk_d256_elem", 3, 64, 8, 2, 256, 64, "elementwise", seed=509)
    f = _form("silu", "add", heads=True, norm=True)
    print(f"[gate forms] {w.name} {_label(f)}", flush=True)
    et, dd, G = tdt(w), w.head_dim, w.n_kv_heads
    x = inputs.make_prefill(w)
    L = np.array([0, 40, 130], dtype=np.int32)
    cl = np.array([64, 30, 1], dtype=np.int32)
    max_len, cap = 130, 130 + w.seq_len
    gen = torch.Generator().manual_seed(520)
    kc = torch.zeros((w.batch, cap, G, dd), dtype=et, device="cuda")
    vc = torch.zeros_like(kc)
    prefix = {}
    for b in range(w.batch):
        kp = torch.randn((int(L[b]), G, dd), generator=gen).to(et)
        vp = torch.randn((int(L[b]), G, dd), generator=gen).to(et)
        kc[b, :L[b]], vc[b, :L[b]] = kp.cuda(), vp.cuda()
        prefix[b] = (kp.double().numpy(), vp.double().numpy())
    z = _gate_logits(w, (w.batch, w.seq_len), f, 521)
    nw = _norm_w(w, 522)
    d, of = _descs(w, f, nw)
    assert api.ga_prefill_chunk_kernel(d, w.seq_len, cap) == "mirror"
    out = api.ga_prefill_chunk(d, dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), kc, vc, dev(L), max_len,
                               gate=dev(z, et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]),
                               chunk_lens=dev(cl))
    torch.cuda.synchronize()
    kw = dict(q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], k_cache_rows=lambda b: prefix[b], cache_lens=L,
              chunk_lens=cl, max_cache_len=max_len, rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    want, _ = oracle.prefill_chunk(x["q"], x["k"], x["v"], z, gate_mode=w.gate_mode, gate_form=of, **kw)
    plain, _ = oracle.prefill_chunk(x["q"], x["k"], x["v"], None, gate_mode="none", **kw)
    zf = oracle.expand_gate(z, w.gate_mode, of, (w.batch, w.seq_len), w.n_q_heads)
    got = host(out)
    for b in range(w.batch):
        _assert_variant(got[b, :cl[b]], want[b, :cl[b]], plain[b, :cl[b]], w, f, zf[b, :cl[b]], nw,
                        f"{w.name} seq {b}")


def _decode_case(name, lens, H, G, d, rot, gate, seed):
    return inputs.Workload(name, "decode", len(lens), 1, H, G, d, rot, "bf16", gate, seed=seed,
                           extra={"lens": list(lens)})


DECODE = [
    (_decode_case("fused_d256_elem", [0, 1, 700, 1536], 8, 2, 256, 64, "elementwise", 531),
     _form("silu", "add", norm=True)),
    (_decode_case("fused_d128_head", [5, 511, 513], 16, 8, 128, 32, "headwise", 532), _form(heads=True)),
    (_decode_case("fused_d64_elem", [100, 3], 16, 2, 64, 16, "elementwise", 533),
     _form("ns_sigmoid", tokens=True, norm=True)),
    (_decode_case("generic_g3_elem", [0, 40, 300], 6, 2, 128, 32, "elementwise", 534),
     _form("identity", "add", heads=True, tokens=True, norm=True)),
]


@pytest.mark.parametrize("w,f", DECODE, ids=[f"{w.name}-{_label(f)}" for w, f in DECODE])
def test_gate_forms_decode(w, f):
    print(f"[gate forms] decode {w.name} {_label(f)}", flush=True)
    et, dd = tdt(w), w.head_dim
    x = inputs.make_decode(w, cache_lens=np.array(w.extra["lens"], dtype=np.int32))
    L = x["cache_lens"]
    max_len = int(L.max())
    cap = max_len + 2
    kc = torch.zeros((w.batch, cap, w.n_kv_heads, dd), dtype=et, device="cuda")
    vc = torch.zeros_like(kc)
    rows = {}

    def put(b, kh, vv):
        rows[b] = (kh, vv)
        if len(kh):
            kc[b, :len(kh)] = dev(kh, et)
            vc[b, :len(vv)] = dev(vv, et)

    inputs.for_each_cache_rows(w, L, put)
    z = _gate_logits(w, (w.batch,), f, w.seed + 10)
    nw = _norm_w(w, w.seed + 11)
    d, of = _descs(w, f, nw)
    out = api.ga_decode(d, dev(x["q"], et), dev(x["k_new"], et), dev(x["v_new"], et), kc, vc, dev(L), max_len,
                        gate=dev(z, et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]))
    torch.cuda.synchronize()
    kw = dict(q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], k_cache_rows=lambda b: rows[b], cache_lens=L,
              rms_eps=w.rms_eps, rope_base=w.rope_base, rot_dim=w.rot_dim)
    want, _ = oracle.decode(x["q"], x["k_new"], x["v_new"], _oracle_z(z, f), gate_mode=w.gate_mode, gate_form=of,
                            **kw)
    plain, _ = oracle.decode(x["q"], x["k_new"], x["v_new"], None, gate_mode="none", **kw)
    zf = oracle.expand_gate(_oracle_z(z, f), w.gate_mode, of, (w.batch,), w.n_q_heads)
    mx, mean, smax = _assert_variant(host(out), want, plain, w, f, zf, nw, f"{w.name} {_label(f)}")
    print(f"  max-abs {mx:.2e} mean-abs {mean:.2e} (max S {smax:.1f})", flush=True)


def test_gate_forms_full_workload_sampled():
    """The 4096-token workload with the extended epilogue the bench times
    (elementwise SiLU gate after the per-head output RMSNorm): sampled rows."""
    w = inputs.WORKLOADS["qwen35_0p8b_prefill"]
    f = _form("silu", "mul", norm=True)
    print(f"[gate forms] {w.name} {_label(f)} full size", flush=True)
    x = inputs.make_prefill(w)
    et = tdt(w)
    nw = _norm_w(w, 541)
    d, of = _descs(w, f, nw)
    assert api.ga_prefill_attention_kernel(d, w.seq_len) == "mirror"
    out = api.ga_prefill(d, dev(x["q"], et), dev(x["k"], et), dev(x["v"], et), dev(x["gate"], et),
                         dev(x["q_norm_w"]), dev(x["k_norm_w"]), dev(x["positions"]))
    torch.cuda.synchronize()
    rows = [(0, 0, 0), (0, 1, 7), (0, 1000, 3), (0, 2049, 4), (0, 4095, 5), (0, 4095, 0)]
    kw = dict(q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], positions=x["positions"], rms_eps=w.rms_eps,
              rope_base=w.rope_base, rot_dim=w.rot_dim)
    want = oracle.prefill_rows(x["q"], x["k"], x["v"], x["gate"], rows, gate_mode=w.gate_mode, gate_form=of, **kw)
    plain = oracle.prefill_rows(x["q"], x["k"], x["v"], None, rows, gate_mode="none", **kw)
    got = host(out)
    dd = w.head_dim
    w1 = w.with_(batch=1, seq_len=len(rows), n_q_heads=1, n_kv_heads=1)
    z1 = np.stack([x["gate"][b, i, h] for b, i, h in rows])[:, None]
    _assert_variant(np.stack([got[b, i, h * dd:(h + 1) * dd] for b, i, h in rows]), want, plain, w1, f, z1, nw,
                    w.name)
