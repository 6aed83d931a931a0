"""ga_decode_noalloc (partials in the library's static device scratch, no
workspace) against ga_decode (caller workspace) through the C ABI: two calls
in a row, the second with a smaller batch and shorter caches (the scratch
keeps the first call's contents), then the full 64-sequence decode workload,
whose partials nearly fill the scratch. Same kernels, so the outputs and the
appended cache slots must be identical; the outputs are also checked against
the oracle at the bf16 bar."""
import numpy as np
import pytest
import torch

from gated_gqa_softmax_amd import _lib, api, inputs
from oracle import attention as oracle
from tests.gpu_helpers import assert_close, dev, desc_for, host, tdt

pytestmark = pytest.mark.gpu


def _case(name, lens, seed):
    return inputs.Workload(name, "decode", len(lens), 1, 8, 2, 256, 64, "bf16", "elementwise", seed=seed,
                           extra={"lens": list(lens)})


def _caches(w, lens):
    cap = int(max(lens)) + 1
    kc = torch.zeros((w.batch, cap, w.n_kv_heads, w.head_dim), dtype=tdt(w), device="cuda")
    vc = torch.zeros_like(kc)
    rows = {}

    def put(b, kh, vv):
        rows[b] = (kh, vv)
        if len(kh):
            kc[b, :len(kh)] = dev(kh, tdt(w))
            vc[b, :len(vv)] = dev(vv, tdt(w))

    inputs.for_each_cache_rows(w, np.asarray(lens, np.int32), put)
    return kc, vc, rows


def _both(w, lens, check_oracle=True):
    et = tdt(w)
    x = inputs.make_decode(w, cache_lens=np.asarray(lens, np.int32))
    kc, vc, rows = _caches(w, lens)
    kc2, vc2 = kc.clone(), vc.clone()
    d = desc_for(w)
    args = (dev(x["q"], et), dev(x["k_new"], et), dev(x["v_new"], et))
    L = dev(x["cache_lens"])
    max_len = int(max(lens))
    kw = dict(gate=dev(x["gate"], et), q_norm_w=dev(x["q_norm_w"]), k_norm_w=dev(x["k_norm_w"]))
    want = api.ga_decode(d, *args, kc, vc, L, max_len, **kw)
    out = torch.empty_like(want)
    got = api.ga_decode_noalloc(d, *args, kc2, vc2, L, max_len, out, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got, want), "no-alloc decode differs from ga_decode"
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc), "appended cache slots differ"
    if check_oracle:
        ref, _ = oracle.decode(x["q"], x["k_new"], x["v_new"], x["gate"], gate_mode=w.gate_mode,
                               q_norm_w=x["q_norm_w"], k_norm_w=x["k_norm_w"], k_cache_rows=lambda b: rows[b],
                               cache_lens=x["cache_lens"], rms_eps=w.rms_eps, rope_base=w.rope_base,
                               rot_dim=w.rot_dim)
        assert_close(host(got), ref, w, w.name)
    return got


def test_noalloc_decode_two_calls_second_smaller():
    print("[noalloc] 8 sequences, then 3 shorter ones", flush=True)
    first = _case("noalloc_big", [9000, 17, 4096, 513, 0, 2500, 8191, 1], seed=251)
    _both(first, first.extra["lens"])
    second = _case("noalloc_small", [700, 5, 64], seed=252)
    _both(second, second.extra["lens"])


def test_noalloc_decode_full_workload():
    w = inputs.WORKLOADS["decode_64seq"]
    x = inputs.make_decode(w)
    need = api.ga_decode_workspace_bytes(desc_for(w), int(x["cache_lens"].max()))
    print(f"[noalloc] decode_64seq: {need} bytes of partials in the static scratch", flush=True)
    assert need <= _lib.GA_NOALLOC_SCRATCH_BYTES
    _both(w, x["cache_lens"], check_oracle=False)


def test_noalloc_decode_rejects_oversized_steps():
    w = _case("noalloc_over", [10, 10], seed=253)
    x = inputs.make_decode(w, cache_lens=np.array([10, 10], np.int32))
    et = tdt(w)
    big = 1 << 22     # partials of 2 x 8 heads x 8192 splits x 258 floats > the scratch
    kc = torch.zeros((2, 16, 2, 256), dtype=et, device="cuda")
    out = torch.empty((2, 8 * 256), dtype=et, device="cuda")
    d = desc_for(w)
    assert api.ga_decode_workspace_bytes(d, big) > _lib.GA_NOALLOC_SCRATCH_BYTES
    lib = _lib.load()
    st = lib.ga_decode_noalloc(d, dev(x["q"], et).data_ptr(), None, None, None, None, None, kc.data_ptr(),
                               kc.data_ptr(), big + 1, dev(x["cache_lens"]).data_ptr(), big, out.data_ptr(), None)
    assert st == _lib.GA_ERR_WORKSPACE
    assert b"static scratch" in lib.ga_last_error()
