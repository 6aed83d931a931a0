"""Host-side checks of the Python binding: every tensor's shape is compared
with the descriptor before a pointer reaches the library, so a mismatched
descriptor can never make a kernel read or write out of bounds.

These tests run on the CPU: the binding's device check is relaxed to accept
CPU tensors, and the library is replaced by a stub that fails the test if any
call reaches it (each case must raise ValueError first)."""
import pytest
import torch

from gated_gqa_softmax_amd import _lib, api


class _NoLibrary:
    def __getattr__(self, name):
        def reached(*args, **kwargs):
            raise AssertionError(f"{name} reached the library with inconsistent arguments")
        return reached


@pytest.fixture(autouse=True)
def host_only(monkeypatch):
    real_ptr = api._ptr

    def ptr(t, name, dtype=None):
        if t is None:
            return None
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        return 1 << 20

    def head_rows(t, name, dtype, lead, n_heads, width):
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}")
        return api.head_stride(t.shape, t.stride(), lead, n_heads, width, name)

    monkeypatch.setattr(api, "_ptr", ptr)
    monkeypatch.setattr(api, "_head_rows", head_rows)
    monkeypatch.setattr(_lib, "load", lambda *a, **k: _NoLibrary())
    monkeypatch.setattr(api, "ga_prefill_workspace_bytes", lambda d, n: 1024)
    monkeypatch.setattr(api, "ga_prefill_chunk_workspace_bytes", lambda d, n, c, m: 0)
    monkeypatch.setattr(api, "ga_decode_workspace_bytes", lambda d, m: 1024)
    monkeypatch.setattr(api, "ga_prefill_backward_workspace_bytes", lambda d, n: 1024)
    yield real_ptr


B, N, H, G, D = 2, 16, 8, 2, 128
bf = torch.bfloat16


def _desc(gate="elementwise", batch=B):
    return api.make_desc(batch, H, G, D, 32, 10000.0, 1e-6, 0.0, bf, gate)


def _t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def _prefill_args(**over):
    a = dict(q=_t(B, N, H, D), k=_t(B, N, G, D), v=_t(B, N, G, D), gate=_t(B, N, H, D),
             q_norm_w=_t(D, dtype=torch.float32), k_norm_w=_t(D, dtype=torch.float32),
             positions=_t(B, N, dtype=torch.int32), out=_t(B, N, H * D), workspace=_t(1024, dtype=torch.uint8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(q=_t(B + 1, N, H, D)), "q has shape"),                      # batch differs from the descriptor
    (dict(k=_t(B, N, G + 1, D)), "k has shape"),
    (dict(k=_t(B, N - 1, G, D)), "k has shape"),
    (dict(v=_t(B, N, G, D - 8)), "v has shape"),
    (dict(gate=_t(B, N + 1, H, D)), "gate has shape"),
    (dict(gate=_t(1, N, H, D)), "gate has shape"),
    (dict(gate=None), "gate is required"),
    (dict(q_norm_w=_t(D - 4, dtype=torch.float32)), "q_norm_w has shape"),
    (dict(k_norm_w=_t(2 * D, dtype=torch.float32)), "k_norm_w has shape"),
    (dict(positions=_t(B, N - 1, dtype=torch.int32)), "positions has shape"),
    (dict(positions=_t(B * N, dtype=torch.int32)), "positions has shape"),
    (dict(out=_t(B, N, H * D - 8)), "out has shape"),
    (dict(out=_t(B + 1, N, H * D)), "out has shape"),
    (dict(workspace=_t(16, dtype=torch.uint8)), "workspace holds"),
])
def test_prefill_shapes(over, msg):
    with pytest.raises(ValueError, match=msg):
        api.ga_prefill(_desc(), **_prefill_args(**over))


def test_prefill_cache_shapes():
    a = _prefill_args()
    with pytest.raises(ValueError, match="v_cache has shape"):
        api.ga_prefill(_desc(), **a, k_cache=_t(B, 32, G, D), v_cache=_t(B, 16, G, D))
    with pytest.raises(ValueError, match="k_cache has shape"):
        api.ga_prefill(_desc(), **a, k_cache=_t(B, 32, G + 1, D), v_cache=_t(B, 32, G + 1, D))
    with pytest.raises(ValueError, match="capacity"):
        api.ga_prefill(_desc(), **a, k_cache=_t(B, N - 1, G, D), v_cache=_t(B, N - 1, G, D))
    with pytest.raises(ValueError, match="both required"):
        api.ga_prefill(_desc(), **a, k_cache=_t(B, 32, G, D))


def test_headwise_gate_shape():
    a = _prefill_args(gate=_t(B, N, H, D))
    with pytest.raises(ValueError, match="gate has shape"):
        api.ga_prefill(_desc("headwise"), **a)


def test_prefill_stages_shapes():
    a = _prefill_args()
    with pytest.raises(ValueError, match="k_hat holds"):
        api.ga_prefill_keys(_desc(), a["k"], k_hat=_t(B, N - 1, G, D))
    with pytest.raises(ValueError, match="v_out has shape"):
        api.ga_prefill_keys(_desc(), a["k"], a["v"], k_hat=_t(B, N, G, D), v_out=_t(B, N + 1, G, D))
    with pytest.raises(ValueError, match="v has shape"):
        api.ga_prefill_attention(_desc(), a["q"], _t(B, N, G, D), _t(B, N, G + 1, D), a["gate"])
    with pytest.raises(ValueError, match="rows per sequence"):
        api.ga_prefill_attention(_desc(), a["q"], _t(B, N, G, D), _t(B, N - 1, G, D), a["gate"])


def _decode_args(**over):
    cap = 65
    a = dict(q=_t(B, H, D), k_new=_t(B, G, D), v_new=_t(B, G, D), k_cache=_t(B, cap, G, D),
             v_cache=_t(B, cap, G, D), cache_lens=_t(B, dtype=torch.int32), max_cache_len=64, gate=_t(B, H, D),
             q_norm_w=_t(D, dtype=torch.float32), k_norm_w=_t(D, dtype=torch.float32), out=_t(B, H * D),
             workspace=_t(1024, dtype=torch.uint8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(q=_t(B + 1, H, D)), "q has shape"),
    (dict(k_new=_t(B, G, D + 8)), "k_new has shape"),
    (dict(v_new=_t(B - 1, G, D)), "v_new has shape"),
    (dict(v_cache=_t(B, 64, G, D)), "v_cache has shape"),
    (dict(k_cache=_t(B + 1, 65, G, D), v_cache=_t(B + 1, 65, G, D)), "k_cache has shape"),
    (dict(max_cache_len=65), "capacity"),                             # no slot for the appended token
    (dict(cache_lens=_t(B - 1, dtype=torch.int32)), "cache_lens"),
    (dict(cache_lens=_t(B, 1, dtype=torch.int32)), "cache_lens"),
    (dict(gate=_t(B + 1, H, D)), "gate has shape"),
    (dict(q_norm_w=_t(D + 1, dtype=torch.float32)), "q_norm_w has shape"),
    (dict(out=_t(B, H * D + 8)), "out has shape"),
])
def test_decode_shapes(over, msg):
    a = _decode_args(**over)
    with pytest.raises(ValueError, match=msg):
        api.ga_decode(_desc(), **a)
    if "gate" not in over and "out" not in over and "k_new" not in over and "v_new" not in over \
            and "k_norm_w" not in over:
        with pytest.raises(ValueError, match=msg):
            api.ga_decode_partials(_desc(), a["q"], a["k_cache"], a["v_cache"], a["cache_lens"],
                                   a["max_cache_len"], a["workspace"], q_norm_w=a["q_norm_w"])


def test_chunk_shapes():
    lens = _t(B, dtype=torch.int32)
    a = _prefill_args()
    cache = lambda cap, g=G: _t(B, cap, g, D)
    with pytest.raises(ValueError, match="capacity"):               # cap < max_cache_len + seq_len
        api.ga_prefill_chunk(_desc(), a["q"], a["k"], a["v"], cache(40), cache(40), lens, 30, gate=a["gate"])
    with pytest.raises(ValueError, match="v_cache has shape"):
        api.ga_prefill_chunk(_desc(), a["q"], a["k"], a["v"], cache(64), cache(64, G + 1), lens, 30,
                             gate=a["gate"])
    with pytest.raises(ValueError, match="chunk_lens"):
        api.ga_prefill_chunk(_desc(), a["q"], a["k"], a["v"], cache(64), cache(64), lens, 30, gate=a["gate"],
                             chunk_lens=_t(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="k has shape"):
        api.ga_prefill_chunk(_desc(), a["q"], _t(B, N + 1, G, D), a["v"], cache(64), cache(64), lens, 30,
                             gate=a["gate"])
    with pytest.raises(ValueError, match="q has shape"):
        api.ga_prefill_chunk_attention(_desc(), _t(B + 1, N, H, D), cache(64), cache(64), lens, 30,
                                       gate=a["gate"])
    with pytest.raises(ValueError, match="cache_lens"):
        api.ga_prefill_chunk_keys(_desc(), a["k"], a["v"], cache(64), cache(64), _t(1, dtype=torch.int32), 30)


def test_backward_shapes():
    a = _prefill_args()
    dout = _t(B, N, H * D)
    with pytest.raises(ValueError, match="dout has shape"):
        api.ga_prefill_backward(_desc(), a["q"], a["k"], a["v"], _t(B, N, H * D - 8), gate=a["gate"])
    with pytest.raises(ValueError, match="v has shape"):
        api.ga_prefill_backward(_desc(), a["q"], a["k"], _t(B, N, G, D + 8), dout, gate=a["gate"])
    with pytest.raises(ValueError, match="gate has shape"):
        api.ga_prefill_backward(_desc("headwise"), a["q"], a["k"], a["v"], dout, gate=a["gate"])
    with pytest.raises(ValueError, match="dq has shape"):
        api.ga_prefill_backward(_desc(), a["q"], a["k"], a["v"], dout, gate=a["gate"],
                                grads=dict(dq=_t(B, N, H, D - 8)))
