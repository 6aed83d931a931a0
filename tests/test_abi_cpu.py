"""Host-side checks of the C ABI: the library loads, exports every entry point
include/ga.h declares, and rejects bad arguments before any GPU work (these
calls never reach a kernel launch, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

from gated_gqa_softmax_amd import _lib
from gated_gqa_softmax_amd._lib import AttnDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_build():
    if not os.path.exists(_lib.LIB_PATH):
        from gated_gqa_softmax_amd.build import build_library
        build_library()
    return _lib.load()


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(ga_[a-z_0-9]+)\s*\(", src))
    return names


def test_library_exports_every_declared_entry_point():
    lib = _lib_or_build()
    declared = _declared()
    assert declared == set(_lib.SIGNATURES), declared ^ set(_lib.SIGNATURES)
    for name in declared:
        assert getattr(lib, name) is not None
    assert lib.ga_version() == 6
    assert ctypes.sizeof(AttnDesc) == 80


def _desc(**kw):
    base = dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=256, rot_dim=64, rope_base=10000.0,
                rms_eps=1e-6, softmax_scale=0.0, dtype=_lib.GA_BF16, gate_mode=_lib.GA_GATE_ELEMENTWISE)
    base.update(kw)
    return AttnDesc(**base)


def test_host_queries():
    lib = _lib_or_build()
    d = _desc()
    # kernel choice: d = 256 -> mirrored; d = 128 with >= 512 token blocks -> wide
    assert lib.ga_prefill_attention_kernel(ctypes.byref(d), 4096) == b"mirror"
    d3 = _desc(batch=4, n_q_heads=16, n_kv_heads=8, head_dim=128, rot_dim=32)
    assert lib.ga_prefill_attention_kernel(ctypes.byref(d3), 2048) == b"wide"
    assert lib.ga_prefill_attention_kernel(ctypes.byref(d3), 100) == b"mirror"
    assert lib.ga_prefill_attention_kernel(ctypes.byref(_desc(dtype=_lib.GA_F32)), 64) == b"generic"
    assert lib.ga_prefill_attention_kernel(ctypes.byref(_desc(head_dim=64, rot_dim=16)), 64) == b"simple"
    assert lib.ga_prefill_attention_kernel(None, 64) == b"invalid"
    # the prefill workspace holds K-hat only
    assert lib.ga_prefill_workspace_bytes(ctypes.byref(d), 4096) == 4096 * 2 * 256 * 2
    ck = lib.ga_decode_split_keys()
    assert ck > 0
    d5 = _desc(batch=64)
    ns = -(-32768 // ck)
    want = 64 * 8 * ns * (256 + 2) * 4
    assert lib.ga_decode_workspace_bytes(ctypes.byref(d5), 32768) == (want + 255) // 256 * 256
    assert lib.ga_fast_path(_lib.GA_BF16, 256, 64, 4) == 3
    assert lib.ga_fast_path(_lib.GA_BF16, 128, 32, 8) == 3
    assert lib.ga_fast_path(_lib.GA_BF16, 128, 32, 3) == 1       # decode: generic kernel
    assert lib.ga_fast_path(_lib.GA_F32, 8, 2, 2) == 0
    assert lib.ga_fast_path(_lib.GA_BF16, 96, 16, 2) == 0
    assert lib.ga_status_string(_lib.GA_ERR_WORKSPACE) == b"GA_ERR_WORKSPACE"


A16 = 1 << 20          # fake, 16-byte aligned "device" addresses: never dereferenced
MIS = A16 + 2


def _prefill(lib, d, n=16, q=A16, k=A16, v=A16, gate=A16, out=A16, ws=A16, ws_bytes=1 << 30,
             k_cache=None, v_cache=None, cap=0):
    return lib.ga_prefill(ctypes.byref(d) if d is not None else None, n, q, k, v, gate, None, None, None,
                          k_cache, v_cache, cap, ws, ws_bytes, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=8, n_kv_heads=3), _lib.GA_ERR_BAD_SHAPE),
    (dict(head_dim=300), _lib.GA_ERR_UNSUPPORTED),
    (dict(head_dim=0), _lib.GA_ERR_BAD_SHAPE),
    (dict(rot_dim=3), _lib.GA_ERR_BAD_SHAPE),
    (dict(rot_dim=258), _lib.GA_ERR_BAD_SHAPE),
    (dict(rope_base=0.0), _lib.GA_ERR_BAD_SHAPE),
    (dict(rms_eps=-1.0), _lib.GA_ERR_BAD_SHAPE),
    (dict(softmax_scale=float("nan")), _lib.GA_ERR_BAD_SHAPE),
    (dict(dtype=7), _lib.GA_ERR_BAD_DTYPE),
    (dict(gate_mode=5), _lib.GA_ERR_BAD_DTYPE),
    (dict(batch=-1), _lib.GA_ERR_BAD_SHAPE),
    (dict(q_head_stride=-8), _lib.GA_ERR_BAD_SHAPE),
    (dict(q_head_stride=255), _lib.GA_ERR_BAD_SHAPE),           # narrower than a head
    (dict(gate_head_stride=128), _lib.GA_ERR_BAD_SHAPE),        # elementwise gate: >= d
    (dict(gate_mode=_lib.GA_GATE_HEADWISE, gate_head_stride=-1), _lib.GA_ERR_BAD_SHAPE),
    (dict(gate_act=4), _lib.GA_ERR_BAD_DTYPE),
    (dict(gate_act=-1), _lib.GA_ERR_BAD_DTYPE),
    (dict(gate_combine=2), _lib.GA_ERR_BAD_DTYPE),
    (dict(gate_share=4), _lib.GA_ERR_BAD_DTYPE),
    (dict(out_norm_w=A16 + 4), _lib.GA_ERR_MISALIGNED),
    (dict(out_norm_w=A16, out_norm_eps=-1.0), _lib.GA_ERR_BAD_SHAPE),
    (dict(out_norm_w=A16, out_norm_eps=float("inf")), _lib.GA_ERR_BAD_SHAPE),
    (dict(kernel=5), _lib.GA_ERR_BAD_DTYPE),
    (dict(kernel=-1), _lib.GA_ERR_BAD_DTYPE),
    (dict(bwd_kernel=2), _lib.GA_ERR_BAD_DTYPE),
])
def test_prefill_rejects_bad_descriptors(kw, status):
    lib = _lib_or_build()
    assert _prefill(lib, _desc(**kw)) == status
    assert lib.ga_last_error() != b""


def test_prefill_rejects_bad_pointers_and_workspace():
    lib = _lib_or_build()
    d = _desc()
    assert _prefill(lib, None) == _lib.GA_ERR_NULL_ARG
    assert _prefill(lib, d, q=None) == _lib.GA_ERR_NULL_ARG
    assert _prefill(lib, d, gate=None) == _lib.GA_ERR_NULL_ARG
    assert _prefill(lib, d, out=MIS) == _lib.GA_ERR_MISALIGNED
    assert _prefill(lib, d, k=MIS) == _lib.GA_ERR_MISALIGNED
    assert _prefill(lib, d, ws=None) == _lib.GA_ERR_WORKSPACE
    assert _prefill(lib, d, ws_bytes=10) == _lib.GA_ERR_WORKSPACE
    assert _prefill(lib, d, k_cache=A16, v_cache=A16, cap=8) == _lib.GA_ERR_BAD_SHAPE   # cap < n
    assert _prefill(lib, d, k_cache=A16, v_cache=None, cap=16) == _lib.GA_ERR_NULL_ARG
    assert _prefill(lib, d, n=-1) == _lib.GA_ERR_BAD_SHAPE
    # empty inputs are a no-op
    assert _prefill(lib, d, n=0, q=None) == _lib.GA_OK
    assert _prefill(lib, _desc(batch=0), q=None) == _lib.GA_OK


def test_head_strides_choose_the_kernel():
    """Fused [q | gate] rows (stride 2d) keep the fused kernels; strides that
    break their 16-byte row reads send the shape to the generic kernel, and
    the split decode stages refuse it."""
    lib = _lib_or_build()
    packed = _desc(q_head_stride=512, gate_head_stride=512)
    assert lib.ga_prefill_attention_kernel(ctypes.byref(packed), 4096) == b"mirror"
    d3 = _desc(batch=4, n_q_heads=16, n_kv_heads=8, head_dim=128, rot_dim=32, q_head_stride=256,
               gate_head_stride=256)
    assert lib.ga_prefill_attention_kernel(ctypes.byref(d3), 2048) == b"wide"
    d64 = _desc(head_dim=64, rot_dim=16, q_head_stride=128, gate_head_stride=128)
    assert lib.ga_prefill_attention_kernel(ctypes.byref(d64), 64) == b"simple"
    # headwise gate packed as [q | z]: q rows d + 1 apart are not 16-byte aligned
    hw = _desc(gate_mode=_lib.GA_GATE_HEADWISE, q_head_stride=257, gate_head_stride=257)
    assert lib.ga_prefill_attention_kernel(ctypes.byref(hw), 4096) == b"generic"
    assert lib.ga_prefill_chunk_kernel(ctypes.byref(hw), 64, 4096) == b"generic"
    hw8 = _desc(gate_mode=_lib.GA_GATE_HEADWISE, q_head_stride=264, gate_head_stride=264)
    assert lib.ga_prefill_attention_kernel(ctypes.byref(hw8), 4096) == b"mirror"
    assert lib.ga_prefill_chunk_kernel(ctypes.byref(hw8), 64, 4096) == b"mirror"
    # an elementwise gate row stride off the 8-element grid
    odd = _desc(q_head_stride=512, gate_head_stride=260)
    assert lib.ga_prefill_attention_kernel(ctypes.byref(odd), 4096) == b"generic"
    assert lib.ga_decode_partials(ctypes.byref(hw), A16, None, A16, A16, 101, A16, 100, A16, 1 << 30,
                                  None) == _lib.GA_ERR_UNSUPPORTED


def test_forced_kernel_field():
    """desc.kernel forces a kernel that serves the shape; one that does not is
    an error (named "unsupported" by the query), never a silent fallback."""
    lib = _lib_or_build()
    d3 = dict(batch=4, n_q_heads=16, n_kv_heads=8, head_dim=128, rot_dim=32)
    for k, name in ((_lib.GA_KERNEL_WIDE, b"wide"), (_lib.GA_KERNEL_MIRROR, b"mirror"),
                    (_lib.GA_KERNEL_SIMPLE, b"simple"), (_lib.GA_KERNEL_GENERIC, b"generic")):
        assert lib.ga_prefill_attention_kernel(ctypes.byref(_desc(kernel=k, **d3)), 100) == name
    d256 = _desc(kernel=_lib.GA_KERNEL_WIDE)                  # the wide kernel serves d = 128 only
    assert lib.ga_prefill_attention_kernel(ctypes.byref(d256), 4096) == b"unsupported"
    assert _prefill(lib, d256) == _lib.GA_ERR_UNSUPPORTED
    assert lib.ga_prefill_attention(ctypes.byref(d256), 16, A16, A16, 16, A16, 16, A16, None, None, None, A16,
                                    None) == _lib.GA_ERR_UNSUPPORTED
    assert lib.ga_prefill_attention(ctypes.byref(_desc()), 16, A16, A16, 16, A16, 16, A16, None, A16 + 4, None, A16,
                                    None) == _lib.GA_ERR_MISALIGNED
    f32 = _desc(dtype=_lib.GA_F32, kernel=_lib.GA_KERNEL_MIRROR)
    assert lib.ga_prefill_attention_kernel(ctypes.byref(f32), 64) == b"unsupported"
    # chunks: mirrored or generic only
    assert lib.ga_prefill_chunk_kernel(ctypes.byref(_desc(kernel=_lib.GA_KERNEL_GENERIC)), 64, 1100) == b"generic"
    assert lib.ga_prefill_chunk_kernel(ctypes.byref(_desc(kernel=_lib.GA_KERNEL_WIDE)), 64, 1100) == b"unsupported"
    assert lib.ga_prefill_chunk_kernel(ctypes.byref(_desc(kernel=_lib.GA_KERNEL_MIRROR, dtype=_lib.GA_F32)), 64,
                                       1100) == b"unsupported"


def test_workspace_queries_depend_on_arguments_only():
    """No kernel needs a prefill-attention or chunk workspace: the sizes are
    functions of the arguments (the forced-kernel field changes nothing)."""
    lib = _lib_or_build()
    for k in range(5):
        d = _desc(kernel=k)
        assert lib.ga_prefill_workspace_bytes(ctypes.byref(d), 4096) == 4096 * 2 * 256 * 2
        assert lib.ga_prefill_chunk_workspace_bytes(ctypes.byref(d), 64, 1100, 1000) == 0


def test_norm_weights_must_be_aligned():
    """The fused kernels read the RMSNorm weights in 16-byte pieces."""
    lib = _lib_or_build()
    d = _desc()
    assert lib.ga_prefill(ctypes.byref(d), 16, A16, A16, A16, A16, A16 + 4, None, None, None, None, 0, A16,
                          1 << 30, A16, None) == _lib.GA_ERR_MISALIGNED
    assert lib.ga_prefill(ctypes.byref(d), 16, A16, A16, A16, A16, None, A16 + 8, None, None, None, 0, A16,
                          1 << 30, A16, None) == _lib.GA_ERR_MISALIGNED
    assert lib.ga_prefill_keys(ctypes.byref(d), 16, A16, None, A16 + 4, None, A16, None, 16,
                               None) == _lib.GA_ERR_MISALIGNED
    assert lib.ga_decode(ctypes.byref(_desc(batch=4)), A16, A16, A16, A16, A16 + 4, None, A16, A16, 101, A16, 100,
                         A16, 1 << 30, A16, None) == _lib.GA_ERR_MISALIGNED


def test_decode_rejects_bad_arguments():
    lib = _lib_or_build()
    d = _desc(batch=4)

    def call(desc=d, cap=101, max_len=100, lens=A16, ws=A16, ws_bytes=1 << 30, q=A16, out=A16):
        return lib.ga_decode(ctypes.byref(desc), q, A16, A16, A16, None, None, A16, A16, cap, lens, max_len,
                             ws, ws_bytes, out, None)

    assert call(cap=100) == _lib.GA_ERR_BAD_SHAPE            # no room for the appended slot
    assert call(max_len=-1) == _lib.GA_ERR_BAD_SHAPE
    assert call(lens=None) == _lib.GA_ERR_NULL_ARG
    assert call(ws_bytes=16) == _lib.GA_ERR_WORKSPACE
    assert call(q=MIS) == _lib.GA_ERR_MISALIGNED
    assert call(desc=_desc(batch=0), q=None) == _lib.GA_OK
    assert lib.ga_decode_partials(ctypes.byref(_desc(head_dim=96, rot_dim=16)), A16, None, A16, A16, 101, A16,
                                  100, A16, 1 << 30, None) == _lib.GA_ERR_UNSUPPORTED


def test_prefill_chunk_rejects_bad_arguments_and_names_its_kernel():
    lib = _lib_or_build()
    d = _desc(batch=2)

    def call(desc=d, n=64, cap=1100, max_len=1000, lens=A16, q=A16, k_cache=A16, out=A16, gate=A16, ws=A16,
             ws_bytes=1 << 30):
        return lib.ga_prefill_chunk(ctypes.byref(desc), n, q, A16, A16, gate, None, None, None, k_cache, A16, cap,
                                    lens, None, max_len, ws, ws_bytes, out, None)

    assert call(cap=1063) == _lib.GA_ERR_BAD_SHAPE             # cap < max_cache_len + seq_len
    assert call(max_len=-1) == _lib.GA_ERR_BAD_SHAPE
    assert call(lens=None) == _lib.GA_ERR_NULL_ARG
    assert call(k_cache=None) == _lib.GA_ERR_NULL_ARG
    assert call(gate=None) == _lib.GA_ERR_NULL_ARG             # elementwise gate required
    assert call(out=MIS) == _lib.GA_ERR_MISALIGNED
    assert call(n=-1) == _lib.GA_ERR_BAD_SHAPE
    assert call(max_len=(1 << 30) - 10, cap=(1 << 30) + 100) == _lib.GA_ERR_UNSUPPORTED
    assert call(desc=_desc(batch=0), q=None) == _lib.GA_OK
    assert lib.ga_prefill_chunk_workspace_bytes(ctypes.byref(d), 64, 1100, 1000) == 0
    assert call(ws=None, ws_bytes=0, lens=None) == _lib.GA_ERR_NULL_ARG
    assert lib.ga_prefill_chunk_keys(ctypes.byref(d), 64, A16, A16, None, None, None, None, 1000, A16, A16, 1100,
                                     None) == _lib.GA_ERR_NULL_ARG
    assert lib.ga_prefill_chunk_attention(ctypes.byref(d), 64, A16, A16, A16, 1000, A16, None, 1000, A16, None,
                                          None, None, A16, 1 << 30, A16, None) == _lib.GA_ERR_BAD_SHAPE
    assert lib.ga_prefill_chunk_kernel(ctypes.byref(d), 64, 1100) == b"mirror"
    assert lib.ga_prefill_chunk_kernel(ctypes.byref(_desc(dtype=_lib.GA_F32)), 64, 1100) == b"generic"
    assert lib.ga_prefill_chunk_kernel(ctypes.byref(_desc(head_dim=64, rot_dim=16)), 64, 1100) == b"generic"


def test_binding_reads_head_strides_from_views():
    """The binding's stride reading (host logic only; CPU tensors)."""
    import torch
    from gated_gqa_softmax_amd.api import head_stride

    def hs(t, lead, H, width):
        return head_stride(t.shape, t.stride(), lead, H, width)

    B, n, H, d = 2, 5, 4, 8
    qg = torch.zeros(B, n, H, 2 * d)
    assert hs(qg[..., :d], 2, H, d) == 2 * d and hs(qg[..., d:], 2, H, d) == 2 * d
    assert hs(torch.zeros(B, n, H, d), 2, H, d) == d                       # dense
    assert hs(torch.zeros(B, n, H), 2, H, 1) == 1                          # dense headwise
    qz = torch.zeros(B, n, H, d + 1)                                       # headwise [q | z]
    assert hs(qz[..., :d], 2, H, d) == d + 1 and hs(qz[..., d], 2, H, 1) == d + 1
    assert hs(qz[..., d:], 2, H, 1) == d + 1                               # [.., H, 1] view
    dq = torch.zeros(B, H, 2 * d)                                          # decode: [B, H, 2d]
    assert hs(dq[..., :d], 1, H, d) == 2 * d
    assert hs(torch.zeros(1, 1, H, 2 * d)[..., :d], 2, H, d) == 2 * d       # size-1 leading dims
    assert hs(torch.zeros(1, 1, 1, 2 * d)[..., d:], 2, 1, d) == d           # nothing to read: dense
    with pytest.raises(ValueError):
        hs(torch.zeros(B, H, n, d).transpose(1, 2), 2, H, d)              # head-major: not rows of a token
    with pytest.raises(ValueError):
        hs(torch.zeros(B, n, H, 2 * d)[..., ::2], 2, H, d)                # innermost dim not dense
    assert hs(torch.zeros(B, n, 2 * H, d)[:, :, ::2], 2, H, d) == 2 * d   # every other head row
    with pytest.raises(ValueError):
        hs(torch.zeros(B, n, H, d), 2, H + 1, d)                          # wrong head count
    with pytest.raises(ValueError):
        hs(torch.zeros(B, 2 * n, H, 2 * d)[:, ::2, :, :d], 2, H, d)       # tokens two rows apart


def test_backward_rejects_bad_arguments():
    lib = _lib_or_build()
    d = _desc(batch=1)
    need = lib.ga_prefill_backward_workspace_bytes(ctypes.byref(d), 64)
    assert need > 0 and need % 256 == 0

    def call(desc=d, n=64, q=A16, gate=A16, dgate=A16, ws=A16, ws_bytes=1 << 40, dq=A16):
        return lib.ga_prefill_backward(ctypes.byref(desc), n, q, A16, A16, gate, None, None, None, A16, dq, A16,
                                       A16, dgate, None, None, ws, ws_bytes, None)

    assert call(n=-1) == _lib.GA_ERR_BAD_SHAPE
    assert call(q=None) == _lib.GA_ERR_NULL_ARG
    assert call(dq=MIS) == _lib.GA_ERR_MISALIGNED
    assert call(gate=None) == _lib.GA_ERR_NULL_ARG                 # elementwise gate needs the gate
    assert call(dgate=None) == _lib.GA_ERR_NULL_ARG                # ... and its gradient
    assert call(ws_bytes=need - 256) == _lib.GA_ERR_WORKSPACE
    assert call(ws=A16 + 16) == _lib.GA_ERR_MISALIGNED             # the workspace is 256-byte aligned
    assert call(desc=_desc(dtype=_lib.GA_F32)) == _lib.GA_ERR_UNSUPPORTED
    assert call(desc=_desc(head_dim=96, rot_dim=16)) == _lib.GA_ERR_UNSUPPORTED
    assert call(desc=_desc(gate_act=_lib.GA_ACT_SILU)) == _lib.GA_ERR_UNSUPPORTED
    assert call(desc=_desc(q_head_stride=512)) == _lib.GA_ERR_UNSUPPORTED
    # empty inputs are a no-op, even without buffers
    assert call(n=0, q=None, ws=None, ws_bytes=0) == _lib.GA_OK
    assert call(desc=_desc(batch=0), q=None, ws=None, ws_bytes=0) == _lib.GA_OK


def test_training_pair_rejects_bad_arguments():
    """ga_prefill_lse and ga_prefill_backward_lse: the backward's shape rules,
    the statistics buffer, the output the backward reads, the workspace."""
    lib = _lib_or_build()
    d = _desc(batch=1)
    need = lib.ga_prefill_lse_workspace_bytes(ctypes.byref(d), 64)
    # bf16 q-hat [1,64,H,d] and k-hat [1,64,G,d], each rounded to 256 bytes
    assert need == 64 * d.n_q_heads * d.head_dim * 2 + 64 * d.n_kv_heads * d.head_dim * 2
    bneed = lib.ga_prefill_backward_workspace_bytes(ctypes.byref(d), 64)

    def fwd(desc=d, n=64, q=A16, gate=A16, ws=A16, ws_bytes=1 << 40, out=A16, lse=A16):
        return lib.ga_prefill_lse(ctypes.byref(desc), n, q, A16, A16, gate, None, None, None, ws, ws_bytes, out, lse,
                                  None)

    def bwd(desc=d, n=64, out=A16, lse=A16, ws_bytes=1 << 40, dq=A16):
        return lib.ga_prefill_backward_lse(ctypes.byref(desc), n, A16, A16, A16, A16, None, None, None, out, lse,
                                           A16, dq, A16, A16, A16, None, None, A16, ws_bytes, None)

    assert fwd(n=-1) == _lib.GA_ERR_BAD_SHAPE
    assert fwd(q=None) == _lib.GA_ERR_NULL_ARG
    assert fwd(gate=None) == _lib.GA_ERR_NULL_ARG
    assert fwd(out=None) == _lib.GA_ERR_NULL_ARG
    assert fwd(lse=None) == _lib.GA_ERR_NULL_ARG
    assert fwd(lse=A16 + 2) == _lib.GA_ERR_MISALIGNED
    assert fwd(ws_bytes=need - 256) == _lib.GA_ERR_WORKSPACE
    assert fwd(ws=A16 + 16) == _lib.GA_ERR_MISALIGNED
    assert fwd(desc=_desc(dtype=_lib.GA_F32)) == _lib.GA_ERR_UNSUPPORTED
    assert fwd(desc=_desc(gate_act=_lib.GA_ACT_SILU)) == _lib.GA_ERR_UNSUPPORTED
    assert fwd(n=0, q=None, ws=None, ws_bytes=0, out=None, lse=None) == _lib.GA_OK
    assert bwd(out=None) == _lib.GA_ERR_NULL_ARG
    assert bwd(lse=None) == _lib.GA_ERR_NULL_ARG
    assert bwd(lse=A16 + 1) == _lib.GA_ERR_MISALIGNED
    assert bwd(dq=MIS) == _lib.GA_ERR_MISALIGNED
    assert bwd(ws_bytes=bneed - 256) == _lib.GA_ERR_WORKSPACE
    assert bwd(desc=_desc(head_dim=96, rot_dim=16)) == _lib.GA_ERR_UNSUPPORTED
    assert bwd(n=0, out=None, lse=None) == _lib.GA_OK


def test_noalloc_decode_rejects_oversized_steps_before_any_launch():
    """The static-scratch decode refuses a step whose partials exceed the
    scratch, before touching a device (q is also NULL, so nothing further
    could run even if the size check were passed)."""
    lib = _lib_or_build()
    d = _desc(batch=64)
    big = 1 << 20
    assert lib.ga_decode_workspace_bytes(ctypes.byref(d), big) > _lib.GA_NOALLOC_SCRATCH_BYTES
    assert lib.ga_decode_noalloc(ctypes.byref(d), None, A16, A16, A16, None, None, A16, A16, big + 1, A16, big, A16,
                                 None) == _lib.GA_ERR_WORKSPACE
    assert b"static scratch" in lib.ga_last_error()
