"""Python binding of the C ABI (include/ga.h), one function per entry point.

Argument marshalling only: each function checks that tensors are on the
GPU, contiguous (q and the gate: rows of heads at a fixed stride, such as the
two halves of a fused q projection's output) and of the declared element
type, fills the ``ga_attn_desc``,
passes raw device pointers and the current HIP stream to libga.so, and
raises ``GaError`` when the library returns a non-OK status. Every step of
the computation runs in the library's HIP kernels. PyTorch supplies device
memory and the stream; workspaces the caller does not pass are allocated
here with torch.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import AttnDesc

_GATE = {"none": _lib.GA_GATE_NONE, "headwise": _lib.GA_GATE_HEADWISE,
         "elementwise": _lib.GA_GATE_ELEMENTWISE}
_DTYPE = {torch.bfloat16: _lib.GA_BF16, torch.float32: _lib.GA_F32}
_ACT = {"sigmoid": _lib.GA_ACT_SIGMOID, "ns_sigmoid": _lib.GA_ACT_NS_SIGMOID, "silu": _lib.GA_ACT_SILU,
        "identity": _lib.GA_ACT_IDENTITY}
_COMBINE = {"mul": _lib.GA_COMBINE_MUL, "add": _lib.GA_COMBINE_ADD}
_KERNEL = {"auto": _lib.GA_KERNEL_AUTO, "wide": _lib.GA_KERNEL_WIDE, "mirror": _lib.GA_KERNEL_MIRROR,
           "simple": _lib.GA_KERNEL_SIMPLE, "generic": _lib.GA_KERNEL_GENERIC}
_BWD_KERNEL = {"auto": _lib.GA_BWD_AUTO, "plain": _lib.GA_BWD_PLAIN}


class GaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        self.status = status
        self.name = lib.ga_status_string(status).decode()
        self.detail = lib.ga_last_error().decode()
        super().__init__(f"{where}: {self.name}: {self.detail}")


def make_desc(batch, n_q_heads, n_kv_heads, head_dim, rot_dim=0, rope_base=10000.0, rms_eps=1e-6,
              softmax_scale=0.0, dtype=torch.bfloat16, gate_mode="none", q_head_stride=0,
              gate_head_stride=0, gate_act="sigmoid", gate_combine="mul", share_heads=False,
              share_tokens=False, out_norm_w: Optional[torch.Tensor] = None, out_norm_eps=1e-6,
              kernel="auto", bwd_kernel="auto") -> AttnDesc:
    """Descriptor. The head strides matter only to the kernel-name queries
    (the entry points below take them from the q and gate tensors). Gate
    variants: ``gate_act`` sigmoid | ns_sigmoid | silu | identity,
    ``gate_combine`` mul | add, ``share_heads`` (gate [.., d] or [..] per
    token), ``share_tokens`` (gate [H, d] or [H]); ``out_norm_w`` a float32
    GPU tensor [d] for the per-head output RMSNorm (the descriptor keeps a
    reference to it). ``kernel`` auto | wide | mirror | simple | generic
    forces the prefill / chunk attention kernel, ``bwd_kernel`` auto | plain
    the backward's product kernels (tests and tuning)."""
    if out_norm_w is not None:
        if not (out_norm_w.is_cuda and out_norm_w.dtype == torch.float32 and out_norm_w.is_contiguous()
                and out_norm_w.numel() == int(head_dim)):
            raise ValueError("out_norm_w must be a contiguous float32 GPU tensor of head_dim values")
    share = (_lib.GA_SHARE_HEADS if share_heads else 0) | (_lib.GA_SHARE_TOKENS if share_tokens else 0)
    d = AttnDesc(int(batch), int(n_q_heads), int(n_kv_heads), int(head_dim), int(rot_dim),
                 float(rope_base), float(rms_eps), float(softmax_scale),
                 _DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
                 _GATE[gate_mode] if isinstance(gate_mode, str) else int(gate_mode),
                 int(q_head_stride), int(gate_head_stride),
                 _ACT[gate_act] if isinstance(gate_act, str) else int(gate_act),
                 _COMBINE[gate_combine] if isinstance(gate_combine, str) else int(gate_combine),
                 share, float(out_norm_eps), out_norm_w.data_ptr() if out_norm_w is not None else None,
                 _KERNEL[kernel] if isinstance(kernel, str) else int(kernel),
                 _BWD_KERNEL[bwd_kernel] if isinstance(bwd_kernel, str) else int(bwd_kernel))
    d._keep = out_norm_w
    return d


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _tensor(t: Optional[torch.Tensor], name: str, shape, dtype, required=True) -> Optional[int]:
    """Pointer of a dense GPU tensor of exactly ``shape`` and ``dtype`` (None
    allowed when not ``required``); ValueError otherwise, so that no kernel is
    ever handed a buffer smaller than the descriptor implies."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if tuple(t.shape) != tuple(int(s) for s in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(s) for s in shape)}")
    return _ptr(t, name, dtype)


def _lens(t: Optional[torch.Tensor], name: str, batch: int, required=True) -> Optional[int]:
    """Pointer of a per-sequence int32 GPU vector with at least ``batch`` entries."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if t.dim() != 1 or t.numel() < batch:
        raise ValueError(f"{name} must be a 1-D tensor of at least {batch} entries, got shape {tuple(t.shape)}")
    return _ptr(t, name, torch.int32)


def _norm_w(t: Optional[torch.Tensor], name: str, desc: AttnDesc) -> Optional[int]:
    return _tensor(t, name, (desc.head_dim,), torch.float32, required=False)


def _cache_pair(k_cache, v_cache, desc: AttnDesc, et, min_cap: int):
    """(k_cache ptr, v_cache ptr, capacity) of two [B, cap, G, d] caches of one shape."""
    if k_cache is None or v_cache is None:
        raise ValueError("k_cache and v_cache are both required")
    cap = int(k_cache.shape[1]) if k_cache.dim() == 4 else -1
    shape = (desc.batch, cap, desc.n_kv_heads, desc.head_dim)
    kp = _tensor(k_cache, "k_cache", shape, et)
    vp = _tensor(v_cache, "v_cache", shape, et)
    if cap < min_cap:
        raise ValueError(f"cache capacity {cap} < {min_cap} required")
    return kp, vp, cap


def _workspace_arg(workspace: Optional[torch.Tensor], nbytes: int, device):
    """(tensor, pointer, bytes) of a workspace of at least ``nbytes`` bytes,
    allocated here (torch) when the caller passes none."""
    if nbytes == 0 and workspace is None:
        return None, None, 0
    if workspace is None:
        workspace = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    nb = workspace.numel() * workspace.element_size()
    if nb < nbytes:
        raise ValueError(f"workspace holds {nb} bytes, {nbytes} required")
    return workspace, _ptr(workspace, "workspace"), nb


def head_stride(shape, strides, lead: int, n_heads: int, width: int, name: str = "tensor") -> int:
    """Head stride (elements) of q or a gate given as a shape and strides, as
    the ABI reads them: dims [*lead, H, width] (a headwise gate: [*lead, H] or
    [*lead, H, 1]) whose innermost dim is dense, with head rows ``stride``
    apart and the rows of one token, then of one sequence, following each
    other. Contiguous tensors and views of a fused [*lead, H, 2d] projection
    output qualify; anything else raises ValueError."""
    shape, strides = list(shape), list(strides)
    if width == 1 and len(shape) == lead + 2 and shape[-1] == 1:
        shape, strides = shape[:-1], strides[:-1]
    rank = lead + (1 if width == 1 else 2)
    if len(shape) != rank or shape[lead] != n_heads or (width > 1 and shape[-1] != width):
        raise ValueError(f"{name} has shape {tuple(shape)}, expected {lead} leading dims, {n_heads} heads"
                         f"{'' if width == 1 else f' and {width} values per head'}")
    if width > 1 and strides[-1] != 1:
        raise ValueError(f"{name}: the innermost dim must be dense")
    # the head stride is what the outermost dims of size > 1 imply (a dim of
    # size 1 has no meaningful stride); every such dim must agree with it
    stride, inner = width, 1
    for dim in range(lead, -1, -1):
        if shape[dim] > 1:
            if strides[dim] % inner:
                raise ValueError(f"{name}: strides {tuple(strides)} are not head rows at one stride")
            stride = strides[dim] // inner
            break
        inner *= shape[dim]
    expect = stride
    for dim in range(lead, -1, -1):
        if shape[dim] > 1 and strides[dim] != expect:
            raise ValueError(f"{name}: strides {tuple(strides)} are not head rows at one stride")
        expect *= shape[dim]
    if stride < width or stride >= 2 ** 31:
        raise ValueError(f"{name}: head stride {stride} out of range")
    return stride


def _head_rows(t: torch.Tensor, name: str, dtype, lead: int, n_heads: int, width: int) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return head_stride(t.shape, t.stride(), lead, n_heads, width, name)


def _qg(desc: AttnDesc, q, gate, lead_shape, et):
    """Copy of ``desc`` with the head strides of q and the gate, and their
    pointers. ``lead_shape`` is (B, n) for prefill, (B,) for decode: q and an
    unshared gate must have exactly those leading dims."""
    lead = len(lead_shape)
    if q is None:
        raise ValueError("q is required")
    if tuple(q.shape[:lead]) != tuple(lead_shape):
        raise ValueError(f"q has shape {tuple(q.shape)}, expected leading dims {tuple(lead_shape)}")
    d2 = AttnDesc.from_buffer_copy(desc)
    d2.q_head_stride = _head_rows(q, "q", et, lead, desc.n_q_heads, desc.head_dim)
    gp = None
    if desc.gate_mode != _lib.GA_GATE_NONE and gate is None:
        raise ValueError("gate is required by the descriptor's gate mode")
    if gate is not None and desc.gate_mode != _lib.GA_GATE_NONE:
        gw = desc.head_dim if desc.gate_mode == _lib.GA_GATE_ELEMENTWISE else 1
        if desc.gate_share:
            d2.gate_head_stride = _shared_gate(gate, desc, lead, et, gw)
        else:
            d2.gate_head_stride = _head_rows(gate, "gate", et, lead, desc.n_q_heads, gw)
        if not (desc.gate_share & _lib.GA_SHARE_TOKENS) and tuple(gate.shape[:lead]) != tuple(lead_shape):
            raise ValueError(f"gate has shape {tuple(gate.shape)}, expected leading dims {tuple(lead_shape)}")
        gp = gate.data_ptr()
    return d2, q.data_ptr(), gp


def _shared_gate(gate: torch.Tensor, desc: AttnDesc, lead: int, et, width: int) -> int:
    """A gate without its head dim and/or its batch and token dims: a dense
    tensor of [*lead] (unless shared by the tokens) + [H] (unless shared by
    the heads) + [d] (elementwise) values."""
    if not gate.is_cuda or gate.dtype != et:
        raise ValueError(f"gate must be a {et} GPU tensor")
    if not gate.is_contiguous():
        raise ValueError("a shared gate must be contiguous")
    tail = (desc.head_dim,) if width > 1 else ()
    heads = () if desc.gate_share & _lib.GA_SHARE_HEADS else (desc.n_q_heads,)
    want = heads + tail
    shape = tuple(gate.shape)
    if desc.gate_share & _lib.GA_SHARE_TOKENS:
        ok = shape == want or (not want and shape in ((1,),))
    else:
        ok = len(shape) == lead + len(want) and shape[lead:] == want
    if not ok:
        raise ValueError(f"gate has shape {shape}; the shared gate needs [{'' if desc.gate_share & 2 else 'lead dims, '}"
                         f"{', '.join(map(str, want))}]")
    return 0


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str):
    if status != _lib.GA_OK:
        raise GaError(status, where)


def _elem_dtype(desc: AttnDesc):
    return torch.bfloat16 if desc.dtype == _lib.GA_BF16 else torch.float32


def ga_version() -> int:
    return _lib.load().ga_version()


def ga_status_string(status: int) -> str:
    return _lib.load().ga_status_string(status).decode()


def ga_last_error() -> str:
    return _lib.load().ga_last_error().decode()


def ga_fast_path(dtype, head_dim: int, rot_dim: int, group: int) -> int:
    dt = _DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return _lib.load().ga_fast_path(dt, head_dim, rot_dim, group)


def ga_decode_split_keys() -> int:
    return _lib.load().ga_decode_split_keys()


def ga_prefill_workspace_bytes(desc: AttnDesc, seq_len: int) -> int:
    return _lib.load().ga_prefill_workspace_bytes(ctypes.byref(desc), seq_len)


def ga_prefill_attention_kernel(desc: AttnDesc, seq_len: int) -> str:
    return _lib.load().ga_prefill_attention_kernel(ctypes.byref(desc), seq_len).decode()


def ga_decode_workspace_bytes(desc: AttnDesc, max_cache_len: int) -> int:
    return _lib.load().ga_decode_workspace_bytes(ctypes.byref(desc), max_cache_len)


def _seq(q, lead: int = 2):
    if q is None or q.dim() < lead:
        raise ValueError("q must have batch and token dims")
    return int(q.shape[0]), int(q.shape[1])


def ga_prefill(desc: AttnDesc, q, k, v, gate=None, q_norm_w=None, k_norm_w=None, positions=None,
               k_cache=None, v_cache=None, out=None, workspace=None, stream=None) -> torch.Tensor:
    """out [B,n,H*d] = gated GQA causal attention of q [B,n,H,d], k, v [B,n,G,d]."""
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, n = desc.batch, _seq(q)[1]
    G, hd = desc.n_kv_heads, desc.head_dim
    d2, qp, gp = _qg(desc, q, gate, (B, n), et)
    if out is None:
        out = torch.empty((B, n, desc.n_q_heads * hd), dtype=et, device=q.device)
    op = _tensor(out, "out", (B, n, desc.n_q_heads * hd), et)
    kp = _tensor(k, "k", (B, n, G, hd), et)
    vp = _tensor(v, "v", (B, n, G, hd), et)
    cap, kcp, vcp = 0, None, None
    if k_cache is not None or v_cache is not None:
        kcp, vcp, cap = _cache_pair(k_cache, v_cache, desc, et, n)
        ws, wp, wb = _workspace_arg(workspace, 0, q.device)
    else:
        ws, wp, wb = _workspace_arg(workspace, ga_prefill_workspace_bytes(desc, n), q.device)
    st = lib.ga_prefill(ctypes.byref(d2), n, qp, kp, vp, gp, _norm_w(q_norm_w, "q_norm_w", desc),
                        _norm_w(k_norm_w, "k_norm_w", desc),
                        _tensor(positions, "positions", (B, n), torch.int32, required=False),
                        kcp, vcp, cap, wp, wb, op, _stream(stream))
    _check(st, "ga_prefill")
    return out


def ga_prefill_keys(desc: AttnDesc, k, v=None, k_norm_w=None, positions=None, k_hat=None, v_out=None,
                    stream=None) -> torch.Tensor:
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, n = desc.batch, _seq(k)[1]
    G, hd = desc.n_kv_heads, desc.head_dim
    kp = _tensor(k, "k", (B, n, G, hd), et)
    if k_hat is None:
        k_hat = torch.empty_like(k)
    cap = int(k_hat.shape[1]) if k_hat.dim() == 4 else -1
    khp = _tensor(k_hat, "k_hat", (B, cap, G, hd), et)
    if cap < n:
        raise ValueError(f"k_hat holds {cap} rows per sequence, {n} required")
    vp = vop = None
    if v_out is not None:
        vp = _tensor(v, "v", (B, n, G, hd), et)
        vop = _tensor(v_out, "v_out", (B, cap, G, hd), et)
    st = lib.ga_prefill_keys(ctypes.byref(desc), n, kp, vp, _norm_w(k_norm_w, "k_norm_w", desc),
                             _tensor(positions, "positions", (B, n), torch.int32, required=False),
                             khp, vop, cap, _stream(stream))
    _check(st, "ga_prefill_keys")
    return k_hat


def ga_prefill_attention(desc: AttnDesc, q, k_hat, v, gate=None, q_norm_w=None, positions=None, out=None,
                         stream=None, k_norm_w=None) -> torch.Tensor:
    """Attention stage of ga_prefill over prepared keys; ``k_norm_w`` = the
    weights ga_prefill_keys normed k_hat with (lets the kernels bound the
    scores), or None."""
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, n = desc.batch, _seq(q)[1]
    G, hd = desc.n_kv_heads, desc.head_dim
    d2, qp, gp = _qg(desc, q, gate, (B, n), et)
    if out is None:
        out = torch.empty((B, n, desc.n_q_heads * hd), dtype=et, device=q.device)
    op = _tensor(out, "out", (B, n, desc.n_q_heads * hd), et)
    kcap = int(k_hat.shape[1]) if k_hat is not None and k_hat.dim() == 4 else -1
    vcap = int(v.shape[1]) if v is not None and v.dim() == 4 else -1
    khp = _tensor(k_hat, "k_hat", (B, kcap, G, hd), et)
    vp = _tensor(v, "v", (B, vcap, G, hd), et)
    if kcap < n or vcap < n:
        raise ValueError(f"k_hat / v hold {kcap} / {vcap} rows per sequence, {n} required")
    st = lib.ga_prefill_attention(ctypes.byref(d2), n, qp, khp, kcap, vp, vcap, gp,
                                  _norm_w(q_norm_w, "q_norm_w", desc), _norm_w(k_norm_w, "k_norm_w", desc),
                                  _tensor(positions, "positions", (B, n), torch.int32, required=False),
                                  op, _stream(stream))
    _check(st, "ga_prefill_attention")
    return out


def ga_prefill_chunk_kernel(desc: AttnDesc, seq_len: int, cache_cap: int) -> str:
    return _lib.load().ga_prefill_chunk_kernel(ctypes.byref(desc), seq_len, cache_cap).decode()


def ga_prefill_chunk_workspace_bytes(desc: AttnDesc, seq_len: int, cache_cap: int, max_cache_len: int) -> int:
    return int(_lib.load().ga_prefill_chunk_workspace_bytes(ctypes.byref(desc), seq_len, cache_cap, max_cache_len))


def _chunk_args(desc, q, k_cache, v_cache, cache_lens, chunk_lens, max_cache_len, workspace, et):
    B, n = desc.batch, _seq(q)[1]
    if int(max_cache_len) < 0:
        raise ValueError("max_cache_len must be >= 0")
    kcp, vcp, cap = _cache_pair(k_cache, v_cache, desc, et, int(max_cache_len) + n)
    lp = _lens(cache_lens, "cache_lens", B)
    clp = _lens(chunk_lens, "chunk_lens", B, required=False)
    nbytes = ga_prefill_chunk_workspace_bytes(desc, n, cap, int(max_cache_len))
    ws, wp, wb = _workspace_arg(workspace, nbytes, q.device)
    return B, n, kcp, vcp, cap, lp, clp, ws, wp, wb


def ga_prefill_chunk(desc: AttnDesc, q, k, v, k_cache, v_cache, cache_lens, max_cache_len: int, gate=None,
                     q_norm_w=None, k_norm_w=None, positions=None, chunk_lens=None, out=None,
                     workspace=None, stream=None) -> torch.Tensor:
    """Chunk of seq_len new rows per sequence after cache_lens[b] cached tokens.

    Writes K-hat/V of the real rows to cache slots [L_b, L_b + n_b) and the
    gated attention of those rows to out [B,seq_len,H*d]; padding rows
    (i >= chunk_lens[b]) are left as they were.
    """
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, n, kcp, vcp, cap, lp, clp, _ws, wp, wb = _chunk_args(desc, q, k_cache, v_cache, cache_lens, chunk_lens,
                                                            max_cache_len, workspace, et)
    G, hd = desc.n_kv_heads, desc.head_dim
    d2, qp, gp = _qg(desc, q, gate, (B, n), et)
    if out is None:
        out = torch.zeros((B, n, desc.n_q_heads * hd), dtype=et, device=q.device)
    op = _tensor(out, "out", (B, n, desc.n_q_heads * hd), et)
    st = lib.ga_prefill_chunk(ctypes.byref(d2), n, qp, _tensor(k, "k", (B, n, G, hd), et),
                              _tensor(v, "v", (B, n, G, hd), et), gp, _norm_w(q_norm_w, "q_norm_w", desc),
                              _norm_w(k_norm_w, "k_norm_w", desc),
                              _tensor(positions, "positions", (B, n), torch.int32, required=False),
                              kcp, vcp, cap, lp, clp, int(max_cache_len), wp, wb, op, _stream(stream))
    _check(st, "ga_prefill_chunk")
    return out


def ga_prefill_chunk_keys(desc: AttnDesc, k, v, k_cache, v_cache, cache_lens, max_cache_len: int, k_norm_w=None,
                          positions=None, chunk_lens=None, stream=None):
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, n = desc.batch, _seq(k)[1]
    G, hd = desc.n_kv_heads, desc.head_dim
    if int(max_cache_len) < 0:
        raise ValueError("max_cache_len must be >= 0")
    kcp, vcp, cap = _cache_pair(k_cache, v_cache, desc, et, int(max_cache_len) + n)
    st = lib.ga_prefill_chunk_keys(ctypes.byref(desc), n, _tensor(k, "k", (B, n, G, hd), et),
                                   _tensor(v, "v", (B, n, G, hd), et), _norm_w(k_norm_w, "k_norm_w", desc),
                                   _tensor(positions, "positions", (B, n), torch.int32, required=False),
                                   _lens(cache_lens, "cache_lens", B), _lens(chunk_lens, "chunk_lens", B, False),
                                   int(max_cache_len), kcp, vcp, cap, _stream(stream))
    _check(st, "ga_prefill_chunk_keys")


def ga_prefill_chunk_attention(desc: AttnDesc, q, k_cache, v_cache, cache_lens, max_cache_len: int, gate=None,
                               q_norm_w=None, k_norm_w=None, positions=None, chunk_lens=None, out=None,
                               workspace=None, stream=None) -> torch.Tensor:
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, n, kcp, vcp, cap, lp, clp, _ws, wp, wb = _chunk_args(desc, q, k_cache, v_cache, cache_lens, chunk_lens,
                                                            max_cache_len, workspace, et)
    hd = desc.head_dim
    d2, qp, gp = _qg(desc, q, gate, (B, n), et)
    if out is None:
        out = torch.zeros((B, n, desc.n_q_heads * hd), dtype=et, device=q.device)
    op = _tensor(out, "out", (B, n, desc.n_q_heads * hd), et)
    st = lib.ga_prefill_chunk_attention(ctypes.byref(d2), n, qp, kcp, vcp, cap, lp, clp, int(max_cache_len),
                                        gp, _norm_w(q_norm_w, "q_norm_w", desc), _norm_w(k_norm_w, "k_norm_w", desc),
                                        _tensor(positions, "positions", (B, n), torch.int32, required=False),
                                        wp, wb, op, _stream(stream))
    _check(st, "ga_prefill_chunk_attention")
    return out


def ga_prefill_backward_workspace_bytes(desc: AttnDesc, seq_len: int) -> int:
    return int(_lib.load().ga_prefill_backward_workspace_bytes(ctypes.byref(desc), seq_len))


def _gate_shape(desc: AttnDesc, qshape):
    if desc.gate_mode == _lib.GA_GATE_NONE:
        return None
    return qshape if desc.gate_mode == _lib.GA_GATE_ELEMENTWISE else qshape[:3]


def ga_prefill_lse_workspace_bytes(desc: AttnDesc, seq_len: int) -> int:
    return int(_lib.load().ga_prefill_lse_workspace_bytes(ctypes.byref(desc), seq_len))


def ga_prefill_lse(desc: AttnDesc, q, k, v, gate=None, q_norm_w=None, k_norm_w=None, positions=None, out=None,
                   lse=None, workspace=None, stream=None):
    """Training forward: (out [B,n,H*d], lse [B,n,H] float32), lse the log2
    of each causal softmax row's normalising sum, for ga_prefill_backward_lse."""
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, n = desc.batch, _seq(q)[1]
    H, G, hd = desc.n_q_heads, desc.n_kv_heads, desc.head_dim
    qshape, kshape = (B, n, H, hd), (B, n, G, hd)
    gshape = _gate_shape(desc, qshape)
    if out is None:
        out = torch.empty((B, n, H * hd), dtype=et, device=q.device)
    if lse is None:
        lse = torch.empty((B, n, H), dtype=torch.float32, device=q.device)
    ws, wp, wb = _workspace_arg(workspace, ga_prefill_lse_workspace_bytes(desc, n), q.device)
    st = lib.ga_prefill_lse(ctypes.byref(desc), n, _tensor(q, "q", qshape, et), _tensor(k, "k", kshape, et),
                            _tensor(v, "v", kshape, et),
                            _tensor(gate, "gate", gshape, et) if gshape is not None else None,
                            _norm_w(q_norm_w, "q_norm_w", desc), _norm_w(k_norm_w, "k_norm_w", desc),
                            _tensor(positions, "positions", (B, n), torch.int32, required=False), wp, wb,
                            _tensor(out, "out", (B, n, H * hd), et), _tensor(lse, "lse", (B, n, H), torch.float32),
                            _stream(stream))
    _check(st, "ga_prefill_lse")
    return out, lse


def ga_prefill_backward(desc: AttnDesc, q, k, v, dout, gate=None, q_norm_w=None, k_norm_w=None, positions=None,
                        workspace=None, stream=None, weight_grads=True, grads: Optional[dict] = None,
                        out=None, lse=None) -> dict:
    """Gradients of sum(dout * ga_prefill(...)): dict with dq, dk, dv, dgate
    (None without a gate) and dq_norm_w, dk_norm_w (None without that norm
    weight, or with weight_grads=False). ``grads`` may hold preallocated
    output tensors under the same keys. With ``out`` and ``lse`` from
    ga_prefill_lse on the same inputs, ga_prefill_backward_lse runs instead
    (no recomputation of the forward attention)."""
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, n = desc.batch, _seq(q)[1]
    H, G, hd = desc.n_q_heads, desc.n_kv_heads, desc.head_dim
    qshape, kshape = (B, n, H, hd), (B, n, G, hd)
    gshape = _gate_shape(desc, qshape)
    if (out is None) != (lse is None):
        raise ValueError("out and lse go together")
    grads = grads or {}
    dq = grads.get("dq", None)
    dq = torch.empty(qshape, dtype=et, device=q.device) if dq is None else dq
    dk = grads.get("dk", None)
    dk = torch.empty(kshape, dtype=et, device=q.device) if dk is None else dk
    dv = grads.get("dv", None)
    dv = torch.empty(kshape, dtype=et, device=q.device) if dv is None else dv
    dgate = grads.get("dgate", None)
    if dgate is None and gshape is not None:
        dgate = torch.empty(gshape, dtype=et, device=q.device)
    dwq = grads.get("dq_norm_w", None)
    if dwq is None and q_norm_w is not None and weight_grads:
        dwq = torch.empty_like(q_norm_w)
    dwk = grads.get("dk_norm_w", None)
    if dwk is None and k_norm_w is not None and weight_grads:
        dwk = torch.empty_like(k_norm_w)
    ws, wp, wb = _workspace_arg(workspace, ga_prefill_backward_workspace_bytes(desc, n), q.device)
    front = (ctypes.byref(desc), n, _tensor(q, "q", qshape, et), _tensor(k, "k", kshape, et),
              _tensor(v, "v", kshape, et), _tensor(gate, "gate", gshape, et) if gshape is not None else None,
              _norm_w(q_norm_w, "q_norm_w", desc), _norm_w(k_norm_w, "k_norm_w", desc),
              _tensor(positions, "positions", (B, n), torch.int32, required=False))
    rest = (_tensor(dout, "dout", (B, n, H * hd), et), _tensor(dq, "dq", qshape, et), _tensor(dk, "dk", kshape, et),
            _tensor(dv, "dv", kshape, et), _tensor(dgate, "dgate", gshape, et) if gshape is not None else None,
            _norm_w(dwq, "dq_norm_w", desc), _norm_w(dwk, "dk_norm_w", desc), wp, wb, _stream(stream))
    if lse is None:
        st = lib.ga_prefill_backward(*front, *rest)
        _check(st, "ga_prefill_backward")
    else:
        st = lib.ga_prefill_backward_lse(*front, _tensor(out, "out", (B, n, H * hd), et),
                                         _tensor(lse, "lse", (B, n, H), torch.float32), *rest)
        _check(st, "ga_prefill_backward_lse")
    return dict(dq=dq, dk=dk, dv=dv, dgate=dgate, dq_norm_w=dwq, dk_norm_w=dwk)


def _decode_args(desc, q, k_cache, v_cache, cache_lens, max_cache_len, et):
    B = desc.batch
    if int(max_cache_len) < 0:
        raise ValueError("max_cache_len must be >= 0")
    kcp, vcp, cap = _cache_pair(k_cache, v_cache, desc, et, int(max_cache_len) + 1)
    return B, kcp, vcp, cap, _lens(cache_lens, "cache_lens", B)


def ga_decode(desc: AttnDesc, q, k_new, v_new, k_cache, v_cache, cache_lens, max_cache_len: int, gate=None,
              q_norm_w=None, k_norm_w=None, out=None, workspace=None, stream=None) -> torch.Tensor:
    """out [B,H*d] for one new token per sequence; appends K-hat/V at slot cache_lens[b]."""
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, kcp, vcp, cap, lp = _decode_args(desc, q, k_cache, v_cache, cache_lens, max_cache_len, et)
    G, hd = desc.n_kv_heads, desc.head_dim
    d2, qp, gp = _qg(desc, q, gate, (B,), et)
    if out is None:
        out = torch.empty((B, desc.n_q_heads * hd), dtype=et, device=q.device)
    op = _tensor(out, "out", (B, desc.n_q_heads * hd), et)
    ws, wp, wb = _workspace_arg(workspace, ga_decode_workspace_bytes(desc, max_cache_len), q.device)
    st = lib.ga_decode(ctypes.byref(d2), qp, _tensor(k_new, "k_new", (B, G, hd), et),
                       _tensor(v_new, "v_new", (B, G, hd), et), gp, _norm_w(q_norm_w, "q_norm_w", desc),
                       _norm_w(k_norm_w, "k_norm_w", desc), kcp, vcp, cap, lp, int(max_cache_len), wp, wb, op,
                       _stream(stream))
    _check(st, "ga_decode")
    return out


def ga_decode_partials(desc: AttnDesc, q, k_cache, v_cache, cache_lens, max_cache_len: int, workspace,
                       q_norm_w=None, stream=None) -> torch.Tensor:
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, kcp, vcp, cap, lp = _decode_args(desc, q, k_cache, v_cache, cache_lens, max_cache_len, et)
    d2, qp, _ = _qg(_no_gate(desc), q, None, (B,), et)  # (the partials read no gate)
    ws, wp, wb = _workspace_arg(workspace, ga_decode_workspace_bytes(desc, max_cache_len), q.device)
    st = lib.ga_decode_partials(ctypes.byref(d2), qp, _norm_w(q_norm_w, "q_norm_w", desc), kcp, vcp, cap, lp,
                                int(max_cache_len), wp, wb, _stream(stream))
    _check(st, "ga_decode_partials")
    return ws


def _no_gate(desc: AttnDesc) -> AttnDesc:
    d2 = AttnDesc.from_buffer_copy(desc)
    d2.gate_mode = _lib.GA_GATE_NONE
    d2.gate_share = 0
    return d2


def ga_decode_merge(desc: AttnDesc, q, k_new, v_new, k_cache, v_cache, cache_lens, max_cache_len: int, workspace,
                    gate=None, q_norm_w=None, k_norm_w=None, out=None, stream=None) -> torch.Tensor:
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, kcp, vcp, cap, lp = _decode_args(desc, q, k_cache, v_cache, cache_lens, max_cache_len, et)
    G, hd = desc.n_kv_heads, desc.head_dim
    d2, qp, gp = _qg(desc, q, gate, (B,), et)
    if out is None:
        out = torch.empty((B, desc.n_q_heads * hd), dtype=et, device=q.device)
    op = _tensor(out, "out", (B, desc.n_q_heads * hd), et)
    ws, wp, wb = _workspace_arg(workspace, ga_decode_workspace_bytes(desc, max_cache_len), q.device)
    st = lib.ga_decode_merge(ctypes.byref(d2), qp, _tensor(k_new, "k_new", (B, G, hd), et),
                             _tensor(v_new, "v_new", (B, G, hd), et), gp, _norm_w(q_norm_w, "q_norm_w", desc),
                             _norm_w(k_norm_w, "k_norm_w", desc), kcp, vcp, cap, lp, int(max_cache_len), wp, wb,
                             op, _stream(stream))
    _check(st, "ga_decode_merge")
    return out


def ga_decode_noalloc(desc: AttnDesc, q, k_new, v_new, k_cache, v_cache, cache_lens, max_cache_len: int, out,
                      gate=None, q_norm_w=None, k_norm_w=None, stream=None) -> torch.Tensor:
    """ga_decode without a workspace (partials in the library's static device
    scratch; see include/ga.h): allocates nothing, so ``out`` is required."""
    lib = _lib.load()
    et = _elem_dtype(desc)
    B, kcp, vcp, cap, lp = _decode_args(desc, q, k_cache, v_cache, cache_lens, max_cache_len, et)
    G, hd = desc.n_kv_heads, desc.head_dim
    d2, qp, gp = _qg(desc, q, gate, (B,), et)
    op = _tensor(out, "out", (B, desc.n_q_heads * hd), et)
    st = lib.ga_decode_noalloc(ctypes.byref(d2), qp, _tensor(k_new, "k_new", (B, G, hd), et),
                               _tensor(v_new, "v_new", (B, G, hd), et), gp, _norm_w(q_norm_w, "q_norm_w", desc),
                               _norm_w(k_norm_w, "k_norm_w", desc), kcp, vcp, cap, lp, int(max_cache_len), op,
                               _stream(stream))
    _check(st, "ga_decode_noalloc")
    return out
