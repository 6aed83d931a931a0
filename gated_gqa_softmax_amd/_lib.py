"""ctypes loader for libga.so and the C declarations of include/ga.h.

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in the package.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libga.so")

GA_OK = 0
GA_ERR_NULL_ARG = 1
GA_ERR_BAD_SHAPE = 2
GA_ERR_BAD_DTYPE = 3
GA_ERR_UNSUPPORTED = 4
GA_ERR_MISALIGNED = 5
GA_ERR_WORKSPACE = 6
GA_ERR_HIP = 7

GA_BF16 = 0
GA_F32 = 1
GA_GATE_NONE = 0
GA_GATE_HEADWISE = 1
GA_GATE_ELEMENTWISE = 2
GA_ACT_SIGMOID, GA_ACT_NS_SIGMOID, GA_ACT_SILU, GA_ACT_IDENTITY = 0, 1, 2, 3
GA_COMBINE_MUL, GA_COMBINE_ADD = 0, 1
GA_SHARE_HEADS, GA_SHARE_TOKENS = 1, 2
GA_KERNEL_AUTO, GA_KERNEL_WIDE, GA_KERNEL_MIRROR, GA_KERNEL_SIMPLE, GA_KERNEL_GENERIC = 0, 1, 2, 3, 4
GA_BWD_AUTO, GA_BWD_PLAIN = 0, 1
GA_NOALLOC_SCRATCH_BYTES = 48 * 1024 * 1024


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rot_dim", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("gate_mode", ctypes.c_int32),
        ("q_head_stride", ctypes.c_int32),
        ("gate_head_stride", ctypes.c_int32),
        ("gate_act", ctypes.c_int32),
        ("gate_combine", ctypes.c_int32),
        ("gate_share", ctypes.c_int32),
        ("out_norm_eps", ctypes.c_float),
        ("out_norm_w", ctypes.c_void_p),
        ("kernel", ctypes.c_int32),
        ("bwd_kernel", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_D = ctypes.POINTER(AttnDesc)

SIGNATURES = {
    "ga_prefill_workspace_bytes": (_S, [_D, _I]),
    "ga_prefill_attention_kernel": (ctypes.c_char_p, [_D, _I]),
    "ga_prefill": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _S, _P, _P]),
    "ga_prefill_keys": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _I, _P]),
    "ga_prefill_attention": (_I, [_D, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P, _P, _P]),
    "ga_prefill_chunk": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _P, _S, _P, _P]),
    "ga_prefill_chunk_workspace_bytes": (_S, [_D, _I, _I, _I]),
    "ga_prefill_chunk_keys": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _P]),
    "ga_prefill_chunk_attention": (_I, [_D, _I, _P, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P, _S, _P, _P]),
    "ga_prefill_chunk_kernel": (ctypes.c_char_p, [_D, _I, _I]),
    "ga_prefill_backward_workspace_bytes": (_S, [_D, _I]),
    "ga_prefill_backward": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "ga_prefill_lse_workspace_bytes": (_S, [_D, _I]),
    "ga_prefill_lse": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P, _P, _P]),
    "ga_prefill_backward_lse": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _S, _P]),
    "ga_decode_split_keys": (_I, []),
    "ga_decode_workspace_bytes": (_S, [_D, _I]),
    "ga_decode": (_I, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _S, _P, _P]),
    "ga_decode_noalloc": (_I, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _P]),
    "ga_decode_partials": (_I, [_D, _P, _P, _P, _P, _I, _P, _I, _P, _S, _P]),
    "ga_decode_merge": (_I, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _S, _P, _P]),
    "ga_status_string": (ctypes.c_char_p, [_I]),
    "ga_last_error": (ctypes.c_char_p, []),
    "ga_fast_path": (_I, [_I, _I, _I, _I]),
    "ga_version": (_I, []),
}

_lock = threading.Lock()
_lib = None


class LibraryNotBuilt(RuntimeError):
    pass


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libga.so once and attach the declared signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise LibraryNotBuilt(
                f"{path} not found: build it with `python -m gated_gqa_softmax_amd.build` "
                "(the package has no non-HIP implementation)")
        # The library links libamdhip64; when the process also uses PyTorch,
        # let torch load its HIP runtime first so that one runtime serves both.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib
