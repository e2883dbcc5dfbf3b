"""ctypes view of ``libkvc.so`` (declared in ``include/kvc.h``).

Loading fails loudly when the library has not been built; there is no other
implementation behind these names.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KVC_LIB names another build of the same library (e.g. the host-sanitized
# libkvc_asan.so for CPU-side checks); it must exist like the default.
LIB_PATH = os.environ.get("KVC_LIB") or os.path.join(HERE, "libkvc.so")

KVC_OK = 0
KVC_ERR_INVALID = -1
KVC_ERR_UNSUPPORTED = -2
KVC_ERR_WORKSPACE = -3
KVC_ERR_HIP = -4

KVC_F16 = 0
KVC_BF16 = 1
KVC_F32 = 2

KVC_MAX_T = 2048  # new tokens per sequence in one attention call (include/kvc.h)
KVC_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static scratch of kvc_attn_noalloc (include/kvc.h)

# Every symbol the header declares, in declaration order.
EXPORTS = (
    "kvc_append",
    "kvc_attn_decode",
    "kvc_attn_verify",
    "kvc_append_attend",
    "kvc_attn",
    "kvc_attn_noalloc",
    "kvc_workspace_bytes",
    "kvc_plan_kernel",
    "kvc_status_string",
    "kvc_gather",
    "kvc_partition_ranges",
    "kvc_partition_ranges_costed",
)


class KvcCache(ctypes.Structure):
    """Mirror of ``struct kvc_cache``."""

    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("stride_seq", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("stride_tok", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class KvcAttnOptions(ctypes.Structure):
    """Mirror of ``kvc_attn_options``."""

    _fields_ = [
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
        ("tree_mask", ctypes.c_void_p),
        ("window", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and return the library with its signatures set."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m kv_cached_gqa_attention_amd.build` "
            "(or __graft_entry__.build())"
        )
    lib = ctypes.CDLL(p)
    c_int, c_float, c_size_t, vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    cache_p = ctypes.POINTER(KvcCache)
    lib.kvc_append.argtypes = [cache_p, vp, vp, c_int, c_int, c_int, c_int, vp, vp]
    lib.kvc_append.restype = c_int
    lib.kvc_attn_decode.argtypes = [cache_p, vp, vp, c_int, vp, c_int, c_int, c_int, c_int, vp,
                                    c_int, c_float, c_int, vp, c_size_t, vp]
    lib.kvc_attn_decode.restype = c_int
    lib.kvc_attn_verify.argtypes = [cache_p, vp, vp, c_int, vp, c_int, c_int, c_int, c_int, c_int,
                                    vp, c_int, c_float, c_int, vp, c_size_t, vp]
    lib.kvc_attn_verify.restype = c_int
    lib.kvc_append_attend.argtypes = [cache_p, vp, vp, vp, vp, c_int, vp, c_int, c_int, c_int,
                                      c_int, c_int, vp, c_int, ctypes.c_float, c_int, vp, c_size_t,
                                      vp]
    lib.kvc_append_attend.restype = c_int
    opts_p = ctypes.POINTER(KvcAttnOptions)
    lib.kvc_attn.argtypes = [cache_p, opts_p, vp, vp, c_int, vp, c_int, c_int, c_int, c_int, c_int,
                             vp, c_int, ctypes.c_float, c_int, vp, c_size_t, vp]
    lib.kvc_attn.restype = c_int
    lib.kvc_attn_noalloc.argtypes = [cache_p, opts_p, vp, vp, c_int, vp, c_int, c_int, c_int, c_int,
                                     c_int, vp, c_int, ctypes.c_float, c_int, vp]
    lib.kvc_attn_noalloc.restype = c_int
    lib.kvc_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int]
    lib.kvc_workspace_bytes.restype = c_size_t
    lib.kvc_plan_kernel.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int]
    lib.kvc_plan_kernel.restype = ctypes.c_char_p
    lib.kvc_status_string.argtypes = [c_int]
    lib.kvc_status_string.restype = ctypes.c_char_p
    lib.kvc_gather.argtypes = [cache_p, vp, vp, c_int, c_int, c_int, vp, c_int, vp]
    lib.kvc_gather.restype = c_int
    lib.kvc_partition_ranges.argtypes = [ctypes.c_int64, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                         vp, vp]
    lib.kvc_partition_ranges.restype = c_int
    lib.kvc_partition_ranges_costed.argtypes = [c_int, c_int, c_int, vp, c_int, c_int, vp, vp]
    lib.kvc_partition_ranges_costed.restype = c_int
    if path is None:
        _lib = lib
    return lib
