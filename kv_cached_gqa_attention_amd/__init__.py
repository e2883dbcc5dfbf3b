"""KV-cached grouped-query attention for AMD MI355X (gfx950).

The product is the C-ABI library ``libkvc.so`` (``include/kvc.h``): append of
new K/V rows, split-KV decode and causal verify attention over contiguous or
block-paged caches, and both fused in one call, in hand-written HIP kernels. This package is its Python
binding; PyTorch supplies device memory and streams.
"""

from .api import (
    Cache,
    KvcError,
    append,
    append_attend,
    attend,
    attend_noalloc,
    decode,
    gather,
    plan_kernel,
    status_string,
    verify,
    workspace,
    workspace_bytes,
)

__all__ = [
    "Cache",
    "KvcError",
    "append",
    "append_attend",
    "attend",
    "attend_noalloc",
    "decode",
    "gather",
    "plan_kernel",
    "status_string",
    "verify",
    "workspace",
    "workspace_bytes",
]
