"""Torch-facing binding of the C ABI: same operations, argument marshalling only.

Tensors must live on the GPU; every call enqueues on torch's current stream
of the tensors' device and returns without synchronising. Nothing here
computes attention: each function checks shapes, builds the ``kvc_cache``
descriptor and calls the library.
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib

_DT = {torch.float16: _lib.KVC_F16, torch.bfloat16: _lib.KVC_BF16, torch.float32: _lib.KVC_F32}


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.load().kvc_status_string(status).decode()
        super().__init__(f"{where}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != _lib.KVC_OK:
        raise KvcError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _gpu(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


@dataclass
class Cache:
    """One layer's K and V cache: contiguous ``[B, K, capacity, H]``-style
    (any strides, head dim unit-stride) or paged pools ``[num_blocks, K,
    block_size, H]`` with an int32 ``block_table [B, max_blocks]``."""

    k: torch.Tensor
    v: torch.Tensor
    block_table: torch.Tensor | None = None

    def __post_init__(self):
        _gpu(self.k, "k")
        _gpu(self.v, "v")
        if self.k.dim() != 4 or self.k.shape != self.v.shape or self.k.stride() != self.v.stride():
            raise ValueError("k and v must be 4-D with the same shape and strides")
        if self.k.dtype != self.v.dtype or self.k.dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("k and v must both be float16 or both bfloat16")
        if self.k.stride(3) != 1:
            raise ValueError("the head dimension must be unit-stride")
        if self.block_table is not None:
            _gpu(self.block_table, "block_table")
            if self.block_table.dtype != torch.int32 or self.block_table.dim() != 2:
                raise ValueError("block_table must be int32 [B, max_blocks]")
            if not self.block_table.is_contiguous():
                raise ValueError("block_table must be contiguous")

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def head_dim(self) -> int:
        return self.k.shape[3]

    @property
    def capacity(self) -> int:
        if self.paged:
            return self.block_table.shape[1] * self.k.shape[2]
        return self.k.shape[2]

    def descriptor(self) -> _lib.KvcCache:
        c = _lib.KvcCache()
        c.k = self.k.data_ptr()
        c.v = self.v.data_ptr()
        s = self.k.stride()
        c.stride_seq, c.stride_head, c.stride_tok = s[0], s[1], s[2]
        c.dtype = _DT[self.k.dtype]
        if self.paged:
            c.block_table = self.block_table.data_ptr()
            c.capacity = 0
            c.block_size = self.k.shape[2]
            c.max_blocks_per_seq = self.block_table.shape[1]
            c.num_blocks = self.k.shape[0]
        else:
            c.block_table = None
            c.capacity = self.k.shape[2]
        c.reserved = 0
        return c


def status_string(status: int) -> str:
    return _lib.load().kvc_status_string(status).decode()


def workspace_bytes(B, T, N, K, H, max_seq_len, num_workgroups=0) -> int:
    return int(_lib.load().kvc_workspace_bytes(B, T, N, K, H, max_seq_len, num_workgroups))


def plan_kernel(B, T, N, K, H, max_seq_len, num_workgroups=0) -> str | None:
    """Name of the attention kernel the library's plan picks for this shape."""
    r = _lib.load().kvc_plan_kernel(B, T, N, K, H, max_seq_len, num_workgroups)
    return None if r is None else r.decode()


_ws_cache: dict = {}
# Buffers replaced by a larger one stay referenced until the process ends: a
# call still queued on the GPU (or a graph captured with an explicit buffer
# taken from here) may point at them, so they are never handed back to the
# allocator.
_ws_retired: list = []


def workspace(device, nbytes: int, stream=None) -> torch.Tensor:
    """A zero-filled workspace of at least ``nbytes``, reused per (device,
    stream).

    The library leaves the counter region zero after every call, so one
    buffer serves every call on one stream; calls on different streams may
    overlap in time and get different buffers. During stream capture there
    is no implicit workspace: pass one explicitly, so the captured graph
    owns memory that outlives it.
    """
    device = torch.device(device)
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("kvc: pass an explicit workspace (ws=...) when capturing a graph")
    if stream is None:
        stream = torch.cuda.current_stream(device)
    key = (device.type, device.index, stream.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _ws_retired.append(buf)
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def append(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, seq_lens: torch.Tensor):
    """Write ``k_new``/``v_new`` [B, T, K, H] at positions seq_lens[b] - T + t."""
    _check_new_rows(cache, k_new, v_new, seq_lens)
    B, T, K, H = k_new.shape
    desc = cache.descriptor()
    st = _lib.load().kvc_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), B, T, K, H,
                                _ptr(seq_lens), _stream(k_new.device))
    _check(st, "kvc_append")


def _check_new_rows(cache, k_new, v_new, seq_lens):
    _gpu(k_new, "k_new")
    _gpu(v_new, "v_new")
    _gpu(seq_lens, "seq_lens")
    if k_new.shape != v_new.shape or k_new.dim() != 4:
        raise ValueError("k_new and v_new must be [B, T, K, H]")
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("k_new and v_new must be contiguous")
    if k_new.dtype != cache.k.dtype or v_new.dtype != cache.k.dtype:
        raise ValueError("new rows must have the cache dtype")
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")


def _attn(q, cache, seq_lens, max_seq_len, scale, out_dtype, num_workgroups, return_lse, out, ws, T,
          new_rows=None, opts=None):
    _gpu(q, "q")
    _gpu(seq_lens, "seq_lens")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if q.dtype != cache.k.dtype:
        raise ValueError("q must have the cache dtype")
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    B, N, H = q.shape[0], q.shape[-2], q.shape[-1]
    K = cache.num_kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(H)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous with q's shape and out_dtype")
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device) if return_lse else None
    need = workspace_bytes(B, T, N, K, H, max_seq_len, num_workgroups)
    if ws is None:
        ws = workspace(q.device, need)
    desc = cache.descriptor()
    lib = _lib.load()
    common = (_ptr(seq_lens), int(max_seq_len), float(scale), int(num_workgroups), _ptr(ws),
              ws.numel() * ws.element_size(), _stream(q.device))
    if opts is not None:
        st = lib.kvc_attn(ctypes.byref(desc), ctypes.byref(opts), _ptr(q), _ptr(out), _DT[out_dtype],
                          _ptr(lse), B, T, N, K, H, *common)
        where = "kvc_attn"
    elif new_rows is not None:
        k_new, v_new = new_rows
        st = lib.kvc_append_attend(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                   _DT[out_dtype], _ptr(lse), B, T, N, K, H, *common)
        where = "kvc_append_attend"
    elif T == 1 and q.dim() == 3:
        st = lib.kvc_attn_decode(ctypes.byref(desc), _ptr(q), _ptr(out), _DT[out_dtype], _ptr(lse),
                                 B, N, K, H, *common)
        where = "kvc_attn_decode"
    else:
        st = lib.kvc_attn_verify(ctypes.byref(desc), _ptr(q), _ptr(out), _DT[out_dtype], _ptr(lse),
                                 B, T, N, K, H, *common)
        where = "kvc_attn_verify"
    _check(st, where)
    return (out, lse) if return_lse else out


def decode(q, cache: Cache, seq_lens, max_seq_len, scale=None, out_dtype=None, num_workgroups=0,
           return_lse=False, out=None, ws=None):
    """One new token per sequence: q [B, N, H] -> out [B, N, H] (and lse [B, N])."""
    if q.dim() != 3:
        raise ValueError("decode takes q [B, N, H]")
    return _attn(q, cache, seq_lens, max_seq_len, scale, out_dtype, num_workgroups, return_lse, out,
                 ws, 1)


def verify(q, cache: Cache, seq_lens, max_seq_len, scale=None, out_dtype=None, num_workgroups=0,
           return_lse=False, out=None, ws=None):
    """T new tokens per sequence, causal inside the block: q [B, T, N, H]."""
    if q.dim() != 4:
        raise ValueError("verify takes q [B, T, N, H]")
    return _attn(q, cache, seq_lens, max_seq_len, scale, out_dtype, num_workgroups, return_lse, out,
                 ws, q.shape[1])


def append_attend(q, k_new, v_new, cache: Cache, seq_lens, max_seq_len, scale=None, out_dtype=None,
                  num_workgroups=0, return_lse=False, out=None, ws=None):
    """``append`` then ``decode`` (q [B, N, H]) or ``verify`` (q [B, T, N, H]) in one call.

    k_new, v_new: [B, T, K, H]. Same results as the two calls.
    """
    if q.dim() not in (3, 4):
        raise ValueError("append_attend takes q [B, N, H] or [B, T, N, H]")
    _check_new_rows(cache, k_new, v_new, seq_lens)
    T = 1 if q.dim() == 3 else q.shape[1]
    if k_new.shape[0] != q.shape[0] or k_new.shape[1] != T:
        raise ValueError("k_new must be [B, T, K, H] for q's B and T")
    return _attn(q, cache, seq_lens, max_seq_len, scale, out_dtype, num_workgroups, return_lse, out,
                 ws, T, new_rows=(k_new, v_new))


def attend(q, cache: Cache, seq_lens, max_seq_len, window=0, tree_mask=None, k_new=None, v_new=None,
           scale=None, out_dtype=None, num_workgroups=0, return_lse=False, out=None, ws=None):
    """Attention of the new tokens with options: ``kvc_attn``.

    q: [B, N, H] (one new token) or [B, T, N, H]. window: 0 or the number of
    most recent positions each new token sees (itself included). tree_mask:
    None (causal inside the block) or int32 [B, T, (T + 31) // 32] mask
    rows ([B, T] for T <= 32): bit u of row (b, t), in word u // 32, set =
    new token t sees new token u. k_new, v_new: optional rows to append
    first ([B, T, K, H]).
    """
    if q.dim() not in (3, 4):
        raise ValueError("attend takes q [B, N, H] or [B, T, N, H]")
    T = 1 if q.dim() == 3 else q.shape[1]
    opts = _lib.KvcAttnOptions()
    opts.window = int(window)
    if tree_mask is not None:
        _check_tree_mask(tree_mask, q.shape[0], T)
        opts.tree_mask = _ptr(tree_mask)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _check_new_rows(cache, k_new, v_new, seq_lens)
        if k_new.shape[0] != q.shape[0] or k_new.shape[1] != T:
            raise ValueError("k_new must be [B, T, K, H] for q's B and T")
        opts.k_new = _ptr(k_new)
        opts.v_new = _ptr(v_new)
    return _attn(q, cache, seq_lens, max_seq_len, scale, out_dtype, num_workgroups, return_lse, out,
                 ws, T, opts=opts)


def attend_noalloc(q, cache: Cache, seq_lens, max_seq_len, out, lse=None, window=0, tree_mask=None,
                   k_new=None, v_new=None, scale=None, num_workgroups=0):
    """``attend`` without any allocation: ``kvc_attn_noalloc``.

    The caller passes ``out`` (q's shape; fp32, fp16 or bf16) and optionally
    ``lse`` (fp32, q's shape without the head dim); the counters and partials
    live in the library's per-device static scratch, so calls that overlap in
    time on one device must not be issued (they share it). Nothing here
    allocates device memory.
    """
    if q.dim() not in (3, 4):
        raise ValueError("attend_noalloc takes q [B, N, H] or [B, T, N, H]")
    _gpu(q, "q")
    _gpu(seq_lens, "seq_lens")
    _gpu(out, "out")
    if not q.is_contiguous() or q.dtype != cache.k.dtype:
        raise ValueError("q must be contiguous with the cache dtype")
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    if out.shape != q.shape or not out.is_contiguous() or out.dtype not in _DT:
        raise ValueError("out must be contiguous with q's shape (fp32, fp16 or bf16)")
    if lse is not None:
        _gpu(lse, "lse")
        if lse.shape != q.shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be contiguous fp32 with q's shape minus the head dim")
    T = 1 if q.dim() == 3 else q.shape[1]
    B, N, H = q.shape[0], q.shape[-2], q.shape[-1]
    opts = _lib.KvcAttnOptions()
    opts.window = int(window)
    if tree_mask is not None:
        _check_tree_mask(tree_mask, B, T)
        opts.tree_mask = _ptr(tree_mask)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _check_new_rows(cache, k_new, v_new, seq_lens)
        if k_new.shape[0] != B or k_new.shape[1] != T:
            raise ValueError("k_new must be [B, T, K, H] for q's B and T")
        opts.k_new = _ptr(k_new)
        opts.v_new = _ptr(v_new)
    if scale is None:
        scale = 1.0 / math.sqrt(H)
    desc = cache.descriptor()
    st = _lib.load().kvc_attn_noalloc(ctypes.byref(desc), ctypes.byref(opts), _ptr(q), _ptr(out),
                                      _DT[out.dtype], _ptr(lse), B, T, N, cache.num_kv_heads, H,
                                      _ptr(seq_lens), int(max_seq_len), float(scale),
                                      int(num_workgroups), _stream(q.device))
    _check(st, "kvc_attn_noalloc")
    return out


def _check_tree_mask(tree_mask, B, T):
    """int32 [B, T, (T + 31) // 32] mask rows (bit u of a row in word u // 32),
    or [B, T] when one word per token suffices (T <= 32)."""
    _gpu(tree_mask, "tree_mask")
    tw = (T + 31) // 32
    shapes = {(B, T, tw)} | ({(B, T)} if tw == 1 else set())
    if tree_mask.dtype != torch.int32 or tuple(tree_mask.shape) not in shapes:
        raise ValueError(f"tree_mask must be int32 [B, T, {tw}]" + (" or [B, T]" if tw == 1 else ""))
    if not tree_mask.is_contiguous():
        raise ValueError("tree_mask must be contiguous")


def gather(cache: Cache, seq_lens, max_seq_len):
    """Paged cache -> contiguous (k, v) [B, K, max_seq_len, H]; rows past seq_lens[b] are zero."""
    if not cache.paged:
        raise ValueError("gather needs a paged cache")
    _gpu(seq_lens, "seq_lens")
    B = cache.block_table.shape[0]
    K, H = cache.num_kv_heads, cache.head_dim
    dk = torch.zeros((B, K, max_seq_len, H), dtype=cache.k.dtype, device=cache.k.device)
    dv = torch.zeros_like(dk)
    desc = cache.descriptor()
    st = _lib.load().kvc_gather(ctypes.byref(desc), _ptr(dk), _ptr(dv), B, K, H, _ptr(seq_lens),
                                int(max_seq_len), _stream(dk.device))
    _check(st, "kvc_gather")
    return dk, dv
