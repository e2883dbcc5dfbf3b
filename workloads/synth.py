"""Seeded input draws and cache layouts.

Nothing here computes attention. The functions draw N(0,1) float32 values,
round them to the storage dtype (round-to-nearest-even, torch's ``.to``), and
place the PRIOR context rows into one of the two cache layouts that the
library reads:

* contiguous: per layer, K and V each ``[B, K, capacity, H]`` with the head
  dimension unit-stride (the per-layer ``(1, 2, 295, 64)`` tensors printed on
  "Making inference cheap: KV cache, batching and quantization" are this
  layout with K and V stacked);
* paged: pools ``[num_blocks, K, block_size, H]`` plus an int32 block table
  ``[B, max_blocks]``; logical token t of sequence b lives in block
  ``table[b, t // block_size]`` at slot ``t % block_size``; unused entries
  are -1 ("CS336, lectures 10 and 12: inference and evaluation", section
  "PagedAttention": fixed-size blocks, logical-to-physical block table).

The T new rows (``k_new``, ``v_new``) are NOT placed into the cache: that is
the library's append step. The logical per-sequence arrays that the oracle
reads are ``prior rows ++ new rows`` taken from the draws themselves.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# Rows drawn per torch.randn call when generating large contexts, to bound the
# float32 staging buffer.
_CHUNK_ELEMS = 1 << 27


def draw_prior_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Prior context lengths P_b ~ U{lo..hi} (inclusive), PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi, endpoint=True, size=B).astype(np.int64)


@dataclass
class Inputs:
    """One batch of draws. All tensors live on ``device``."""

    B: int
    T: int
    N: int
    K: int
    H: int
    dtype: torch.dtype
    prior: np.ndarray          # int64 [B], prior cached tokens P_b
    q: torch.Tensor            # [B, T, N, H]
    k_new: torch.Tensor        # [B, T, K, H]
    v_new: torch.Tensor        # [B, T, K, H]
    ctx_k: torch.Tensor        # [sum_b P_b, K, H], prior rows of all sequences back to back
    ctx_v: torch.Tensor
    ctx_off: np.ndarray        # int64 [B+1], row offsets of each sequence in ctx_k/ctx_v

    @property
    def seq_lens(self) -> np.ndarray:
        """Valid cache length after the T new rows are appended."""
        return self.prior + self.T

    @property
    def device(self) -> torch.device:
        return self.q.device


def _normal(g: torch.Generator, shape, dtype, device) -> torch.Tensor:
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK_ELEMS):
        e = min(n, s + _CHUNK_ELEMS)
        flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def draw_inputs(B, T, N, K, H, dtype, prior, seed, device="cpu") -> Inputs:
    """Draw q, k_new, v_new and the prior context rows, N(0,1) rounded to dtype.

    Draw order from one torch generator seeded with ``seed``: q, k_new,
    v_new, ctx_k, ctx_v.
    """
    prior = np.asarray(prior, dtype=np.int64)
    assert prior.shape == (B,)
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    q = _normal(g, (B, T, N, H), dtype, device)
    k_new = _normal(g, (B, T, K, H), dtype, device)
    v_new = _normal(g, (B, T, K, H), dtype, device)
    total = int(prior.sum())
    ctx_k = _normal(g, (total, K, H), dtype, device)
    ctx_v = _normal(g, (total, K, H), dtype, device)
    off = np.zeros(B + 1, dtype=np.int64)
    off[1:] = np.cumsum(prior)
    return Inputs(B, T, N, K, H, dtype, prior, q, k_new, v_new, ctx_k, ctx_v, off)


def logical_kv(inp: Inputs, b: int):
    """Logical K and V of sequence b after the append: ``[P_b + T, K, H]`` each."""
    s, e = int(inp.ctx_off[b]), int(inp.ctx_off[b + 1])
    kb = torch.cat([inp.ctx_k[s:e], inp.k_new[b]], dim=0)
    vb = torch.cat([inp.ctx_v[s:e], inp.v_new[b]], dim=0)
    return kb, vb


def layout_contiguous(inp: Inputs, capacity: int | None = None, pad_value=float("nan")):
    """Place the prior rows into ``[B, K, capacity, H]`` K and V caches.

    Rows at or beyond P_b are filled with ``pad_value`` (NaN by default, so a
    kernel that reads a row it must not read produces NaN).
    """
    cap = int(capacity) if capacity is not None else int(inp.seq_lens.max(initial=0))
    assert cap >= int(inp.seq_lens.max(initial=0))
    shape = (inp.B, inp.K, cap, inp.H)
    ck = torch.full(shape, pad_value, dtype=inp.dtype, device=inp.device)
    cv = torch.full(shape, pad_value, dtype=inp.dtype, device=inp.device)
    for b in range(inp.B):
        s, e = int(inp.ctx_off[b]), int(inp.ctx_off[b + 1])
        ck[b, :, : e - s, :] = inp.ctx_k[s:e].permute(1, 0, 2)
        cv[b, :, : e - s, :] = inp.ctx_v[s:e].permute(1, 0, 2)
    return ck, cv


def make_block_table(seed: int, seq_lens, block_size: int, extra_blocks: int = 0):
    """Block table for ``seq_lens`` tokens per sequence.

    Sequence b needs ceil(seq_lens[b] / block_size) blocks. The pool holds
    their sum plus ``extra_blocks`` never-referenced blocks; a PCG64(seed)
    permutation of the pool indices is dealt out to the sequences in order.
    Returns ``(table int32 [B, max_blocks], num_blocks)`` with -1 in unused
    entries.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    nblk = (seq_lens + block_size - 1) // block_size
    used = int(nblk.sum())
    num_blocks = used + int(extra_blocks)
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(num_blocks).astype(np.int32)
    max_blocks = max(int(nblk.max(initial=0)), 1)
    table = np.full((len(seq_lens), max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos : pos + n]
        pos += int(n)
    return table, num_blocks


def layout_paged(inp: Inputs, table: np.ndarray, num_blocks: int, block_size: int,
                 pad_value=float("nan")):
    """Place the prior rows into ``[num_blocks, K, block_size, H]`` pools."""
    shape = (num_blocks, inp.K, block_size, inp.H)
    pk = torch.full(shape, pad_value, dtype=inp.dtype, device=inp.device)
    pv = torch.full(shape, pad_value, dtype=inp.dtype, device=inp.device)
    blk_idx, slot_idx = [], []
    for b in range(inp.B):
        t = np.arange(int(inp.prior[b]), dtype=np.int64)
        blk_idx.append(table[b, t // block_size].astype(np.int64))
        slot_idx.append(t % block_size)
    if inp.ctx_k.shape[0]:
        blk = torch.from_numpy(np.concatenate(blk_idx)).to(inp.device)
        slot = torch.from_numpy(np.concatenate(slot_idx)).to(inp.device)
        pk[blk, :, slot, :] = inp.ctx_k
        pv[blk, :, slot, :] = inp.ctx_v
    return pk, pv


def tree_mask_rows(parents) -> np.ndarray:
    """The mask rows of a draft tree as the attention call takes them for any
    T: uint32 [T, (T + 31) // 32], bit u of row t (word u // 32, bit u % 32)
    set when new token u is t itself or one of its ancestors."""
    T = len(parents)
    tw = (T + 31) // 32
    rows = np.zeros((T, tw), dtype=np.uint32)
    for t in range(T):
        u = t
        while u >= 0:
            if parents[u] >= u:
                raise ValueError("a parent must come before its child")
            rows[t, u // 32] |= np.uint32(1 << (u % 32))
            u = parents[u]
    return rows


def tree_mask_words(parents) -> np.ndarray:
    """Mask words describing a draft tree among the T new tokens, as the
    caller hands them to the attention call: word t has bit u set when new
    token u is t itself or one of its ancestors (parents[u] is u's parent, an
    earlier token, or -1 for a root). uint32 [T]."""
    T = len(parents)
    words = np.zeros(T, dtype=np.uint32)
    for t in range(T):
        u = t
        while u >= 0:
            if parents[u] >= u:
                raise ValueError("a parent must come before its child")
            words[t] |= np.uint32(1 << u)
            u = parents[u]
    return words
