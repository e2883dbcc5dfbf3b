"""Shared helpers of the GPU parity tests: draw a case, run the library on it,
and compute the oracle for chosen (sequence, key-value head) units.

The oracle receives the logical per-sequence arrays drawn by ``workloads``
(prior rows ++ new rows), never anything the GPU wrote.
"""

from __future__ import annotations

import math
import sys
from dataclasses import dataclass

import numpy as np
import torch

import kv_cached_gqa_attention_amd as kvc
from oracle import attend
from workloads import draw_inputs, layout_contiguous, layout_paged, logical_kv, make_block_table

TOL = 2e-3  # max |delta| for fp32 outputs and the LSE


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@dataclass
class Run:
    inp: object
    cache: kvc.Cache
    seq_lens: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor | None
    scale: float
    table: np.ndarray | None = None
    window: int = 0
    tree: list | None = None  # per sequence, T mask words


def build_cache(inp, layout, seed, block_size=16, extra_blocks=3, capacity=None, pad=float("nan")):
    dev = inp.device
    if layout == "contiguous":
        ck, cv = layout_contiguous(inp, capacity=capacity, pad_value=pad)
        return kvc.Cache(ck, cv), None
    table, nb = make_block_table(seed + 7, inp.seq_lens, block_size, extra_blocks=extra_blocks)
    pk, pv = layout_paged(inp, table, nb, block_size, pad_value=pad)
    return kvc.Cache(pk, pv, torch.from_numpy(table).to(dev)), table


def run_case(B, T, N, K, H, dtype, prior, layout="contiguous", seed=1, num_workgroups=0,
             out_dtype=torch.float32, block_size=16, scale=None, device="cuda", draw_device="cpu",
             capacity=None, fused=False, window=0, tree=None):
    """Build the cache from the prior rows, then append the new rows and attend:
    two calls (append, then decode/verify) or, with ``fused``, one
    append_attend call."""
    prior = np.asarray(prior, dtype=np.int64)
    say(f"case B={B} T={T} N={N} K={K} H={H} {dtype} {layout} prior[max]={int(prior.max(initial=0))} "
        f"seed={seed} wg={num_workgroups}")
    inp = draw_inputs(B, T, N, K, H, dtype, prior, seed, device=draw_device)
    if draw_device != device:
        inp = to_device(inp, device)
    cache, table = build_cache(inp, layout, seed, block_size=block_size, capacity=capacity)
    seq_lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(device)
    max_len = int(inp.seq_lens.max())
    scale = 1.0 / math.sqrt(H) if scale is None else scale
    if window or tree is not None:
        q = inp.q[:, 0].contiguous() if T == 1 else inp.q
        tm = None
        if tree is not None:
            tm = torch.from_numpy(pack_tree_rows(tree, T)).to(device)
        kw = dict(k_new=inp.k_new, v_new=inp.v_new) if fused else {}
        if not fused:
            kvc.append(cache, inp.k_new, inp.v_new, seq_lens)
        out, lse = kvc.attend(q, cache, seq_lens, max_len, window=window, tree_mask=tm, scale=scale,
                              out_dtype=out_dtype, num_workgroups=num_workgroups, return_lse=True,
                              **kw)
        if T == 1:
            out, lse = out[:, None], lse[:, None]
        torch.cuda.synchronize()
        return Run(inp, cache, seq_lens, out, lse, scale, table, window, tree)
    if fused:
        q = inp.q[:, 0].contiguous() if T == 1 else inp.q
        out, lse = kvc.append_attend(q, inp.k_new, inp.v_new, cache, seq_lens, max_len, scale=scale,
                                     out_dtype=out_dtype, num_workgroups=num_workgroups,
                                     return_lse=True)
        if T == 1:
            out, lse = out[:, None], lse[:, None]
        torch.cuda.synchronize()
        return Run(inp, cache, seq_lens, out, lse, scale, table)
    kvc.append(cache, inp.k_new, inp.v_new, seq_lens)
    if T == 1:
        out, lse = kvc.decode(inp.q[:, 0].contiguous(), cache, seq_lens, max_len, scale=scale,
                              out_dtype=out_dtype, num_workgroups=num_workgroups, return_lse=True)
        out = out[:, None]
        lse = lse[:, None]
    else:
        out, lse = kvc.verify(inp.q, cache, seq_lens, max_len, scale=scale, out_dtype=out_dtype,
                              num_workgroups=num_workgroups, return_lse=True)
    torch.cuda.synchronize()
    return Run(inp, cache, seq_lens, out, lse, scale, table)


def pack_tree_rows(tree, T):
    """Per sequence T mask rows given as Python ints (bit u = sees new token
    u) -> int32 [B, T, (T + 31) // 32], bit u in word u // 32."""
    tw = (T + 31) // 32
    rows = np.zeros((len(tree), T, tw), dtype=np.uint32)
    for b, words in enumerate(tree):
        for t, m in enumerate(words):
            for w in range(tw):
                rows[b, t, w] = (int(m) >> (32 * w)) & 0xFFFFFFFF
    return rows.view(np.int32)


def to_device(inp, device):
    import copy

    out = copy.copy(inp)
    for name in ("q", "k_new", "v_new", "ctx_k", "ctx_v"):
        setattr(out, name, getattr(inp, name).to(device))
    return out


def oracle_unit(inp, b, k, scale, window=0, tree=None, kv=None):
    """Oracle output [T, G, H] and lse [T, G] of sequence b, key-value head k
    (optionally with a window and the sequence's tree words; ``kv``: the
    sequence's logical K and V when already gathered)."""
    G = inp.N // inp.K
    kb, vb = logical_kv(inp, b) if kv is None else kv
    kk = kb[:, k : k + 1, :].double().cpu().numpy()
    vv = vb[:, k : k + 1, :].double().cpu().numpy()
    q = inp.q[b : b + 1, :, k * G : (k + 1) * G, :].double().cpu().numpy()
    o, l = attend(q, [kk], [vv], scale, window=window,
                  tree_words=None if tree is None else [tree[b]])
    return o[0], l[0]


def compare_units(run, units, out_tol=TOL, lse_tol=TOL):
    """Max |delta| of out (fp32 mode) and lse over the given units."""
    inp = run.inp
    G = inp.N // inp.K
    worst_o = worst_l = 0.0
    kv_b, kv = None, None
    for b, k in sorted(units):
        if b != kv_b:  # gather each sequence's logical rows once
            kv_b, kv = b, logical_kv(inp, b)
        o_ref, l_ref = oracle_unit(inp, b, k, run.scale, run.window, run.tree, kv=kv)
        o = run.out[b, :, k * G : (k + 1) * G, :].double().cpu().numpy()
        l = run.lse[b, :, k * G : (k + 1) * G].double().cpu().numpy()
        assert np.all(np.isfinite(o)), f"non-finite output in unit {(b, k)}"
        worst_o = max(worst_o, float(np.abs(o - o_ref).max()))
        worst_l = max(worst_l, float(np.abs(l - l_ref).max()))
    say(f"  max|dout|={worst_o:.3e} max|dlse|={worst_l:.3e} over {len(units)} units")
    assert worst_o <= out_tol, worst_o
    assert worst_l <= lse_tol, worst_l
    return worst_o, worst_l


def all_units(inp):
    return [(b, k) for b in range(inp.B) for k in range(inp.K)]
