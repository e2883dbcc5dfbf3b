"""The allocation-free entry point (kvc_attn_noalloc) against the workspace
entry point it mirrors (kvc_attn), through the C ABI.

Two calls in a row on the library's per-device static scratch, the second
with a smaller input (fewer sequences, a different kernel): each output and
LSE is bit-equal to kvc_attn's on the same inputs with a caller-allocated
workspace (same kernels, same plan), and matches the oracle within 2e-3.
"""

import math

import numpy as np
import pytest
import torch

import kv_cached_gqa_attention_amd as kvc
from gpu_cases import Run, all_units, build_cache, compare_units, say
from workloads import draw_inputs

pytestmark = pytest.mark.gpu

BF, HF = torch.bfloat16, torch.float16


def _one(dev, B, T, N, K, H, dtype, prior, layout, seed, nwg, window=0, fused=False):
    say(f"noalloc case B={B} T={T} N={N} K={K} H={H} {layout} nwg={nwg} window={window} fused={fused}")
    inp = draw_inputs(B, T, N, K, H, dtype, np.array(prior), seed, device=dev)
    seq_lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(dev)
    L = int(inp.seq_lens.max())
    q = inp.q[:, 0].contiguous() if T == 1 else inp.q
    scale = 1.0 / math.sqrt(H)
    results = []
    for noalloc in (False, True):
        cache, _ = build_cache(inp, layout, seed)
        if not fused:
            kvc.append(cache, inp.k_new, inp.v_new, seq_lens)
        kw = dict(k_new=inp.k_new, v_new=inp.v_new) if fused else {}
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=dev)
        lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        if noalloc:
            kvc.attend_noalloc(q, cache, seq_lens, L, out, lse=lse, window=window, scale=scale,
                               num_workgroups=nwg, **kw)
        else:
            ws = torch.zeros(kvc.workspace_bytes(B, T, N, K, H, L, nwg), dtype=torch.uint8, device=dev)
            o, l = kvc.attend(q, cache, seq_lens, L, window=window, scale=scale, out_dtype=torch.float32,
                              num_workgroups=nwg, return_lse=True, ws=ws, **kw)
            out.copy_(o)
            lse.copy_(l)
        torch.cuda.synchronize()
        results.append((cache, out, lse))
    (c0, o0, l0), (c1, o1, l1) = results
    assert torch.equal(o0, o1), "output differs from the workspace entry point"
    assert torch.equal(l0, l1), "lse differs from the workspace entry point"
    assert torch.equal(c0.k.view(torch.int16), c1.k.view(torch.int16))
    assert torch.equal(c0.v.view(torch.int16), c1.v.view(torch.int16))
    if T == 1:
        o1, l1 = o1[:, None], l1[:, None]
    compare_units(Run(inp, c1, seq_lens, o1, l1, scale, window=window), all_units(inp))


def test_noalloc_two_calls_second_smaller(gpu_device):
    dev = gpu_device
    # a verify block on the matrix cores over a grid that splits units (partials
    # and merges in the scratch), then a smaller decode on the vector ALUs
    _one(dev, 6, 5, 64, 8, 128, BF, [3000, 17, 800, 2047, 5, 1500], "contiguous", 701, nwg=0)
    _one(dev, 3, 1, 32, 8, 128, BF, [700, 65, 2000], "paged", 702, nwg=7)


def test_noalloc_options_and_repeats(gpu_device):
    """Window, fused append, another head size; then the first shape again
    (the counters left by earlier calls are zero)."""
    dev = gpu_device
    _one(dev, 4, 1, 14, 2, 64, HF, [295, 1000, 3, 4000], "contiguous", 703, nwg=5, window=300)
    _one(dev, 2, 3, 16, 4, 128, BF, [100, 900], "paged", 704, nwg=0, fused=True)
    _one(dev, 6, 5, 64, 8, 128, BF, [3000, 17, 800, 2047, 5, 1500], "contiguous", 701, nwg=0)


def test_noalloc_rejects_calls_beyond_the_scratch(gpu_device):
    """A call needing more than the static array fails before any launch and
    leaves the output untouched."""
    dev = gpu_device
    B, T, N, K, H = 8, 512, 32, 8, 128
    need = kvc.workspace_bytes(B, T, N, K, H, T + 16, 0)
    assert need > 64 << 20
    q = torch.zeros((B, T, N, H), dtype=BF, device=dev)
    ck = torch.zeros((B, K, T + 16, H), dtype=BF, device=dev)
    cache = kvc.Cache(ck, ck.clone())
    sl = torch.full((B,), T + 16, dtype=torch.int32, device=dev)
    out = torch.full(q.shape, 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(kvc.KvcError, match="WORKSPACE"):
        kvc.attend_noalloc(q, cache, sl, T + 16, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
