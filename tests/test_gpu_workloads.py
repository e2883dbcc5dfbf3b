"""GPU parity at the workloads' full sizes, in the launch configuration
the bench times (automatic workgroup count). Where the oracle would take too
long on every unit, a seeded sample of (sequence, key-value head) units is
checked; each sampled unit is checked on every query row and every dim.
"""

import math

import numpy as np
import pytest
import torch

import kv_cached_gqa_attention_amd as kvc
from gpu_cases import all_units, compare_units, run_case, say
from oracle import full_recompute
from workloads import WORKLOADS, draw_inputs, draw_prior_lengths, logical_kv

pytestmark = pytest.mark.gpu


def _prior(w):
    return draw_prior_lengths(w.seed, w.B, w.prior_lo, w.prior_hi)


def test_single_layer_against_full_causal_recompute(gpu_device):
    """295 cached tokens + 1 new: the new row equals the last row of the
    uncached, masked n x n recompute (queries of earlier positions are drawn
    too, only the last one is the decode query)."""
    w = WORKLOADS["single_layer_b1_ctx295"]
    run = run_case(w.B, w.T, w.N, w.K, w.H, w.dtype, _prior(w), layout=w.layout, seed=w.seed)
    compare_units(run, all_units(run.inp))
    kb, vb = logical_kv(run.inp, 0)
    L = kb.shape[0]
    g = torch.Generator().manual_seed(w.seed + 99)
    q_all = torch.randn((L, w.N, w.H), generator=g).to(w.dtype)
    q_all[L - 1] = run.inp.q[0, 0].cpu()
    ref, ref_lse = full_recompute(q_all.double().numpy(), kb.double().cpu().numpy(),
                                  vb.double().cpu().numpy(), run.scale)
    got = run.out[0, 0].double().cpu().numpy()
    d = float(np.abs(got - ref[L - 1]).max())
    say(f"  vs full recompute: max|d|={d:.3e}")
    assert d <= 2e-3
    assert float(np.abs(run.lse[0, 0].double().cpu().numpy() - ref_lse[L - 1]).max()) <= 2e-3


@pytest.mark.parametrize("ctx", WORKLOADS["layers24_b1_sweep"].prior_sweep)
def test_layers24_slice_strided_per_layer(gpu_device, ctx):
    """One [L, 2, K, C, H] cache tensor; each layer's K and V are views (pointer
    offsets, shared strides) handed to the library one layer per call."""
    w = WORKLOADS["layers24_b1_sweep"]
    dev = gpu_device
    C = ctx + w.T
    cache = torch.full((w.layers, 2, w.K, C, w.H), float("nan"), dtype=w.dtype, device=dev)
    seq_lens = torch.tensor([ctx + w.T], dtype=torch.int32, device=dev)
    worst = 0.0
    for layer in range(w.layers):
        inp = draw_inputs(1, w.T, w.N, w.K, w.H, w.dtype, np.array([ctx]), w.seed * 1000 + layer,
                          device=dev)
        kc, vc = cache[layer, 0][None], cache[layer, 1][None]
        kc[0, :, :ctx] = inp.ctx_k.permute(1, 0, 2)
        vc[0, :, :ctx] = inp.ctx_v.permute(1, 0, 2)
        c = kvc.Cache(kc, vc)
        kvc.append(c, inp.k_new, inp.v_new, seq_lens)
        out, lse = kvc.decode(inp.q[:, 0].contiguous(), c, seq_lens, C, out_dtype=torch.float32,
                              return_lse=True)
        torch.cuda.synchronize()
        from gpu_cases import Run

        run = Run(inp, c, seq_lens, out[:, None], lse[:, None], 1 / math.sqrt(w.H))
        o, _ = compare_units(run, all_units(inp))
        worst = max(worst, o)
    say(f"  ctx={ctx}: worst over 24 layers {worst:.3e}")


def test_batched_decode_b64_all_units(gpu_device):
    w = WORKLOADS["batched_decode_b64"]
    run = run_case(w.B, w.T, w.N, w.K, w.H, w.dtype, _prior(w), layout=w.layout, seed=w.seed,
                   draw_device=gpu_device)
    compare_units(run, all_units(run.inp))


def test_spec_verify_b32_t5_sampled(gpu_device):
    w = WORKLOADS["spec_verify_b32_t5"]
    run = run_case(w.B, w.T, w.N, w.K, w.H, w.dtype, _prior(w), layout=w.layout, seed=w.seed,
                   draw_device=gpu_device)
    rng = np.random.default_rng(w.seed)
    units = [(int(b), int(rng.integers(0, w.K))) for b in rng.permutation(w.B)[:24]]
    compare_units(run, units)
    assert torch.isfinite(run.out).all()


def test_paged_long_b8_all_units(gpu_device):
    w = WORKLOADS["paged_long_b8"]
    run = run_case(w.B, w.T, w.N, w.K, w.H, w.dtype, _prior(w), layout=w.layout, seed=w.seed,
                   draw_device=gpu_device, block_size=w.block_size)
    compare_units(run, all_units(run.inp))


def test_sliding_window_b32_sampled(gpu_device):
    w = WORKLOADS["sliding_window_b32"]
    run = run_case(w.B, w.T, w.N, w.K, w.H, w.dtype, _prior(w), layout=w.layout, seed=w.seed,
                   draw_device=gpu_device, window=w.window)
    rng = np.random.default_rng(w.seed)
    units = [(int(b), int(rng.integers(0, w.K))) for b in rng.permutation(w.B)[:12]]
    compare_units(run, units)
    assert torch.isfinite(run.out).all()


def test_tree_verify_b32_t8_sampled(gpu_device):
    from workloads import tree_mask_words

    w = WORKLOADS["tree_verify_b32_t8"]
    words = [list(tree_mask_words(w.tree_parents))] * w.B
    run = run_case(w.B, w.T, w.N, w.K, w.H, w.dtype, _prior(w), layout=w.layout, seed=w.seed,
                   draw_device=gpu_device, tree=words)
    rng = np.random.default_rng(w.seed)
    units = [(int(b), int(rng.integers(0, w.K))) for b in rng.permutation(w.B)[:24]]
    compare_units(run, units)
    assert torch.isfinite(run.out).all()


def test_prefill_chunk_b8_t512_sampled(gpu_device):
    w = WORKLOADS["prefill_chunk_b8_t512"]
    run = run_case(w.B, w.T, w.N, w.K, w.H, w.dtype, _prior(w), layout=w.layout, seed=w.seed,
                   draw_device=gpu_device)
    rng = np.random.default_rng(w.seed)
    units = [(int(b), int(rng.integers(0, w.K))) for b in rng.permutation(w.B)[:4]]
    compare_units(run, units)
    assert torch.isfinite(run.out).all()
