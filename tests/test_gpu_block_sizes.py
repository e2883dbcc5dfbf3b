"""GPU parity of the decode and verify kernels on paged caches of every block
size class, against the fp64 oracle.

A K/V tile is 32 token rows; one copy instruction covers 4 rows at head size
128 and 8 rows at head size 64. Blocks of at least 32 rows hold a whole tile
(one table entry per tile), blocks of 4..16 (8..16) rows hold whole
instructions (one entry per instruction), and smaller blocks take one entry
per lane. Each class runs here on the vector-ALU kernel (few query rows:
single-token decode, small verify blocks) and on the matrix-core kernel (the
verify shapes: 40 and 64 rows per (b, k), and a head size of 64), with
automatic and fixed grids, a window, a draft tree, the fused append, a block
entry outside the pool, and bit-equality with the contiguous layout.
"""

import math

import numpy as np
import pytest
import torch

import kv_cached_gqa_attention_amd as kvc
from gpu_cases import Run, all_units, compare_units, run_case, say
from workloads import draw_inputs, layout_paged, make_block_table

pytestmark = pytest.mark.gpu

BF, HF = torch.bfloat16, torch.float16
BLOCK_SIZES = [1, 2, 4, 8, 32, 64, 256]

CASES = [
    # B, T, N, K, H, dtype, prior                     kernel and rows per (b, k)
    (3, 1, 32, 8, 128, BF, [0, 77, 300]),             # vector ALU, 4 rows (batched-decode heads)
    (3, 1, 16, 2, 64, HF, [5, 130, 260]),             # vector ALU, 8 rows at H = 64
    (2, 2, 4, 2, 64, BF, [33, 200]),                  # vector ALU, verify of 2 tokens
    (2, 5, 64, 8, 128, BF, [100, 555]),               # matrix cores, 40 rows (the verify shape)
    (2, 8, 8, 1, 128, BF, [50, 1000]),                # matrix cores, 64 rows
    (2, 4, 16, 4, 64, HF, [33, 129]),                 # matrix cores, 16 rows at H = 64
]


def _ids(cases):
    return [f"B{c[0]}T{c[1]}N{c[2]}K{c[3]}H{c[4]}{'bf' if c[5] is BF else 'hf'}" for c in cases]


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("case", CASES, ids=_ids(CASES))
def test_decode_and_verify_any_block_size(gpu_device, case, bs):
    """Automatic grid (every unit its own worker) and a 5-workgroup grid
    (units split across workgroups at tile boundaries inside blocks)."""
    B, T, N, K, H, dtype, prior = case
    for nwg in (0, 5):
        run = run_case(B, T, N, K, H, dtype, prior, layout="paged", block_size=bs,
                       seed=600 + bs + T, num_workgroups=nwg)
        compare_units(run, all_units(run.inp))


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("T,N,K,H", [(1, 32, 8, 128), (5, 64, 8, 128), (3, 6, 2, 64), (4, 16, 4, 64)])
def test_paged_equals_contiguous_bitwise_any_block_size(gpu_device, T, N, K, H, bs):
    """The block-table gather changes nothing: the same grid on the contiguous
    layout gives bit-equal outputs and LSE."""
    kw = dict(B=4, T=T, N=N, K=K, H=H, dtype=BF, prior=[1, 200, 1500, 64], seed=610,
              num_workgroups=37)
    a = run_case(layout="contiguous", **kw)
    b = run_case(layout="paged", block_size=bs, **kw)
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.lse, b.lse)


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[3], CASES[5]], ids=_ids([CASES[0], CASES[1], CASES[3], CASES[5]]))
def test_window_any_block_size(gpu_device, case, bs):
    """A window of 40 positions: the first visible position falls inside a
    block (or a tile) and reads are clamped there."""
    B, T, N, K, H, dtype, prior = case
    run = run_case(B, T, N, K, H, dtype, prior, layout="paged", block_size=bs, seed=620 + bs,
                   window=40)
    compare_units(run, all_units(run.inp))


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 32, 256])
@pytest.mark.parametrize("T,N,K,H", [(1, 32, 8, 128), (5, 64, 8, 128), (3, 8, 2, 64)])
def test_window_never_reads_blocks_before_it_any_block_size(gpu_device, T, N, K, H, bs):
    """Blocks wholly before the first visible position are unmapped (-1) and
    the pool is NaN wherever they pointed: outputs match the oracle."""
    B, W = 3, 100
    dev = gpu_device
    inp = draw_inputs(B, T, N, K, H, BF, np.array([1000, 77, 513]), 630 + T + bs, device="cpu")
    for name in ("q", "k_new", "v_new", "ctx_k", "ctx_v"):
        setattr(inp, name, getattr(inp, name).to(dev))
    table, nb = make_block_table(631 + bs, inp.seq_lens, bs, extra_blocks=2)
    pk, pv = layout_paged(inp, table, nb, bs, pad_value=float("nan"))
    cut = table.copy()
    for b in range(B):
        first = max(0, int(inp.seq_lens[b]) - T - W + 1)
        for blk in range(first // bs):
            pk[cut[b, blk]] = float("nan")
            pv[cut[b, blk]] = float("nan")
            cut[b, blk] = -1
    cache = kvc.Cache(pk, pv, torch.from_numpy(cut).to(dev))
    seq_lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(dev)
    kvc.append(cache, inp.k_new, inp.v_new, seq_lens)
    L = int(inp.seq_lens.max())
    q = inp.q[:, 0].contiguous() if T == 1 else inp.q
    out, lse = kvc.attend(q, cache, seq_lens, L, window=W, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    if T == 1:
        out, lse = out[:, None], lse[:, None]
    run = Run(inp, cache, seq_lens, out, lse, 1 / math.sqrt(H), window=W)
    compare_units(run, all_units(inp))


@pytest.mark.parametrize("bs", BLOCK_SIZES)
def test_draft_tree_any_block_size(gpu_device, bs):
    from oracle import ancestor_words

    B, T, N, K, H = 3, 6, 64, 8, 128
    rng = np.random.default_rng(640 + bs)
    words = []
    for _ in range(B):
        parents = [-1] + [int(rng.integers(-1, u)) for u in range(1, T)]
        words.append(ancestor_words(parents))
    run = run_case(B, T, N, K, H, BF, [90, 0, 700], layout="paged", block_size=bs, seed=641 + bs,
                   tree=words)
    compare_units(run, all_units(run.inp))


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[5]], ids=_ids([CASES[0], CASES[3], CASES[5]]))
def test_fused_append_attend_any_block_size(gpu_device, case, bs):
    """The fused entry point writes the new rows through the block table
    inside the attention kernel: cache and outputs bit-equal to the two
    separate calls, outputs at the oracle."""
    B, T, N, K, H, dtype, prior = case
    kw = dict(layout="paged", block_size=bs, seed=650 + bs, num_workgroups=0)
    fused = run_case(B, T, N, K, H, dtype, prior, fused=True, **kw)
    compare_units(fused, all_units(fused.inp))
    sep = run_case(B, T, N, K, H, dtype, prior, **kw)
    assert torch.equal(fused.cache.k.view(torch.int16), sep.cache.k.view(torch.int16))
    assert torch.equal(fused.cache.v.view(torch.int16), sep.cache.v.view(torch.int16))
    assert torch.equal(fused.out, sep.out) and torch.equal(fused.lse, sep.lse)


@pytest.mark.parametrize("bs", [1, 2, 4])
@pytest.mark.parametrize("T,N,K,H", [(1, 8, 2, 128), (5, 64, 8, 128), (1, 16, 2, 64), (4, 16, 4, 64)])
def test_out_of_range_entry_small_blocks(gpu_device, T, N, K, H, bs):
    """Blocks smaller than one copy instruction's rows take per-lane table
    entries; one entry outside the pool makes that sequence's rows NaN (output
    and LSE) and leaves the others at the oracle."""
    dev = gpu_device
    B = 3
    inp = draw_inputs(B, T, N, K, H, BF, np.array([40, 40, 40]), seed=660 + bs + T, device=dev)
    table, nb = make_block_table(661, inp.seq_lens, bs)
    pk, pv = layout_paged(inp, table, nb, bs)
    seq_lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(dev)
    cache = kvc.Cache(pk, pv, torch.from_numpy(table).to(dev))
    kvc.append(cache, inp.k_new, inp.v_new, seq_lens)
    bad = table.copy()
    bad[1, 17 // bs] = nb + 1000  # token 17: inside the first tile
    cache_bad = kvc.Cache(pk, pv, torch.from_numpy(bad).to(dev))
    q = inp.q[:, 0].contiguous() if T == 1 else inp.q
    L = int(inp.seq_lens.max())
    out, lse = kvc.attend(q, cache_bad, seq_lens, L, out_dtype=torch.float32, return_lse=True,
                          num_workgroups=3)
    torch.cuda.synchronize()
    if T == 1:
        out, lse = out[:, None], lse[:, None]
    assert torch.isnan(out[1]).all() and torch.isnan(lse[1]).all()
    run = Run(inp, cache_bad, seq_lens, out, lse, 1 / math.sqrt(H))
    say(f"  bad entry at bs={bs}: sequence 1 NaN")
    compare_units(run, [(b, k) for b in (0, 2) for k in range(K)])
