"""Host-side checks of the seeded generator and the two cache layouts."""

import numpy as np
import pytest
import torch

from kv_cached_gqa_attention_amd import _lib
from workloads import (
    WORKLOADS,
    draw_inputs,
    draw_prior_lengths,
    layout_contiguous,
    layout_paged,
    logical_kv,
    make_block_table,
)


def test_lengths_deterministic_and_in_range():
    a = draw_prior_lengths(123, 64, 512, 4096)
    b = draw_prior_lengths(123, 64, 512, 4096)
    assert np.array_equal(a, b)
    assert a.min() >= 512 and a.max() <= 4096
    assert not np.array_equal(a, draw_prior_lengths(124, 64, 512, 4096))


def test_draws_deterministic_and_rounded():
    prior = np.array([3, 0, 7])
    x = draw_inputs(3, 2, 4, 2, 8, torch.bfloat16, prior, seed=5)
    y = draw_inputs(3, 2, 4, 2, 8, torch.bfloat16, prior, seed=5)
    for name in ("q", "k_new", "v_new", "ctx_k", "ctx_v"):
        assert torch.equal(getattr(x, name), getattr(y, name))
        assert getattr(x, name).dtype == torch.bfloat16
    assert x.ctx_k.shape == (10, 2, 8)
    assert list(x.ctx_off) == [0, 3, 3, 10]
    # N(0,1): sample moments of a larger draw
    z = draw_inputs(1, 1, 1, 1, 64, torch.float32, np.array([20000]), seed=9).ctx_k.double()
    assert abs(z.mean().item()) < 0.02 and abs(z.std().item() - 1) < 0.02


def test_contiguous_layout_places_prior_rows_and_poisons_padding():
    prior = np.array([2, 5])
    inp = draw_inputs(2, 1, 2, 2, 4, torch.float16, prior, seed=1)
    ck, cv = layout_contiguous(inp, capacity=8)
    assert ck.shape == (2, 2, 8, 4)
    for b in range(2):
        kb, vb = logical_kv(inp, b)
        p = prior[b]
        assert torch.equal(ck[b, :, :p, :].permute(1, 0, 2), kb[:p])
        assert torch.equal(cv[b, :, :p, :].permute(1, 0, 2), vb[:p])
        assert torch.isnan(ck[b, :, p:, :]).all()


def test_block_table_is_a_dealt_permutation():
    seq_lens = np.array([1, 16, 17, 40])
    table, nb = make_block_table(7, seq_lens, 16, extra_blocks=3)
    need = [1, 1, 2, 3]
    assert nb == sum(need) + 3
    used = []
    for b, n in enumerate(need):
        assert (table[b, :n] >= 0).all() and (table[b, n:] == -1).all()
        used += table[b, :n].tolist()
    assert len(set(used)) == len(used) and max(used) < nb


def test_paged_layout_round_trips_through_the_table():
    prior = np.array([0, 15, 16, 33])
    T, bs = 2, 16
    inp = draw_inputs(4, T, 4, 2, 8, torch.bfloat16, prior, seed=3)
    table, nb = make_block_table(11, inp.seq_lens, bs)
    pk, pv = layout_paged(inp, table, nb, bs)
    for b in range(4):
        kb, vb = logical_kv(inp, b)
        for t in range(int(prior[b])):
            blk, slot = table[b, t // bs], t % bs
            assert torch.equal(pk[blk, :, slot, :], kb[t])
            assert torch.equal(pv[blk, :, slot, :], vb[t])
    # exactly the prior rows are written; everything else is NaN
    written = int(prior.sum()) * 2 * 8
    assert int((~torch.isnan(pk)).sum()) == written


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_shapes(name):
    w = WORKLOADS[name]
    assert w.N % w.K == 0 and w.H in (64, 128) and 1 <= w.T <= _lib.KVC_MAX_T
    assert w.dtype in (torch.float16, torch.bfloat16)
    assert w.window >= 0
    if w.tree_parents:
        assert len(w.tree_parents) == w.T and w.tree_parents[0] == -1
        assert all(-1 <= p < u for u, p in enumerate(w.tree_parents))


def test_tree_mask_words_agree_with_the_oracle_reading():
    """The input generator's words and the oracle's are written separately;
    they must agree on chains, stars and the measured tree."""
    from oracle import ancestor_words
    from workloads import tree_mask_words

    for parents in ([-1], [-1, 0, 1, 2], [-1, 0, 0, 0, 0], [-1, 0, 0, 1, 1, 2, 2, 3], [-1, -1, 1, 0],
                    WORKLOADS["tree_verify_b32_t8"].tree_parents):
        assert [int(x) for x in tree_mask_words(list(parents))] == ancestor_words(list(parents))


def test_tree_mask_rows_agree_with_the_oracle_reading_for_long_blocks():
    """Rows of several 32-bit words (T up to 256): bit u of row t, in word
    u // 32, is bit u of the oracle's ancestor mask."""
    from oracle import ancestor_words
    from workloads import tree_mask_rows

    rng = np.random.default_rng(5)
    for T in (1, 31, 32, 33, 64, 100, 256):
        parents = [-1] + [int(rng.integers(-1, u)) for u in range(1, T)]
        rows = tree_mask_rows(parents)
        assert rows.shape == (T, (T + 31) // 32) and rows.dtype == np.uint32
        ref = ancestor_words(parents)
        for t in range(T):
            got = sum(int(rows[t, w]) << (32 * w) for w in range(rows.shape[1]))
            assert got == ref[t], (T, t)
