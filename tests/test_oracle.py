"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the mistake it is there to catch. No test re-types the
oracle's own formula: expected values are literals from the pages, closed
forms worked by hand, a separate brute-force or full-recompute code path,
or invariants of the definition.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    ancestor_words,
    attend,
    causal_tree_words,
    brute_attend,
    full_recompute,
    kv_cache_bytes,
    merge_partials,
    score_bytes,
    split_attend_row,
    visible_keys,
)
from workloads import draw_inputs, layout_contiguous

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_bytes.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand_problem(rng, B, T, N, K, H, prior):
    q = rng.standard_normal((B, T, N, H))
    ks = [rng.standard_normal((p + T, K, H)) for p in prior]
    vs = [rng.standard_normal((p + T, K, H)) for p in prior]
    return q, ks, vs


# --------------------------------------------------------------------------- bytes


def test_bytes_per_token_golden():
    """Printed bytes/token; catches a missing factor 2 (K and V) or a wrong head count."""
    for row in _golden()["bytes_per_token"]:
        got = kv_cache_bytes(1, row["layers"], row["kv_heads"], row["head_dim"], row["elem_bytes"])
        assert got == row["bytes_per_token"], row["cite"]


def test_allocator_check_on_laid_out_tensors():
    """The page measured 3,624,960 B for 295 tokens on (1, 2, 295, 64) fp16 per-layer tensors.

    Lay the cache out with the harness (one layer: K and V caches of
    [B=1, K=2, 295, 64]) and count the bytes the allocation really holds.
    """
    g = _golden()["allocator_check"]
    inp = draw_inputs(1, 1, 14, 2, 64, torch.float16, np.array([g["tokens"] - 1]), seed=1)
    ck, cv = layout_contiguous(inp)
    assert tuple(ck.shape) == tuple(g["per_layer_shape"])
    per_layer = ck.nbytes + cv.nbytes
    assert per_layer * g["layers"] == g["measured_bytes"], g["cite"]
    assert kv_cache_bytes(g["tokens"], g["layers"], 2, 64, 2) == g["measured_bytes"]
    # The one-tensor-per-model layout [L, 2, K, C, H] holds the same bytes.
    whole = torch.empty((g["layers"], 2, 2, g["tokens"], 64), dtype=torch.float16)
    assert whole.nbytes == g["measured_bytes"]


def test_resident_tokens_golden():
    """Cache size depends only on resident tokens: 768 MiB for each split of 65,536."""
    g = _golden()["resident_tokens"]
    for users, toks in g["splits"]:
        total = users * kv_cache_bytes(toks, g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
        assert total == g["mebibytes"] * 2**20, g["cite"]


def test_llama2_13b_golden():
    g = _golden()["llama2_13b_per_sequence"]
    assert kv_cache_bytes(g["tokens"], g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"]) == g["bytes"]


def test_score_bytes_golden():
    """67 MB vs 16 KB at 4,096 tokens are 4-byte (fp32) scores: n x n vs 1 x n."""
    g = _golden()["score_bytes"]
    n = g["tokens"]
    assert round(score_bytes(n, n) / 1e6) == g["recompute_megabytes_decimal_rounded"]
    assert score_bytes(1, n) == g["cached_kilobytes"] * 1024
    # 2-byte scores would give 34 MB / 8 KB: the printed pair fixes 4 bytes.
    assert round(score_bytes(n, n, 2) / 1e6) != g["recompute_megabytes_decimal_rounded"]


# --------------------------------------------------------------------------- closed forms


def _one(q_rows, keys, values, scale, T=1):
    """Single sequence, single head: q_rows [T, H], keys/values [L, H]."""
    q = np.asarray(q_rows, dtype=np.float64)[None, :, None, :]
    k = np.asarray(keys, dtype=np.float64)[:, None, :]
    v = np.asarray(values, dtype=np.float64)[:, None, :]
    out, lse = attend(q, [k], [v], scale)
    return out[0, :, 0, :], lse[0, :, 0]


def test_two_keys_closed_form_scale_one():
    """Scores ln3 and 0 give weights 3/4 and 1/4.

    Catches a flipped softmax sign (weights 1/4, 3/4 -> o = [1, 6]),
    swapped operands, and a log base other than e (lse = ln 4).
    """
    out, lse = _one([[math.log(3.0), 0.0]], [[1.0, 0.0], [0.0, 0.0]], [[4.0, 0.0], [0.0, 8.0]], 1.0)
    np.testing.assert_allclose(out[0], [3.0, 2.0], rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(4.0)) < 1e-14


def test_two_keys_closed_form_scale_half():
    """scale = 1/2 turns the score ln3 into ln sqrt3; catches a dropped or squared scale."""
    r3 = math.sqrt(3.0)
    out, lse = _one([[math.log(3.0), 0.0]], [[1.0, 0.0], [0.0, 0.0]], [[4.0, 0.0], [0.0, 8.0]], 0.5)
    np.testing.assert_allclose(out[0], [4 * r3 / (1 + r3), 8 / (1 + r3)], rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(1 + r3)) < 1e-14


def test_single_visible_key_returns_its_value():
    """Empty prior context, T = 1: the token sees only itself. Catches a strict (j < i) mask."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 8))
    v = rng.standard_normal((1, 8))
    q = rng.standard_normal((1, 8))
    out, lse = _one(q, k, v, 0.25)
    assert np.array_equal(out[0], v[0])
    assert abs(lse[0] - 0.25 * float(q[0] @ k[0])) < 1e-14


def test_zero_scale_is_mean_of_visible_rows_per_block_position():
    """scale = 0: every visible key weighs the same, so row t is the mean of rows 0..P+t.

    Catches a wrong visible extent inside a verify block (off-by-one, or all
    block tokens seeing the whole block).
    """
    P, T, H = 5, 4, 3
    values = np.arange((P + T) * H, dtype=np.float64).reshape(P + T, H)
    keys = np.ones((P + T, H))
    out, lse = _one(np.ones((T, H)), keys, values, 0.0, T=T)
    for t in range(T):
        n_vis = P + t + 1
        expect = values[:n_vis].sum(axis=0) / n_vis
        np.testing.assert_allclose(out[t], expect, rtol=0, atol=1e-12)
        assert abs(lse[t] - math.log(n_vis)) < 1e-14


def test_identical_keys_give_the_mean():
    rng = np.random.default_rng(4)
    keys = np.tile(rng.standard_normal((1, 6)), (7, 1))
    values = rng.standard_normal((7, 6))
    out, _ = _one(rng.standard_normal((1, 6)), keys, values, 0.4)
    np.testing.assert_allclose(out[0], values.mean(axis=0), rtol=0, atol=1e-13)


def test_dominant_key_and_large_scores_stay_finite():
    """One score 60 above the rest returns that key's value within e^-60; scores near
    +-1000 must not overflow (catches a missing max subtraction)."""
    H = 4
    values = np.array([[1.0, 2, 3, 4], [5, 6, 7, 8], [-1, -2, -3, -4]])
    keys = np.array([[0.0, 0, 0, 0], [60.0, 0, 0, 0], [0.0, 0, 0, 0]])
    out, _ = _one([[1.0, 0, 0, 0]], keys, values, 1.0)
    np.testing.assert_allclose(out[0], values[1], rtol=0, atol=10 * math.exp(-60) * 10)
    keys_big = keys * (1000.0 / 60.0)
    out, lse = _one([[1.0, 0, 0, 0]], keys_big, values, 1.0)
    assert np.all(np.isfinite(out)) and math.isfinite(lse[0])
    np.testing.assert_allclose(out[0], values[1], rtol=0, atol=1e-12)
    assert abs(lse[0] - 1000.0) < 1e-9
    del H


def test_head_mapping_groups_are_contiguous():
    """K = 2, G = 3: query heads 0..2 read KV head 0 and 3..5 read KV head 1.

    Catches an interleaved mapping (k = n % K).
    """
    P, T, N, K, H = 4, 1, 6, 2, 3
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, T, N, H))
    k = rng.standard_normal((P + T, K, H))
    v = np.empty((P + T, K, H))
    v[:, 0, :] = 1.0
    v[:, 1, :] = 2.0
    out, _ = attend(q, [k], [v], 0.3)
    np.testing.assert_allclose(out[0, 0, :3], 1.0, atol=1e-14)
    np.testing.assert_allclose(out[0, 0, 3:], 2.0, atol=1e-14)


def test_mqa_heads_with_equal_queries_agree():
    """K = 1: every head reads the same cache; equal queries give equal outputs."""
    rng = np.random.default_rng(6)
    N, H, P = 5, 8, 9
    qrow = rng.standard_normal(H)
    q = np.tile(qrow, (1, 1, N, 1))
    k = rng.standard_normal((P + 1, 1, H))
    v = rng.standard_normal((P + 1, 1, H))
    out, lse = attend(q, [k], [v], 0.35)
    for n in range(1, N):
        assert np.array_equal(out[0, 0, n], out[0, 0, 0])
        assert lse[0, 0, n] == lse[0, 0, 0]


def test_mha_equals_independent_heads():
    """G = 1: head n with KV head n is one independent single-head problem."""
    rng = np.random.default_rng(7)
    B, T, N, H = 2, 2, 3, 5
    prior = [3, 6]
    q, ks, vs = _rand_problem(rng, B, T, N, N, H, prior)
    out, lse = attend(q, ks, vs, 0.5)
    for n in range(N):
        o1, l1 = attend(q[:, :, n : n + 1, :], [k[:, n : n + 1] for k in ks], [v[:, n : n + 1] for v in vs], 0.5)
        np.testing.assert_allclose(out[:, :, n : n + 1], o1, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[:, :, n : n + 1], l1, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------- cached == recompute


@pytest.mark.parametrize("T", [1, 3, 5, 20, 37])
@pytest.mark.parametrize("N,K", [(6, 2), (4, 4), (4, 1)])
def test_cached_equals_full_causal_recompute(T, N, K):
    """Caching is exact: the last T rows of the uncached, masked n x n recompute
    equal the cached oracle over the first L - T rows plus the T new ones
    (T = 20: a chunk of prefill against a 17-row prefix; T = L: the whole
    prompt against an empty cache)."""
    rng = np.random.default_rng(100 + 10 * T + N + K)
    L, H = 37, 16
    q_all = rng.standard_normal((L, N, H))
    k_all = rng.standard_normal((L, K, H))
    v_all = rng.standard_normal((L, K, H))
    full_o, full_l = full_recompute(q_all, k_all, v_all, 1 / math.sqrt(H))
    out, lse = attend(q_all[None, L - T :], [k_all], [v_all], 1 / math.sqrt(H))
    np.testing.assert_allclose(out[0], full_o[L - T :], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], full_l[L - T :], rtol=0, atol=1e-12)


def test_verify_row_ignores_later_block_rows():
    """Changing block rows after t leaves row t unchanged (causal inside the block)."""
    rng = np.random.default_rng(8)
    P, T, N, K, H = 6, 4, 4, 2, 8
    q, ks, vs = _rand_problem(rng, 1, T, N, K, H, [P])
    out, _ = attend(q, ks, vs, 0.3)
    k2, v2 = ks[0].copy(), vs[0].copy()
    k2[P + 2 :] += 10.0
    v2[P + 2 :] -= 7.0
    out2, _ = attend(q, [k2], [v2], 0.3)
    assert np.array_equal(out2[0, :2], out[0, :2])
    assert not np.allclose(out2[0, 2:], out[0, 2:])


# --------------------------------------------------------------------------- invariants


def test_rows_sum_to_one():
    """sum_j exp(s_j - lse) = 1 for every row, including verify rows of every length."""
    rng = np.random.default_rng(9)
    B, T, N, K, H = 2, 3, 4, 2, 8
    prior = [0, 11]
    q, ks, vs = _rand_problem(rng, B, T, N, K, H, prior)
    scale = 0.2
    _, lse = attend(q, ks, vs, scale)
    G = N // K
    for b in range(B):
        for t in range(T):
            for n in range(N):
                vis = prior[b] + t + 1
                s = scale * (ks[b][:vis, n // G, :] @ q[b, t, n])
                assert abs(math.fsum(np.exp(s - lse[b, t, n])) - 1.0) < 1e-12


def test_brute_force_agrees_on_tiny_shapes():
    rng = np.random.default_rng(10)
    for B, T, N, K, H in [(1, 1, 1, 1, 1), (2, 3, 4, 2, 8), (2, 2, 4, 1, 5), (1, 3, 2, 2, 3)]:
        prior = list(rng.integers(0, 10, size=B))
        q, ks, vs = _rand_problem(rng, B, T, N, K, H, prior)
        out, lse = attend(q, ks, vs, 0.7)
        bo, bl = brute_attend(q.tolist(), [k.tolist() for k in ks], [v.tolist() for v in vs], 0.7)
        np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def test_permutation_of_context_rows_is_irrelevant_for_one_token():
    """T = 1: the same permutation of K and V rows leaves the output unchanged;
    only WHICH rows are visible matters (the paged gather order is free)."""
    rng = np.random.default_rng(11)
    P, N, K, H = 20, 4, 2, 8
    q, ks, vs = _rand_problem(rng, 1, 1, N, K, H, [P])
    perm = rng.permutation(P + 1)
    out, lse = attend(q, ks, vs, 0.3)
    out_p, lse_p = attend(q, [ks[0][perm]], [vs[0][perm]], 0.3)
    np.testing.assert_allclose(out_p, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_p, lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 20])
def test_split_merge_equals_unsplit(nsplit):
    """LSE merge of per-range partials reproduces the unsplit row (ranges may be empty)."""
    rng = np.random.default_rng(12 + nsplit)
    n, H = 50, 16
    q = rng.standard_normal(H)
    keys = rng.standard_normal((n, H)) * 2
    values = rng.standard_normal((n, H))
    cuts = np.sort(rng.integers(0, n + 1, size=nsplit - 1))
    bounds = [0, *cuts.tolist(), n]
    o, l = merge_partials(split_attend_row(q, keys, values, 0.5, bounds))
    full_o, full_l = attend(q[None, None, None, :], [keys[:, None, :]], [values[:, None, :]], 0.5)
    np.testing.assert_allclose(o, full_o[0, 0, 0], rtol=0, atol=1e-12)
    assert abs(l - full_l[0, 0, 0]) < 1e-12


def test_attend_rejects_bad_shapes():
    q = np.zeros((1, 2, 3, 4))
    with pytest.raises(ValueError):
        attend(q, [np.zeros((1, 1, 4))], [np.zeros((1, 1, 4))], 1.0)  # L < T
    with pytest.raises(ValueError):
        attend(q, [np.zeros((4, 2, 4))], [np.zeros((4, 2, 4))], 1.0)  # N % K


# --------------------------------------------------------------------------- masks


def _visibility_pattern(P, T, window=0, words=None):
    """With q = 0 every visible score is equal, so out = mean of the visible
    values; one-hot values (value of key j = e_j) turn the mean into 1/|V| on
    exactly the visible keys. Returns the [T, L] pattern the oracle computed."""
    L = P + T
    q = np.zeros((1, T, 1, L))
    k = np.zeros((L, 1, L))
    v = np.eye(L).reshape(L, 1, L)
    out, _ = attend(q, [k], [v], 1.0, window=window, tree_words=None if words is None else [words])
    return out[0, :, 0, :]


@pytest.mark.parametrize("P,T,W", [(0, 1, 1), (5, 1, 1), (5, 1, 3), (5, 1, 6), (5, 1, 50), (9, 4, 1),
                                   (9, 4, 2), (9, 4, 5), (9, 4, 13), (3, 5, 4), (0, 5, 2)])
def test_window_sees_exactly_the_last_w_positions(P, T, W):
    """Catches an off-by-one at either edge of the window: position i sees
    max(0, i - W + 1) .. i, i.e. min(W, i + 1) keys (worked by hand)."""
    pat = _visibility_pattern(P, T, window=W)
    for t in range(T):
        i = P + t
        lo = max(0, i - W + 1)
        want = np.zeros(P + T)
        want[lo : i + 1] = 1.0 / (i + 1 - lo)
        assert np.allclose(pat[t], want, rtol=0, atol=1e-15), (t, pat[t])


def test_window_one_returns_the_own_value_and_score():
    """W = 1: softmax over one key, so out = v_i exactly and lse = s_ii."""
    rng = np.random.default_rng(3)
    q, ks, vs = _rand_problem(rng, 2, 3, 4, 2, 8, [7, 0])
    out, lse = attend(q, ks, vs, 0.3, window=1)
    for b in range(2):
        P = ks[b].shape[0] - 3
        for t in range(3):
            for n in range(4):
                kv = n // 2
                assert np.array_equal(out[b, t, n], vs[b][P + t, kv])
                assert lse[b, t, n] == pytest.approx(0.3 * float(q[b, t, n] @ ks[b][P + t, kv]), abs=1e-12)


def test_window_not_shorter_than_the_sequence_changes_nothing():
    rng = np.random.default_rng(4)
    q, ks, vs = _rand_problem(rng, 2, 2, 4, 2, 8, [20, 3])
    full = attend(q, ks, vs, 0.25)
    for W in (23, 24, 1000):
        win = attend(q, ks, vs, 0.25, window=W)
        assert np.array_equal(full[0], win[0]) and np.array_equal(full[1], win[1])


def test_ancestor_words_by_hand():
    """A chain gives the causal words; a star sees root and self; a small
    tree (0 -> 1 -> 3, 0 -> 2) written out bit by bit."""
    assert ancestor_words([-1, 0, 1, 2]) == [0b1, 0b11, 0b111, 0b1111] == causal_tree_words(4)
    assert ancestor_words([-1, 0, 0, 0]) == [0b1, 0b11, 0b101, 0b1001]
    assert ancestor_words([-1, 0, 0, 1]) == [0b1, 0b11, 0b101, 0b1011]
    assert ancestor_words([-1, -1]) == [0b1, 0b10]
    with pytest.raises(ValueError):
        ancestor_words([-1, 2, 0])


def test_causal_tree_words_reproduce_the_causal_rule():
    rng = np.random.default_rng(5)
    q, ks, vs = _rand_problem(rng, 2, 5, 6, 3, 8, [9, 0])
    a = attend(q, ks, vs, 0.2)
    b = attend(q, ks, vs, 0.2, tree_words=[causal_tree_words(5)] * 2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_tree_visibility_is_prior_plus_own_branch():
    """Catches a mask applied to the prior rows or read with the wrong bit
    order: the visible set is all P prior keys plus exactly the new keys
    whose bit is set."""
    P, T = 6, 5
    words = ancestor_words([-1, 0, 0, 1, 2])
    pat = _visibility_pattern(P, T, words=words)
    for t in range(T):
        vis = list(range(P)) + [P + u for u in range(T) if (words[t] >> u) & 1]
        want = np.zeros(P + T)
        want[vis] = 1.0 / len(vis)
        assert np.allclose(pat[t], want, rtol=0, atol=1e-15), (t, pat[t])


def test_star_tree_equals_attention_over_a_rebuilt_sequence():
    """Drafts 1..T-1 all children of draft 0: draft t is the causal last
    token of the sequence prior + [draft 0, draft t], built by hand."""
    rng = np.random.default_rng(6)
    P, T, N, K, H = 7, 4, 4, 2, 8
    q, ks, vs = _rand_problem(rng, 1, T, N, K, H, [P])
    out, lse = attend(q, ks, vs, 0.4, tree_words=[ancestor_words([-1] + [0] * (T - 1))])
    for t in range(1, T):
        rows = list(range(P)) + [P, P + t]
        k2, v2 = ks[0][rows], vs[0][rows]
        o2, l2 = attend(q[:, t : t + 1], [k2], [v2], 0.4)
        assert np.allclose(out[0, t], o2[0, 0], rtol=0, atol=1e-13)
        assert np.allclose(lse[0, t], l2[0, 0], rtol=0, atol=1e-13)


def test_window_and_tree_compose():
    """Both rules at once: the intersection of the two visible sets."""
    P, T, W = 6, 4, 3
    words = ancestor_words([-1, 0, 0, 2])
    pat = _visibility_pattern(P, T, window=W, words=words)
    for t in range(T):
        i = P + t
        vis = [j for j in list(range(P)) + [P + u for u in range(T) if (words[t] >> u) & 1] if j > i - W]
        assert list(visible_keys(P, T, t, W, words[t])) == vis
        want = np.zeros(P + T)
        want[vis] = 1.0 / len(vis)
        assert np.allclose(pat[t], want, rtol=0, atol=1e-15)
