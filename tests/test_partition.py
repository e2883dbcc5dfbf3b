"""The workers' step ranges of the attention kernels, through the host-side
test export of the kernels' own partition code (no GPU).

What is checked here is the plain definition of the split: the ranges are
contiguous, cover every flat step once, every worker with work gets at
least one step, each worker's size is its weight's share of the steps to
within one step, and the owner lookup the kernels use to find another
worker's part of a unit names the worker whose range holds the step.
Weights: the older workgroup of a CU's pair (the first half of the grid in
launch order, the first half of each XCD's block in XCD order) against the
younger one, times a factor for the parity of the XCD the worker runs on
(workgroup i runs on XCD i mod xcds).
"""

import ctypes

import numpy as np
import pytest

from kv_cached_gqa_attention_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def ranges(lib, total, W, fast=0, xcds=0, wf=5, ws=4, xe=0, xo=0):
    lo_hi = np.zeros(2 * W, dtype=np.int64)
    owners = np.full(max(total, 1), -1, dtype=np.int32)
    st = lib.kvc_partition_ranges(total, W, fast, xcds, wf, ws, xe, xo,
                                  lo_hi.ctypes.data_as(ctypes.c_void_p),
                                  owners.ctypes.data_as(ctypes.c_void_p))
    assert st == 0
    return lo_hi.reshape(W, 2), owners[:total]


def expected_weights(total, W, fast, xcds, wf, ws, xe, xo):
    """Each worker's weight from the definition above (None: equal shares)."""
    w_eff = min(total, W)
    if not (0 < fast < w_eff and total >= 2 * w_eff):
        return np.ones(w_eff)
    if xcds > 0:
        if not (w_eff == W and W == 2 * fast and fast % xcds == 0):
            return np.ones(w_eff)
        per = W // xcds
        older = np.array([(w % per) < per // 2 for w in range(W)])
        parity = np.array([(w // per) % 2 for w in range(W)])
    else:
        older = np.arange(W) < fast
        parity = np.arange(W) % 2
    base = np.where(older, wf, ws).astype(float)
    if xe > 0 and xo > 0 and (xcds > 0 or fast % 2 == 0):
        base *= np.where(parity == 1, xo, xe)
    if total * base.min() < base.sum():  # some worker's share below one step
        return np.ones(w_eff)
    return base[:w_eff]


def check(lib, total, W, fast=0, xcds=0, wf=5, ws=4, xe=0, xo=0):
    r, owners = ranges(lib, total, W, fast, xcds, wf, ws, xe, xo)
    w_eff = min(total, W)
    lo, hi = r[:, 0], r[:, 1]
    if total == 0:
        assert (lo == 0).all() and (hi == 0).all()
        return r
    assert lo[0] == 0 and hi[w_eff - 1] == total
    assert (hi[: w_eff - 1] == lo[1:w_eff]).all()
    assert (hi[:w_eff] > lo[:w_eff]).all(), "a worker with work got no step"
    assert (lo[w_eff:] == 0).all() and (hi[w_eff:] == 0).all()
    want = expected_weights(total, W, fast, xcds, wf, ws, xe, xo)
    exact = total * want / want.sum()
    size = (hi - lo)[:w_eff]
    assert (np.abs(size - exact) < 1 + 1e-9).all(), np.abs(size - exact).max()
    holder = np.repeat(np.arange(w_eff), size)
    assert (owners == holder).all()
    return r


@pytest.mark.parametrize("total", [0, 1, 7, 100, 8543])
@pytest.mark.parametrize("W", [1, 3, 8, 512])
def test_equal_shares(lib, total, W):
    check(lib, total, W)


# launch order: the first `fast` workgroups are the older of their CU
@pytest.mark.parametrize("total", [1024, 1500, 8543, 100003])
@pytest.mark.parametrize("W,fast", [(512, 256), (16, 8), (8, 4)])
@pytest.mark.parametrize("xe,xo", [(0, 0), (16, 15), (14, 13), (1, 3)])
def test_launch_order_weighted(lib, total, W, fast, xe, xo):
    check(lib, total, W, fast, 0, 5, 4, xe, xo)


# XCD order: the first half of each XCD's block is the older
@pytest.mark.parametrize("total", [1024, 4099, 8543, 100003])
@pytest.mark.parametrize("W,fast,xcds", [(512, 256, 8), (16, 8, 8), (64, 32, 8), (48, 24, 4)])
@pytest.mark.parametrize("xe,xo", [(0, 0), (16, 15), (2, 5)])
def test_xcd_order_weighted(lib, total, W, fast, xcds, xe, xo):
    check(lib, total, W, fast, xcds, 6, 5, xe, xo)


def test_weighting_off_where_it_would_not_fit(lib):
    # fewer steps than two per worker: equal shares
    r = check(lib, 900, 512, 256, 0, 5, 4, 16, 15)
    assert set((r[:, 1] - r[:, 0]).tolist()) <= {1, 2}
    # fewer steps than workers: one step each for the first `total`
    r = check(lib, 300, 512, 256, 0, 5, 4, 16, 15)
    assert (r[:300, 1] - r[:300, 0] == 1).all()
    # XCD order with a grid that is not two full halves: equal shares
    check(lib, 8543, 500, 256, 8, 6, 5, 16, 15)
    # an odd number of fast workers in launch order: no XCD factors
    check(lib, 8543, 510, 255, 0, 5, 4, 16, 15)


def test_shares_follow_the_weights(lib):
    # the batched-decode grid: 512 workgroups, 5 : 4 by age, 16 : 15 by XCD parity
    r, _ = ranges(lib, 100000, 512, 256, 0, 5, 4, 16, 15)
    size = r[:, 1] - r[:, 0]
    older_even = size[0:256:2].mean()
    older_odd = size[1:256:2].mean()
    younger_even = size[256::2].mean()
    assert abs(older_even / younger_even - 5 / 4) < 0.01
    assert abs(older_odd / older_even - 15 / 16) < 0.01


@pytest.mark.parametrize("bad", [
    dict(total=-1), dict(W=0), dict(W=(1 << 20) + 1), dict(fast=-1), dict(xcds=-1),
    dict(wf=0), dict(ws=17), dict(xe=-1), dict(xo=65), dict(total=(1 << 32) + 1),
])
def test_rejects_bad_arguments(lib, bad):
    a = dict(total=10, W=4, fast=0, xcds=0, wf=5, ws=4, xe=0, xo=0)
    a.update(bad)
    buf = np.zeros(2 * max(a["W"], 1), dtype=np.int64)
    st = lib.kvc_partition_ranges(a["total"], a["W"], a["fast"], a["xcds"], a["wf"], a["ws"], a["xe"], a["xo"],
                                  buf.ctypes.data_as(ctypes.c_void_p), None)
    assert st == -1  # KVC_ERR_INVALID
    assert lib.kvc_partition_ranges(10, 4, 0, 0, 5, 4, 0, 0, None, None) == -1


# ---- the per-wave matrix-core kernel's costed shares
#
# Definition: lay the steps out unit by unit ((b, k, rb) in that order), each
# unit's steps preceded by c virtual steps that stand for its first step;
# split that list into equal shares (worker w: entries [n w / W', n (w+1) / W')
# of n = len, W' = min(W, n)); a worker's range is [the flat step its first
# entry stands for, the one its end entry stands for), the end of the list
# standing for the last step + 1. Brute force below, on small inputs.

def costed(lib, unit_steps, K, W, c):
    B, RB = unit_steps.shape
    total = int(unit_steps.sum()) * K
    us = np.ascontiguousarray(unit_steps, dtype=np.int32)
    lo_hi = np.zeros(2 * W, dtype=np.int64)
    owners = np.full(max(total, 1), -1, dtype=np.int32)
    st = lib.kvc_partition_ranges_costed(B, K, RB, us.ctypes.data_as(ctypes.c_void_p), W, c,
                                         lo_hi.ctypes.data_as(ctypes.c_void_p),
                                         owners.ctypes.data_as(ctypes.c_void_p))
    assert st == 0
    return lo_hi.reshape(W, 2), owners[:total]


def costed_brute(unit_steps, K, W, c):
    B, RB = unit_steps.shape
    stands, real_pos = [], []  # per virtual entry: the flat step it stands for
    flat = 0
    for b in range(B):
        for k in range(K):
            for rb in range(RB):
                n = int(unit_steps[b, rb])
                stands += [flat] * c
                for i in range(n):
                    real_pos.append(len(stands))
                    stands.append(flat + i)
                flat += n
    total, nv = flat, len(stands)
    w_eff = min(W, nv)
    at = lambda v: stands[v] if v < nv else total
    r = np.zeros((W, 2), dtype=np.int64)
    vb = [nv * w // w_eff for w in range(w_eff + 1)] if w_eff else [0]
    for w in range(w_eff):
        r[w] = (at(vb[w]), at(vb[w + 1]))
    owners = np.array([max(w for w in range(w_eff) if vb[w] <= v) for v in real_pos], dtype=np.int32)
    return r, owners


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("c", [0, 1, 3, 6, 9])
def test_costed_shares_match_their_definition(lib, seed, c):
    rng = np.random.default_rng(1000 + seed)
    B, K, RB = int(rng.integers(1, 7)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
    unit_steps = rng.integers(0, 6, size=(B, RB))
    if seed % 3 == 0:
        unit_steps[rng.random((B, RB)) < 0.4] = 0  # empty units (invalid lengths)
    W = int(rng.choice([1, 2, 3, 7, 16, 50, 300]))
    got, own = costed(lib, unit_steps, K, W, c)
    want, want_own = costed_brute(unit_steps, K, W, c)
    assert (got == want).all(), (got.tolist(), want.tolist())
    assert (own == want_own).all()
    # the plain properties: contiguous, covering, owners hold their steps
    total = int(unit_steps.sum()) * K
    nonempty = got[got[:, 1] > got[:, 0]]
    if total:
        assert nonempty[0, 0] == 0 and nonempty[-1, 1] == total
        assert (nonempty[1:, 0] == nonempty[:-1, 1]).all()
        for x in range(total):
            assert got[own[x], 0] <= x < got[own[x], 1]


def test_costed_shares_with_none_are_the_equal_shares(lib):
    unit_steps = np.array([[40, 0], [7, 3], [100, 1]])
    got, own = costed(lib, unit_steps, 3, 16, 0)
    want, want_own = ranges(lib, int(unit_steps.sum()) * 3, 16)
    assert (got == want).all() and (own == want_own).all()


def test_costed_shares_give_fewer_steps_to_ranges_entering_more_units(lib):
    # 64 one-step units then one unit of 448 steps, 16 workers, c = 6: every
    # share is (64 * 7 + 448 + 6) / 16 = 56.4 virtual steps, so a worker over
    # the short units holds ~8 real steps and one inside the long unit ~56
    unit_steps = np.array([[1]] * 64 + [[448]])
    got, _ = costed(lib, unit_steps, 1, 16, 6)
    size = got[:, 1] - got[:, 0]
    assert size.sum() == 512
    assert size[:7].max() <= 9 and size[9:].min() >= 55


@pytest.mark.parametrize("bad", [
    dict(B=0), dict(B=(1 << 16) + 1), dict(K=0), dict(RB=0), dict(RB=65), dict(W=0),
    dict(W=(1 << 20) + 1), dict(c=-1), dict(c=65), dict(steps=-1), dict(steps=(1 << 20) + 1),
])
def test_costed_rejects_bad_arguments(lib, bad):
    a = dict(B=2, K=2, RB=1, W=4, c=3, steps=5)
    a.update(bad)
    us = np.full(max(a["B"], 1) * max(a["RB"], 1), a["steps"], dtype=np.int32)
    buf = np.zeros(2 * max(a["W"], 1), dtype=np.int64)
    st = lib.kvc_partition_ranges_costed(a["B"], a["K"], a["RB"], us.ctypes.data_as(ctypes.c_void_p), a["W"],
                                         a["c"], buf.ctypes.data_as(ctypes.c_void_p), None)
    assert st == -1  # KVC_ERR_INVALID
    assert lib.kvc_partition_ranges_costed(2, 2, 1, None, 4, 3, buf.ctypes.data_as(ctypes.c_void_p), None) == -1
