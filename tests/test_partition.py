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
