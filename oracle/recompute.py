"""Uncached recompute: full causal attention over a whole sequence.

Test infrastructure only (see the package docstring).

This is the slow path that "Making inference cheap: KV cache, batching and
quantization" compares the cache against: every step rebuilds the full
n x n score matrix with the causal mask, then takes a row softmax. The page
states that the cached step computes the same numbers; the tests check the
last T rows of this recompute against ``attend`` (an independent code path:
a materialised masked matrix here, per-row slices there).
"""

from __future__ import annotations

import numpy as np


def full_recompute(q_all: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, scale: float):
    """Causal attention of every position of one sequence.

    q_all [L, N, H], k_all/v_all [L, K, H], float64.
    Returns (out [L, N, H], lse [L, N]).
    """
    q_all = np.asarray(q_all, dtype=np.float64)
    k_all = np.asarray(k_all, dtype=np.float64)
    v_all = np.asarray(v_all, dtype=np.float64)
    L, N, H = q_all.shape
    K = k_all.shape[1]
    G = N // K
    causal = np.tril(np.ones((L, L), dtype=bool))  # row i sees columns 0..i
    out = np.empty((L, N, H))
    lse = np.empty((L, N))
    for n in range(N):
        k = n // G
        a = scale * (q_all[:, n, :] @ k_all[:, k, :].T)      # [L, L] score matrix
        a = np.where(causal, a, -np.inf)
        m = a.max(axis=1, keepdims=True)
        e = np.exp(a - m)
        z = e.sum(axis=1, keepdims=True)
        out[:, n, :] = (e / z) @ v_all[:, k, :]
        lse[:, n] = (m + np.log(z))[:, 0]
    return out, lse
