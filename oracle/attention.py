"""Cached attention of T new query tokens, by definition, in float64.

Test infrastructure only (see the package docstring).

For sequence b with P_b prior cached tokens and T new tokens, the logical
cache after the append holds L_b = P_b + T rows per key-value head. New token
t sits at absolute position i = P_b + t and, by causality, sees keys
0 .. i ("Making inference cheap: KV cache, batching and quantization", the
paragraph on why position 7 never sees position 8; for the verify block the
drafted tokens are scored in one pass, "Accelerating Sonar through
speculation", section "Speculative decoding" — read here as plain causal
order inside the block, draft t seeing drafts 0 .. t).

For query head n the key-value head is k = n // G with G = N / K: each
key-value head serves a contiguous group of G query heads ("CS336, lectures
10 and 12", section "Reducing the KV cache"; the B x S x T x K x G score
shape in "Stanford CS336 Day 13 - Inference", "Attention layers", puts K
outside G).

Scores: s_j = scale * <q, k_j>. The pages write A = Q K^T with no scale
("Arithmetic intensity of inference"); the scale is an explicit argument
here (callers default to 1/sqrt(H)), and scale = 1 is the pages' literal
product.

Softmax and output: m = max_j s_j, Z = sum_j exp(s_j - m),
o = sum_j exp(s_j - m) / Z * v_j, lse = m + ln Z (natural log), the sums
running over the visible keys (oracle.masks: causal by default, optionally a
sliding window or a draft-tree mask among the new tokens).
"""

from __future__ import annotations

import numpy as np

from .masks import visible_keys


def attend_one_row(q_vec: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Softmax attention of one query over visible rows.

    q_vec [H], keys [n, H], values [n, H], all float64, n >= 1.
    Returns (o [H], lse).
    """
    s = scale * (keys @ q_vec)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    o = (e / z) @ values
    return o, m + np.log(z)


def attend(q: np.ndarray, k_seqs, v_seqs, scale: float, window: int = 0, tree_words=None):
    """Cached attention for a batch.

    q: float64 [B, T, N, H].
    k_seqs, v_seqs: length-B sequences of float64 [L_b, K, H], the logical
    cache of each sequence after the T new rows were appended (prior rows
    first, then the T new rows).
    window: 0, or the sliding-window length (see oracle.masks).
    tree_words: None (causal inside the block), or per sequence a length-T
    list of mask words (see oracle.masks).
    Returns (out float64 [B, T, N, H], lse float64 [B, T, N]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, T, N, H = q.shape
    out = np.empty((B, T, N, H), dtype=np.float64)
    lse = np.empty((B, T, N), dtype=np.float64)
    for b in range(B):
        kb = np.asarray(k_seqs[b], dtype=np.float64)
        vb = np.asarray(v_seqs[b], dtype=np.float64)
        L, K, Hk = kb.shape
        if Hk != H or vb.shape != kb.shape:
            raise ValueError("key/value shapes do not match the query")
        if N % K:
            raise ValueError("query heads must be a multiple of key-value heads")
        if L < T:
            raise ValueError("a sequence must hold at least its T new rows")
        G = N // K
        P = L - T
        for t in range(T):
            word = None if tree_words is None else int(tree_words[b][t])
            vis = visible_keys(P, T, t, window, word)
            for n in range(N):
                k = n // G
                o, l = attend_one_row(q[b, t, n], kb[vis, k, :], vb[vis, k, :], scale)
                out[b, t, n] = o
                lse[b, t, n] = l
    return out, lse
