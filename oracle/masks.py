"""Which cached keys a new query token sees, in plain index form.

Test infrastructure only (see the package docstring).

Positions: sequence b holds P prior rows 0 .. P - 1 and, after the append,
the T new rows P .. P + T - 1; new token t is at position i = P + t.

* Causal (the default): keys 0 .. i ("Making inference cheap: KV cache,
  batching and quantization", the paragraph on why a position never sees a
  later one).
* Tree verify: the drafts form a tree and each one is verified against its
  own branch only, which needs a custom mask among the new tokens
  ("Accelerating Sonar through speculation", section "EAGLE": tree-shaped
  draft sequences are checked with custom attention masks). Reading: every
  prior row stays visible; among the new rows, query t sees new row u exactly
  when bit u of its mask word is set (the caller sets the bits of t's
  ancestors and of t itself). Lower-triangular words give back the causal
  rule.
* Local (sliding-window) attention: a new token looks only at the most
  recent k tokens ("CS336, lectures 10 and 12", section "Reducing the KV
  cache", local attention; "Stanford CS336 Day 13 - Inference", section
  "Reduce KV Cache Size", "Local Attention": only the past k tokens, so older
  rows can leave the cache). Reading: with window
  W >= 1, key j is visible to position i only if i - W < j, i.e. the W
  positions i - W + 1 .. i, the query's own among them; this applies on top
  of the causal or tree rule. W = 0 means no window.
"""

from __future__ import annotations

import numpy as np


def visible_keys(P: int, T: int, t: int, window: int = 0, tree_word: int | None = None) -> np.ndarray:
    """Sorted indices of the keys that new token t (position P + t) sees."""
    if not (0 <= t < T):
        raise ValueError("t out of range")
    i = P + t
    if tree_word is None:
        keys = list(range(0, i + 1))
    else:
        keys = list(range(0, P)) + [P + u for u in range(T) if (tree_word >> u) & 1]
    if window:
        if window < 1:
            raise ValueError("window must be >= 1 (0 = none)")
        keys = [j for j in keys if j > i - window]
    return np.asarray(keys, dtype=np.int64)


def causal_tree_words(T: int) -> list[int]:
    """Mask words equal to the causal rule: query t sees new rows 0 .. t."""
    return [(1 << (t + 1)) - 1 for t in range(T)]


def ancestor_words(parents) -> list[int]:
    """Mask words of a draft tree: parents[u] is the parent of new token u
    (-1 for a root, else an earlier token); token t sees itself and its
    ancestors."""
    words = []
    for t, p in enumerate(parents):
        if p >= t:
            raise ValueError("a parent must come before its child")
        w = 1 << t
        while p >= 0:
            w |= 1 << p
            p = parents[p]
        words.append(w)
    return words
