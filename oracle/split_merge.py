"""Split-and-merge of one attention row by log-sum-exp.

Test infrastructure only (see the package docstring).

The pages name FlashDecoding ("CS336, lectures 10 and 12", section
"PagedAttention", list of other vLLM optimisations) without its mechanism,
and state that tiled attention computes the same function as the plain one
("Making inference cheap: KV cache, batching and quantization", closing note
on FlashAttention). The plain reading: split the visible keys into disjoint
ranges, attend over each range to get (o_s, lse_s), then

    lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s.

This holds exactly because exp(lse_s) is the range's partition sum
Z_s * e^{m_s}, and o_s is that range's weighted mean. The tests pin
``merge_partials(split_attend_row(...))`` to the unsplit definition.
"""

from __future__ import annotations

import numpy as np

from .attention import attend_one_row


def split_attend_row(q_vec, keys, values, scale, bounds):
    """Attend over each key range [bounds[i], bounds[i+1]) separately.

    Empty ranges are skipped. Returns a list of (o_s, lse_s).
    """
    parts = []
    for s, e in zip(bounds[:-1], bounds[1:]):
        if e > s:
            parts.append(attend_one_row(q_vec, keys[s:e], values[s:e], scale))
    return parts


def merge_partials(parts):
    """Combine (o_s, lse_s) partials into (o, lse)."""
    lses = np.array([l for _, l in parts], dtype=np.float64)
    m = lses.max()
    w = np.exp(lses - m)
    lse = m + np.log(w.sum())
    o = sum(np.exp(l - lse) * o_s for o_s, l in parts)
    return o, lse
