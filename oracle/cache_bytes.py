"""Byte counts of the KV cache and of attention scores.

Test infrastructure only (see the package docstring).

* Per cached token, every layer keeps one key and one value vector of size
  H for each key-value head: bytes/token = 2 * L * K * H * elem_bytes
  ("Making inference cheap: KV cache, batching and quantization", the
  paragraph with the formula checked against the allocator; "CS336,
  lectures 10 and 12", section "Throughput and latency",
  ``kv_cache_size = S * (K*H) * L * 2 * 2``).
* Scores: a cached step builds one row of n scores per head, recompute builds
  n x n; the page's 67 MB vs 16 KB at 4,096 tokens are 4-byte scores.
"""

from __future__ import annotations


def kv_cache_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes held by the K and V caches of ``tokens`` resident tokens."""
    return 2 * tokens * layers * kv_heads * head_dim * elem_bytes


def score_bytes(rows: int, cols: int, elem_bytes: int = 4) -> int:
    """Bytes of a rows x cols score block."""
    return rows * cols * elem_bytes
