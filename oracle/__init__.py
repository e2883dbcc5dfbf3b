"""CPU oracle for KV-cached grouped-query attention.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and
the bench's CPU-baseline leg may import this package. The library path never
calls it, and it imports nothing from the library or its binding.

Everything here is the plain definition, in float64, written from these pages:

* "CS336, lectures 10 and 12: inference and evaluation" (Russian translation),
  section "Arithmetic intensity of inference" / attention layers:
  A = Q K^T, Y = softmax(A) V; section "Reducing the KV cache": N query heads
  share K key-value heads in groups of N/K.
* "Stanford CS336 Day 13 - Inference", section "Arithmetic Intensity of
  Inference" / "Attention layers": the same product with the grouped shapes
  (B x S x T x K x G scores against B x S x K x H values).
* "Making inference cheap: KV cache, batching and quantization": the causal
  mask makes cached keys and values exact (the paragraph on position 7 and
  position 8); a cached step builds one 1 x n score row instead of the n x n
  matrix; the bytes-per-token formula checked against the allocator.

* "CS336, lectures 10 and 12", section "Reducing the KV cache", and
  "Stanford CS336 Day 13 - Inference", section "Local Attention": local
  attention looks at the most recent k tokens only.
* "Accelerating Sonar through speculation", section "EAGLE": draft trees are
  verified with custom attention masks among the new tokens.

Readings where the pages are silent (the softmax scale, the head mapping,
the mask inside a verify block, the window's edge, the tree mask's form,
natural-log LSE) are stated where they are used.

Pins: every function here is checked by ``tests/test_oracle.py`` against
closed forms, brute force, the full causal recompute and the byte counts
the pages print (fixtures in ``tests/golden/``). No function is unpinned.
"""

from .attention import attend, attend_one_row
from .brute import brute_attend
from .cache_bytes import kv_cache_bytes, score_bytes
from .masks import ancestor_words, causal_tree_words, visible_keys
from .recompute import full_recompute
from .split_merge import merge_partials, split_attend_row

__all__ = [
    "ancestor_words",
    "causal_tree_words",
    "visible_keys",
    "attend",
    "attend_one_row",
    "brute_attend",
    "full_recompute",
    "kv_cache_bytes",
    "score_bytes",
    "merge_partials",
    "split_attend_row",
]
