"""The synthetic workloads, named by what they are.

Shapes follow the pages on KV-cached inference:

* the ~0.5B model measured on "Making inference cheap: KV cache, batching and
  quantization" (24 layers, 14 query heads, 2 key-value heads, head size 64,
  fp16; the allocator check paragraph holds 295 cached tokens; the decode
  paragraph sweeps the cached context);
* the 7B-class shape of the same page (8 key-value heads of size 128) for the
  batched, verify and long-context cases;
* the verify block of "Accelerating Sonar through speculation" (section
  "Speculative decoding": n drafted tokens scored in one target pass) with
  4 drafts, i.e. T = 5 query tokens;
* 16-token blocks and a per-sequence block table from "CS336, lectures 10 and
  12: inference and evaluation", section "PagedAttention";
* local attention with a 4096-token window over long contexts ("CS336,
  lectures 10 and 12", section "Reducing the KV cache", which names Mistral
  7B among the local-attention models; 4096 is Mistral 7B's published
  window, a reading, as the pages give no number);
* a draft tree of 8 tokens verified in one pass ("Accelerating Sonar through
  speculation", section "EAGLE": top-k branches at each node; the shape
  here, a root with two children and two grandchildren each plus one more
  level, is a reading);
* a 512-token chunk of prefill against a cached prefix ("CS336, lectures 10
  and 12", section on the two stages of inference: prefill runs the prompt
  in one parallel pass and fills the cache; chunking a long prompt and the
  512-token chunk are a reading, the pages give no chunk size).

"Context" in each description is the PRIOR cached context P_b; the T new
tokens are appended on top of it, so a sequence attends over P_b + T keys.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

SEED_BASE = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    B: int
    N: int
    K: int
    H: int
    T: int
    dtype: torch.dtype
    prior_lo: int
    prior_hi: int
    layout: str  # "contiguous" or "paged"
    seed: int
    layers: int = 1
    block_size: int = 16
    prior_sweep: tuple = field(default_factory=tuple)
    window: int = 0  # sliding window (0: full context)
    tree_parents: tuple = ()  # draft tree among the T new tokens (empty: causal)

    @property
    def G(self) -> int:
        return self.N // self.K

    @property
    def elem_bytes(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    def dtype_name(self) -> str:
        return {torch.float16: "f16", torch.bfloat16: "bf16"}[self.dtype]


WORKLOADS = {
    "single_layer_b1_ctx295": Workload(
        name="single_layer_b1_ctx295",
        description="one layer, B=1, N=14, K=2, H=64, fp16, 295 cached tokens, T=1",
        B=1, N=14, K=2, H=64, T=1, dtype=torch.float16,
        prior_lo=295, prior_hi=295, layout="contiguous", seed=SEED_BASE + 1,
    ),
    "layers24_b1_sweep": Workload(
        name="layers24_b1_sweep",
        description="24 layers, B=1, N=14, K=2, H=64, fp16, T=1, cached context "
                    "16/64/256/1024/4096, one [L,2,K,C,H] cache tensor",
        B=1, N=14, K=2, H=64, T=1, dtype=torch.float16,
        prior_lo=16, prior_hi=4096, layout="contiguous", seed=SEED_BASE + 2,
        layers=24, prior_sweep=(16, 64, 256, 1024, 4096),
    ),
    "batched_decode_b64": Workload(
        name="batched_decode_b64",
        description="B=64, N=32, K=8, H=128, bf16, T=1, cached context U[512,4096], "
                    "contiguous cache padded to the longest sequence",
        B=64, N=32, K=8, H=128, T=1, dtype=torch.bfloat16,
        prior_lo=512, prior_hi=4096, layout="contiguous", seed=SEED_BASE + 3,
    ),
    "spec_verify_b32_t5": Workload(
        name="spec_verify_b32_t5",
        description="B=32, N=64, K=8, H=128, bf16, T=5 (4 drafts + 1), causal inside "
                    "the block, cached context U[2048,8192], contiguous",
        B=32, N=64, K=8, H=128, T=5, dtype=torch.bfloat16,
        prior_lo=2048, prior_hi=8192, layout="contiguous", seed=SEED_BASE + 4,
    ),
    "paged_long_b8": Workload(
        name="paged_long_b8",
        description="B=8, N=32, K=8, H=128, bf16, T=1, cached context U[32768,131072], "
                    "16-token blocks scattered by a seeded permutation",
        B=8, N=32, K=8, H=128, T=1, dtype=torch.bfloat16,
        prior_lo=32768, prior_hi=131072, layout="paged", seed=SEED_BASE + 5,
    ),
    "sliding_window_b32": Workload(
        name="sliding_window_b32",
        description="B=32, N=32, K=8, H=128, bf16, T=1, cached context U[8192,32768], "
                    "sliding window of 4096 positions, contiguous",
        B=32, N=32, K=8, H=128, T=1, dtype=torch.bfloat16,
        prior_lo=8192, prior_hi=32768, layout="contiguous", seed=SEED_BASE + 6, window=4096,
    ),
    "tree_verify_b32_t8": Workload(
        name="tree_verify_b32_t8",
        description="B=32, N=64, K=8, H=128, bf16, T=8 draft-tree tokens (parents "
                    "-1,0,0,1,1,2,2,3), cached context U[2048,8192], contiguous",
        B=32, N=64, K=8, H=128, T=8, dtype=torch.bfloat16,
        prior_lo=2048, prior_hi=8192, layout="contiguous", seed=SEED_BASE + 7,
        tree_parents=(-1, 0, 0, 1, 1, 2, 2, 3),
    ),
    "prefill_chunk_b8_t512": Workload(
        name="prefill_chunk_b8_t512",
        description="B=8, N=32, K=8, H=128, bf16, T=512 prompt tokens per sequence (a chunk of "
                    "prefill, causal inside the chunk), cached prefix U[1024,4096], contiguous",
        B=8, N=32, K=8, H=128, T=512, dtype=torch.bfloat16,
        prior_lo=1024, prior_hi=4096, layout="contiguous", seed=SEED_BASE + 8,
    ),
}


def get_workload(name: str) -> Workload:
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    return WORKLOADS[name]
