/*
 * kvc.h - attention of a few new query tokens against a growing key/value
 * cache, with grouped-query heads, on AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages this follows):
 *
 *  - "Making inference cheap: KV cache, batching and quantization": keys and
 *    values of earlier positions never change once computed (the causal-mask
 *    paragraph), so they are stored and each generation step attends the new
 *    token's query over every stored key, one 1 x n score row per head.
 *  - "CS336, lectures 10 and 12: inference and evaluation", section
 *    "Arithmetic intensity of inference" (attention layers): A = Q K^T,
 *    Y = softmax(A) V; section "Reducing the KV cache": N query heads share
 *    K key-value heads, each serving a group of G = N / K query heads.
 *  - "Stanford CS336 Day 13 - Inference", "Attention layers": the grouped
 *    shapes, scores B x S x T x K x G against values B x S x K x H.
 *  - "Accelerating Sonar through speculation", section "Speculative
 *    decoding": the target model scores n drafted tokens in one pass, giving
 *    up to n + 1 tokens; the verify call here is that pass's attention, over
 *    T = n + 1 query tokens, causal inside the block.
 *  - "CS336, lectures 10 and 12", section "PagedAttention": the cache of a
 *    sequence is split into fixed-size blocks (e.g. 16 tokens) and a
 *    per-sequence block table maps logical blocks to physical ones; blocks
 *    may be shared between sequences (prefix sharing).
 *  - "Accelerating Sonar through speculation", section "Inference with
 *    speculative decoding": batch metadata is copied to GPU memory before
 *    the model runs, and the accepted length must not force a GPU-to-CPU
 *    synchronisation; hence lengths and block tables are DEVICE arrays here
 *    and no call ever reads them on the host.
 *
 * Definitions used by every call. Sequence b holds seq_lens[b] valid tokens
 * AFTER its T new tokens are appended; P_b = seq_lens[b] - T tokens were
 * cached before. New token t (0 <= t < T) of sequence b is at absolute
 * position P_b + t and attends keys 0 .. P_b + t. Query head n reads
 * key-value head n / G (each key-value head serves a contiguous group).
 *     s_j   = scale * <q, k_j>
 *     out   = sum_j softmax(s)_j * v_j
 *     lse   = ln sum_j exp(s_j)               (natural log)
 * All arithmetic after the 16-bit loads is fp32.
 *
 * Conventions shared by all entry points:
 *  - Pointers are DEVICE pointers unless marked (host).
 *  - Every call enqueues its work on `stream` (a hipStream_t passed as
 *    void *; NULL is the default stream) of the calling thread's current
 *    device and returns without synchronising. Nothing is allocated or
 *    freed; no pointer is kept after the call returns.
 *  - The caller owns every buffer. Host-checkable argument errors return a
 *    non-zero status BEFORE anything is launched, so no partial work happens.
 *  - Device metadata cannot be validated on the host without a sync. A
 *    sequence with seq_lens[b] < T or > capacity gets NaN in every output row
 *    (and its append writes nothing); one whose block-table entries needed
 *    for its tokens lie outside [0, num_blocks) gets NaN in every output row
 *    that reads them: every row, except in query blocks of more than 128
 *    rows per KV head (G * T > 128, chunks of prefill), whose blocks of 128
 *    rows stop reading at their last row's position under the causal rule.
 *    No memory outside the buffers described here is read or written.
 *  - Tensor element types are kvc_dtype; K/V caches and q are f16 or bf16.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID = -1,     /* bad argument (null pointer, shape, range, alignment) */
  KVC_ERR_UNSUPPORTED = -2, /* valid but not implemented (head size, dtype) */
  KVC_ERR_WORKSPACE = -3,   /* workspace missing or smaller than kvc_workspace_bytes() */
  KVC_ERR_HIP = -4          /* the HIP runtime reported an error at launch */
} kvc_status;

typedef enum { KVC_F16 = 0, KVC_BF16 = 1, KVC_F32 = 2 } kvc_dtype;

/* Per-unit counters at the start of every attention workspace (see
 * kvc_attn_decode). */
#define KVC_WORKSPACE_COUNTERS (1 << 18)

/* Largest number of new tokens per sequence in one attention call. */
#define KVC_MAX_T 2048

/* Largest number of new tokens per sequence with a draft-tree mask. */
#define KVC_MAX_TREE_T 256

/*
 * One layer's key cache and value cache (same layout, same dtype).
 *
 * Contiguous (block_table == NULL): element (b, head, token, h) of the key
 * cache is k[b * stride_seq + head * stride_head + token * stride_tok + h];
 * the default layout [B, K, capacity, H] has stride_seq = K * capacity * H,
 * stride_head = capacity * H, stride_tok = H. A whole-model tensor
 * [L, 2, K, C, H] is described per layer by pointer offsets with the same
 * strides.
 *
 * Paged (block_table != NULL): k and v are pools of num_blocks blocks;
 * logical token t of sequence b is stored in physical block
 * p = block_table[b * max_blocks_per_seq + t / block_size] at slot
 * t % block_size, i.e. element (p, head, slot, h) is
 * k[p * stride_seq + head * stride_head + slot * stride_tok + h]; the default
 * pool layout [num_blocks, K, block_size, H] has stride_seq =
 * K * block_size * H, stride_head = block_size * H, stride_tok = H.
 * Entries that no valid token needs are never read (use -1). Several
 * sequences may map to the same physical block (shared prefixes); appends
 * must not target a shared block.
 *
 * Strides are in elements; the head dimension is unit-stride. k, v and every
 * stride times the element size must be multiples of 16 bytes.
 */
typedef struct kvc_cache {
  void *k;                    /* device */
  void *v;                    /* device */
  const int32_t *block_table; /* device [B, max_blocks_per_seq] or NULL */
  int64_t stride_seq;         /* elements between sequences (contiguous) or blocks (paged) */
  int64_t stride_head;        /* elements between key-value heads */
  int64_t stride_tok;         /* elements between tokens (slots) */
  int32_t dtype;              /* kvc_dtype: KVC_F16 or KVC_BF16 */
  int32_t capacity;           /* contiguous: max tokens per sequence; paged: ignored
                                 (capacity is max_blocks_per_seq * block_size) */
  int32_t block_size;         /* paged: tokens per block, a power of two, 1 .. 4096 */
  int32_t max_blocks_per_seq; /* paged: row length of block_table */
  int32_t num_blocks;         /* paged: blocks in each pool */
  int32_t reserved;           /* must be 0 */
} kvc_cache;

/*
 * Append the T new key and value rows of every sequence to its cache.
 * Prior art: the kernel that writes the next target tokens to their
 * positions in "Accelerating Sonar through speculation", section
 * "Single-token MTP schedule".
 *
 * k_new, v_new: [B, T, K, H] contiguous, in cache->dtype. Row t of sequence b
 * is written at logical position seq_lens[b] - T + t. Bytes are copied
 * unchanged (bit-exact). Nothing else in the cache is written.
 * Errors: KVC_ERR_INVALID for null pointers, B < 0, T < 1, K < 1, bad
 * strides or alignment; KVC_ERR_UNSUPPORTED for H not in {64, 128} or a
 * dtype other than f16/bf16. B == 0 succeeds and launches nothing (the
 * row and length pointers may then be NULL).
 */
kvc_status kvc_append(const kvc_cache *cache, const void *k_new, const void *v_new, int B, int T,
                      int K, int H, const int32_t *seq_lens, void *stream);

/*
 * Decode: one new query token per sequence (T = 1). Same as
 * kvc_attn_verify with T = 1.
 *
 * q: [B, N, H] in cache->dtype. out: [B, N, H] in out_dtype (f32, f16 or
 * bf16, 16-byte aligned; 16-bit outputs are rounded to nearest even). lse: [B, N] fp32, or
 * NULL. max_seq_len (host) is an upper bound on seq_lens[] used only to size
 * the launch (a longer device length is still computed correctly, just with
 * fewer workgroups than ideal); it must satisfy 1 <= max_seq_len <= capacity.
 * scale multiplies q.k (1/sqrt(H) is the usual choice).
 * num_workgroups: how many workgroups share the work (0 = automatic); the
 * result is the same function for every value, up to fp32 rounding order.
 * workspace: device scratch of at least kvc_workspace_bytes(B, 1, N, K, H,
 * max_seq_len, num_workgroups) bytes, 16-byte aligned. Its first
 * KVC_WORKSPACE_COUNTERS * 4 bytes hold per-unit counters: they must be zero
 * when the buffer is first used, and every call that completes leaves them
 * zero again, so one buffer may serve later calls of any shape on the same
 * stream (the rest is scratch that each call writes before reading). Calls
 * that overlap in time must not share a workspace.
 * Errors: as kvc_append, plus KVC_ERR_INVALID for N < 1, N % K != 0,
 * max_seq_len out of range; KVC_ERR_UNSUPPORTED for B > 4096 or more than
 * KVC_WORKSPACE_COUNTERS units (B * K * row blocks, a row block holding up to
 * 64 of the G * T query rows of a (b, k), 128 when there are more than 64);
 * KVC_ERR_WORKSPACE
 * for a missing, misaligned or small workspace.
 */
kvc_status kvc_attn_decode(const kvc_cache *cache, const void *q, void *out, int out_dtype,
                           float *lse, int B, int N, int K, int H, const int32_t *seq_lens,
                           int max_seq_len, float scale, int num_workgroups, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Verify: T new query tokens per sequence (1 <= T <= KVC_MAX_T), causal
 * inside the block: token t sees the P_b prior keys and new tokens 0 .. t.
 * A short block (T = n + 1 for n drafted tokens) is the speculative verify
 * pass; a long one is a chunk of prefill against the cache ("CS336, lectures
 * 10 and 12", section on the two stages of inference: prefill runs the
 * prompt through the model in one parallel pass and fills the KV cache; its
 * attention has intensity about S/2, so it is bound by the matrix cores, not
 * by memory). The new rows must already be in the cache (kvc_append, or use
 * kvc_append_attend).
 * q: [B, T, N, H]; out: [B, T, N, H]; lse: [B, T, N] fp32 or NULL.
 * Other arguments and errors as kvc_attn_decode (max_seq_len >= T), plus
 * KVC_ERR_INVALID for T > KVC_MAX_T.
 */
kvc_status kvc_attn_verify(const kvc_cache *cache, const void *q, void *out, int out_dtype,
                           float *lse, int B, int T, int N, int K, int H, const int32_t *seq_lens,
                           int max_seq_len, float scale, int num_workgroups, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Append and attend in one call: the effect of kvc_append(cache, k_new,
 * v_new, B, T, K, H, seq_lens, stream) followed by kvc_attn_verify (T >= 1;
 * T = 1 is decode) with the same arguments, on the same stream. The new rows
 * are written into the cache as by kvc_append, and the attention sees them
 * ("Making inference cheap: KV cache, batching and quantization": each step
 * extends the cache by the new token's rows and attends over the whole
 * cache). It saves the separate append launch: when every (b, k) is served
 * by one row block (G * T <= 128, true for all decode and short verify
 * shapes) the append happens inside the attention kernel, each new row
 * written by the workgroup that later reads it; otherwise the call enqueues
 * the append kernel and then the attention kernel.
 * k_new, v_new: [B, T, K, H] in cache->dtype, 16-byte aligned (not modified).
 * Workspace as kvc_attn_verify, same size. Errors: as kvc_append and
 * kvc_attn_verify together. Outputs for sequences with an invalid length are
 * NaN and their rows are not appended, as with the two separate calls.
 */
kvc_status kvc_append_attend(const kvc_cache *cache, const void *k_new, const void *v_new,
                             const void *q, void *out, int out_dtype, float *lse, int B, int T,
                             int N, int K, int H, const int32_t *seq_lens, int max_seq_len,
                             float scale, int num_workgroups, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Options of kvc_attn. A zeroed struct (or a NULL pointer) gives exactly
 * kvc_attn_verify.
 *
 * window: 0, or W >= 1 for local (sliding-window) attention ("CS336,
 *   lectures 10 and 12", section "Reducing the KV cache": a token looks only
 *   at the most recent tokens; "Stanford CS336 Day 13 - Inference", section
 *   "Local Attention"): new token t, at position i = seq_lens[b] - T + t,
 *   sees only keys at positions i - W + 1 .. i. Only keys at positions
 *   >= seq_lens[b] - T - W + 1 are ever read (at most W + T - 1 positions per
 *   sequence and head), so with a block table the entries of blocks wholly
 *   before that position are not read and those blocks may be unmapped or
 *   reused: the cache a windowed call needs does not grow with the sequence
 *   ("Stanford CS336 Day 13 - Inference", "Local Attention": rows that left
 *   the window can leave the cache). A rolling cache is a cyclic table:
 *   logical block j of a sequence in ring[j mod R], R blocks covering at
 *   least W + T - 1 + 2 * block_size positions, so that the append of the
 *   new rows overwrites only positions the window no longer needs.
 * tree_mask: NULL for the causal rule inside the block, or device
 *   [B, T, TW] uint32 words, TW = (T + 31) / 32, for draft-tree verification
 *   ("Accelerating Sonar through speculation", section "EAGLE": tree-shaped
 *   drafts are verified with custom attention masks): the TW words of (b, t)
 *   are a T-bit row, bit u in word u / 32 at bit u % 32; new token t of
 *   sequence b sees new token u exactly when bit u of its row is set (set
 *   t's own bit and its ancestors'); every prior row stays visible; bits
 *   >= T are ignored. With T <= 32 this is one word per token, [B, T].
 *   4-byte aligned; T <= KVC_MAX_TREE_T. A query that sees no key at all
 *   gets NaN. Both options compose: a key must pass both rules.
 * k_new, v_new: NULL, or the new rows to append first, as kvc_append_attend.
 * reserved: must be 0.
 */
typedef struct {
  const void *k_new;
  const void *v_new;
  const uint32_t *tree_mask;
  int32_t window;
  int32_t reserved;
} kvc_attn_options;

/*
 * Attention of T >= 1 new tokens with options (window, draft-tree mask,
 * fused append): kvc_attn_verify's arguments and rules plus opts (may be
 * NULL). The workspace size from kvc_workspace_bytes for the same B, T, N,
 * K, H, max_seq_len and num_workgroups is always enough (a window only
 * lowers the need). Errors: as kvc_attn_verify and kvc_append_attend, plus
 * KVC_ERR_INVALID for window < 0, reserved != 0, a misaligned tree_mask or a
 * tree_mask with T > KVC_MAX_TREE_T.
 */
kvc_status kvc_attn(const kvc_cache *cache, const kvc_attn_options *opts, const void *q, void *out,
                    int out_dtype, float *lse, int B, int T, int N, int K, int H,
                    const int32_t *seq_lens, int max_seq_len, float scale, int num_workgroups,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Size of the per-device scratch array kvc_attn_noalloc runs in. */
#define KVC_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Exactly
 * kvc_attn (same arguments, options, kernels and results) without the
 * workspace arguments: the counters and partials live in a static device
 * array of KVC_NOALLOC_SCRATCH_BYTES bytes inside the library, one per
 * device, held from this entry point's first call on that device until the
 * process ends. That first call on a device takes the array's address and
 * clears its counter region on `stream`; every completed call leaves the
 * counters zero again. Nothing is allocated or freed, ever; the caller still
 * passes q, out, lse and the cache.
 * All calls on one device share that device's array: calls that overlap in
 * time on one device (different streams, threads) race and give undefined
 * results; serialise them (one stream, or events).
 * Errors: as kvc_attn, plus KVC_ERR_WORKSPACE (before anything is launched)
 * when the call needs more than KVC_NOALLOC_SCRATCH_BYTES, i.e. when
 * kvc_workspace_bytes(B, T, N, K, H, max_seq_len, num_workgroups) exceeds
 * it (e.g. chunks of prefill of 512 tokens for 8 sequences of 8 key-value
 * heads; a smaller num_workgroups lowers the need); KVC_ERR_HIP when the
 * array's address cannot be taken.
 */
kvc_status kvc_attn_noalloc(const kvc_cache *cache, const kvc_attn_options *opts, const void *q,
                            void *out, int out_dtype, float *lse, int B, int T, int N, int K,
                            int H, const int32_t *seq_lens, int max_seq_len, float scale,
                            int num_workgroups, void *stream);

/*
 * Host query: workspace bytes needed by kvc_attn_decode (T = 1) or
 * kvc_attn_verify with the same B, T, N, K, H, max_seq_len and
 * num_workgroups. Returns 0 for invalid shapes. Uses the current device's
 * compute-unit count when a device is present.
 */
size_t kvc_workspace_bytes(int B, int T, int N, int K, int H, int max_seq_len, int num_workgroups);

/*
 * Host query: the name of the attention kernel a kvc_attn_verify call with
 * these arguments (T = 1: kvc_attn_decode) launches, as the plan chooses it:
 * "attn_valu_kernel" (few query rows per (b, k): vector ALUs),
 * "attn_mfma_kernel" (up to 64 rows: matrix cores) or "attn_wide_kernel"
 * (longer query blocks: matrix cores, units of 128 rows). A static string;
 * NULL for invalid shapes. For reports and profiles; nothing is launched.
 */
const char *kvc_plan_kernel(int B, int T, int N, int K, int H, int max_seq_len, int num_workgroups);

/* Host: a static, human-readable name for a status code (any int: values
 * that are not a kvc_status give "unknown kvc_status"). */
const char *kvc_status_string(int status);

/*
 * Test export: copy the first seq_lens[b] logical tokens of every sequence
 * of a PAGED cache into contiguous dst_k, dst_v [B, K, max_seq_len, H]
 * (cache->dtype), bit-exact. Rows at or beyond seq_lens[b] are not written.
 * A sequence with seq_lens[b] > max_seq_len, or a needed block-table entry
 * outside [0, num_blocks), is skipped. Errors as kvc_append.
 */
kvc_status kvc_gather(const kvc_cache *paged, void *dst_k, void *dst_v, int B, int K, int H,
                      const int32_t *seq_lens, int max_seq_len, void *stream);

/*
 * Test export (host only, nothing is launched): the flat step ranges that
 * the attention kernels give their workers, computed by the kernels' own
 * partition code. `total` steps over W workers; fast_workers, xcds,
 * share_fast, share_slow, xcd_even and xcd_odd as a launch plan sets them
 * (fast_workers 0: equal shares; xcds 0: workers in launch order; xcd_even
 * or xcd_odd 0: no XCD factors). Writes lo_hi[2w] and lo_hi[2w + 1], the
 * range [lo, hi) of worker w, for every w < W (caller-owned, 2W entries)
 * and, when owners is not NULL, owners[x] for every x < total (caller-owned,
 * total entries): the worker the kernels take as holding step x when they
 * look up another worker's part of a unit. (The per-wave matrix-core
 * kernel's shares: kvc_partition_ranges_costed.) KVC_ERR_INVALID for total outside
 * [0, 2^32], W outside [1, 2^20], negative fast_workers or xcds, share
 * weights outside [1, 16], XCD factors outside [0, 64], or lo_hi NULL.
 */
kvc_status kvc_partition_ranges(int64_t total, int W, int fast_workers, int xcds, int share_fast,
                                int share_slow, int xcd_even, int xcd_odd, int64_t *lo_hi,
                                int32_t *owners);

/*
 * Test export (host only, nothing is launched): the flat step ranges of the
 * per-wave matrix-core kernel's costed partition, computed by the kernel's
 * own code: equal shares over W workers of the flat steps plus seg_steps
 * virtual steps placed before each unit, each worker's virtual range mapped
 * back to the flat steps it stands for (a unit's virtual steps stand for its
 * first flat step). Units are (b, k, rb) in that order, B sequences, K heads
 * and RB row blocks each; unit (b, k, rb) has unit_steps[b * RB + rb] steps
 * for every k (caller-owned, B * RB entries). Writes lo_hi[2w], lo_hi[2w + 1]
 * for every w < W (caller-owned, 2W entries) and, when owners is not NULL,
 * owners[x] for every flat step x (caller-owned, K times the sum of
 * unit_steps entries): the worker the kernel takes as holding step x.
 * KVC_ERR_INVALID for B outside [1, 2^16], K outside [1, 1024], RB outside
 * [1, 64], a unit_steps entry outside [0, 2^20], more than 2^32 steps, W
 * outside [1, 2^20], seg_steps outside [0, 64], or unit_steps or lo_hi NULL.
 */
kvc_status kvc_partition_ranges_costed(int B, int K, int RB, const int32_t *unit_steps, int W,
                                       int seg_steps, int64_t *lo_hi, int32_t *owners);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
