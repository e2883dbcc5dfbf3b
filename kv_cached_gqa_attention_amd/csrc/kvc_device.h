// Device-side building blocks shared by the attention kernels.
//
// Work partition. The independent unit of attention is (sequence b, key-value
// head k, query-row block rb): one unit streams the K and V rows of head k of
// sequence b once and serves all G * T query rows that read them ("Stanford
// CS336 Day 13 - Inference", "Attention layers": scores B x S x T x K x G
// against values B x S x K x H). A unit's keys are cut into 32-token tiles.
// All units' tiles are laid end to end in (b, k, rb, tile) order and every
// workgroup takes an equal contiguous share of that flat range, computed on
// the device from seq_lens (no host read of lengths: "Accelerating Sonar
// through speculation", section "Inference with speculative decoding"). A
// unit streams from its first visible key to the last key any of its rows
// sees: with several row blocks per (b, k), a block of early rows stops
// before the sequence's end (unit_steps).
// The range is counted in steps of WAVES tiles (128 tokens): a workgroup's
// waves take one tile of each step, so they always have equal work; the last
// step of a unit may hold tiles past its end, which are masked.
// A workgroup whose share covers part of a unit writes an online-softmax
// partial (m, l, o) for it; the last workgroup to finish the unit merges the
// partials by log-sum-exp. This is the split-KV idea that "CS336, lectures 10
// and 12", section "PagedAttention", names FlashDecoding; the merge algebra is
// the plain one: with partition sums l_s at maxima m_s,
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s o_s 2^(m_s - M) / L.
// Scores are kept in base 2 (q.k * scale * log2 e) so exp2 is one instruction;
// the natural-log LSE is (M + log2 L) * ln 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int TILE = 32;        // tokens per wave iteration
constexpr int WAVES = 4;        // waves per workgroup
constexpr int THREADS = 64 * WAVES;
constexpr int STEP = TILE * WAVES;  // tokens per partition step (one tile per wave)
constexpr float NEG_BIG = -1.0e30f;  // running max before any visible key; exp2(NEG_BIG - x) == 0
constexpr float LN2 = 0.69314718055994531f;
// The running max is raised only when a tile's max exceeds it by more than
// this (log2 units): weights exp2(s - m) then stay <= 2^8 and accumulators
// stay far inside fp32 range, and most tiles skip the rescale. The result is
// the same function: m is only the reference point of l and o.
constexpr float RESCALE_MARGIN = 8.0f;

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf162_t;

// Everything a kernel needs, passed by value.
struct AttnArgs {
  const char* k;  // byte pointers to the K and V caches (or pools)
  const char* v;
  const int32_t* table;  // paged: [B, max_blocks]; nullptr when contiguous
  int64_t stride_seq;    // BYTES between sequences / blocks
  int64_t stride_head;   // BYTES between key-value heads
  int64_t stride_tok;    // BYTES between tokens / slots
  int32_t capacity;      // largest valid seq_len
  int32_t block_shift;   // paged: log2(block_size)
  int32_t max_blocks;    // paged: block table row length
  int32_t num_blocks;    // paged: pool size in blocks
  const char* q;         // [B, T, N, H] in the cache dtype
  void* out;             // [B, T, N, H] in out_dtype
  float* lse;            // [B, T, N] or nullptr
  const int32_t* seq_lens;
  int32_t B, T, N, K, G;
  int32_t R;     // G * T query rows per (b, k)
  int32_t RB;    // query-row blocks per (b, k)
  int32_t RMAX;  // rows per row block (the last block may be partial)
  int32_t out_dtype;  // 0 f16, 1 bf16, 2 f32
  int32_t W;          // workers sharing the tiles (waves or workgroups, per kernel)
  int32_t fast_workers;  // workers with the larger share (0: equal shares; see Partition)
  int32_t share_fast;    // the larger and the smaller share's weights
  int32_t share_slow;
  int32_t xcd_even;      // share factors of workers on even- and odd-numbered
  int32_t xcd_odd;       // XCDs (0: not weighted; see Partition)
  int32_t xcds;       // > 0: workers numbered XCD by XCD (worker_of); 0: worker = workgroup
  float scale_log2;   // scale * log2(e)
  float* part_o;      // [W + units, RMAX, H], slot = worker + unit
  float* part_ml;     // [W + units, RMAX, 2]
  int32_t* counters;  // [units]
  // Fused append (nullptr otherwise): the T new rows of every (b, k),
  // [B, T, K, H] in the cache dtype, which the kernel writes into the cache
  // before attending (append_owned).
  const char* k_new;
  const char* v_new;
  char* k_store;  // the K and V caches again, writable
  char* v_store;
  // Visibility options (both off by default): a sliding window of `window`
  // positions (0: none), and per (b, t) a mask word over the T new rows
  // (nullptr: causal inside the block). See unit_first_step and key_visible.
  int32_t window;
  const uint32_t* tree;  // [B, T, tree_words]
  int32_t tree_words;    // mask words per new token: (T + 31) / 32
  int32_t seg_steps;     // virtual steps charged per unit entered (see make_partition); 0: none
};

// ---------------------------------------------------------------- dtypes

template <bool BF>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (BF) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  c, false);
  }
}

// Low / high 16-bit element of a packed pair, widened to fp32 (exact).
template <bool BF>
__device__ __forceinline__ float lo_f(uint32_t x) {
  if constexpr (BF) {
    return __uint_as_float(x << 16);
  } else {
    return (float)__builtin_bit_cast(half2_t, x)[0];
  }
}
template <bool BF>
__device__ __forceinline__ float hi_f(uint32_t x) {
  if constexpr (BF) {
    return __uint_as_float(x & 0xffff0000u);
  } else {
    return (float)__builtin_bit_cast(half2_t, x)[1];
  }
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ void store_out(void* out, int64_t idx, int out_dtype, float v) {
  if (out_dtype == 2) {
    static_cast<float*>(out)[idx] = v;
  } else if (out_dtype == 1) {
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
  } else {
    static_cast<uint16_t*>(out)[idx] = f32_to_f16_bits(v);
  }
}

// Two consecutive output elements of one row (idx even) in the output
// dtype, one 4- or 8-byte store.
__device__ __forceinline__ void store_out2(void* out, int64_t idx, int out_dtype, float v0, float v1) {
  if (out_dtype == 2) {
    *reinterpret_cast<float2*>(static_cast<float*>(out) + idx) = make_float2(v0, v1);
  } else if (out_dtype == 1) {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + idx) =
        f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16);
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + idx) =
        f32_to_f16_bits(v0) | ((uint32_t)f32_to_f16_bits(v1) << 16);
  }
}
// Four consecutive output elements of one row (idx: the first, a multiple
// of 4) in the output dtype, one 8- or 16-byte store.
__device__ __forceinline__ void store_out4(void* out, int64_t idx, int out_dtype, float v0, float v1, float v2,
                                           float v3) {
  if (out_dtype == 2) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(v0, v1, v2, v3);
  } else {
    uint32_t w0, w1;
    if (out_dtype == 1) {
      w0 = f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16);
      w1 = f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16);
    } else {
      w0 = f32_to_f16_bits(v0) | ((uint32_t)f32_to_f16_bits(v1) << 16);
      w1 = f32_to_f16_bits(v2) | ((uint32_t)f32_to_f16_bits(v3) << 16);
    }
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = make_uint2(w0, w1);
  }
}

__device__ __forceinline__ uint4 load16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Device-coherent scalar store / load (device-scope relaxed atomics: they
// bypass a stale or dirty copy in this XCD's L2).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two consecutive floats (8-byte aligned) as one device-coherent 8-byte
// access: relaxed device-scope atomics, like the scalar pair above (a
// volatile access would be as coherent, but the compiler waits for each
// volatile load or store before the next one).
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_coherent2(float* p, float v0, float v1) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, (float2_t){v0, v1}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2_t load_coherent2(const float* p) {
  return __builtin_bit_cast(float2_t, __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Wait until this wave's outstanding vector memory operations (stores
// included) are acknowledged: s_waitcnt vmcnt(0), leaving the LDS and export
// counters alone. The signal fences keep the compiler from moving memory
// operations across it.
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- cross-lane

// DPP controls (GFX9 encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// Sum over aligned groups of LANES (4, 8 or 16) consecutive lanes; every lane
// of the group receives the total.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  if constexpr (LANES >= 8) x += dpp_f<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (LANES >= 16) x += dpp_f<DPP_ROW_MIRROR>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) {
  return __shfl_xor(x, m, 64);
}

// Reductions over the eight aligned groups of 8 lanes (lane l with l ^ 8,
// l ^ 16, l ^ 32): a DPP rotate by 8 within each 16-lane row (= xor 8), an
// LDS-free swizzle swapping 16-lane halves of each 32 lanes (= xor 16), and a
// swap of the wave's two 32-lane halves (the pair it returns is {x[l],
// x[l ^ 32]} in every lane). Every lane gets the same sum, in the same order.
__device__ __forceinline__ float xor8_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, true));
}
__device__ __forceinline__ float xor16_f(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
__device__ __forceinline__ float sum_groups8(float x) {
  x += xor8_f(x);
  x += xor16_f(x);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_groups8(float x) {
  x = fmaxf(x, xor8_f(x));
  x = fmaxf(x, xor16_f(x));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column of the
// 16 x 16 matrix-core layouts), on the vector ALU: v_permlane16_swap and
// v_permlane32_swap with both operands x return the pair {x[l], x[l ^ 16]}
// (resp. ^ 32) in every lane. Every lane gets the same result.
__device__ __forceinline__ float max_cols4(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float sum_cols4(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// ---------------------------------------------------------------- partition

__device__ __forceinline__ bool seq_valid(int32_t len, int32_t T, int32_t capacity) {
  return len >= T && len <= capacity;
}

// First 128-token step of a sequence of length len that holds a visible
// key: with a window of W positions the earliest key any of the T new
// tokens sees is len - T - W + 1 (for t = 0); without one it is 0.
__device__ __forceinline__ int unit_first_step(const AttnArgs& a, int len) {
  return a.window > 0 ? max(0, len - a.T - a.window + 1) / STEP : 0;
}

// Steps unit (b, k, rb) of a sequence of length len streams (0 for invalid
// lengths): from its first visible step to the step holding the last key
// any of its rows sees. Under the causal rule that is row block rb's last
// new token (a row block of a long query block stops there; the last row
// block, and every unit of a single row block, reach the sequence's end);
// with a tree mask, whose rows may set any bit, the sequence's end.
__device__ __forceinline__ int unit_steps(const AttnArgs& a, int len, int rb) {
  if (!seq_valid(len, a.T, a.capacity)) return 0;
  int end = len;
  if (!a.tree) end = len - a.T + (min((rb + 1) * a.RMAX, a.R) - 1) / a.G + 1;
  return (end + STEP - 1) / STEP - unit_first_step(a, len);
}
// Steps of the RB units of one (b, k).
__device__ __forceinline__ int kv_steps(const AttnArgs& a, int len) {
  int n = 0;
  for (int rb = 0; rb < a.RB; ++rb) n += unit_steps(a, len, rb);
  return n;
}

// First key position a unit's queries can see (0 without a window). Rows
// before it are never read, so with a block table the blocks wholly before
// it need not be mapped: under a window the cache a call touches no longer
// grows with the sequence.
__device__ __forceinline__ int first_visible(const AttnArgs& a, int len) {
  return a.window > 0 ? max(0, len - a.T - a.window + 1) : 0;
}

// Whether key position tok is visible to new token t of a sequence whose new
// rows start at new0 (= seq_len - T), given the word of t's tree-mask row
// that holds the key's bit (word (tok - new0) / 32; ignored without a tree
// mask). Prior rows are visible, new rows by the causal rule or the tree
// row, rows past the sequence never; a window further requires
// tok > new0 + t - W.
__device__ __forceinline__ bool key_visible(const AttnArgs& a, int tok, int new0, int t,
                                            uint32_t word) {
  bool ok;
  if (tok < new0)
    ok = true;
  else if (a.tree)
    ok = tok - new0 < a.T && ((word >> ((tok - new0) & 31)) & 1u);
  else
    ok = tok <= new0 + t;
  if (a.window > 0) ok = ok && tok > new0 + t - a.window;
  return ok;
}

// s_pre[0..B]: exclusive prefix sums of steps per sequence (0 for invalid
// lengths); s_pre[B + 1 + b]: the length of sequence b, so that later reads
// of it are LDS reads rather than global loads (a global load inside the
// unit loop would be waited for together with the tile prefetches).
// s_pre holds 2B + 1 ints. Requires THREADS threads and a scratch of WAVES
// ints.
__device__ __forceinline__ void build_tile_prefix(const AttnArgs& a, int32_t* s_pre, int32_t* s_wave) {
  const int tid = threadIdx.x;
  const int per = (a.B + THREADS - 1) / THREADS;
  const int b0 = tid * per;
  int32_t local = 0;
  for (int i = 0; i < per; ++i) {
    int b = b0 + i;
    if (b < a.B) {
      local += kv_steps(a, a.seq_lens[b]);
    }
  }
  // inclusive scan of `local` over the workgroup
  const int lane = tid & 63;
  int32_t incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int32_t y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wave[tid >> 6] = incl;
  __syncthreads();
  int32_t carry = 0;
  for (int w = 0; w < (tid >> 6); ++w) carry += s_wave[w];
  int32_t run = carry + incl - local;  // exclusive prefix of this thread's chunk
  for (int i = 0; i < per; ++i) {
    int b = b0 + i;
    if (b < a.B) {
      s_pre[b] = run;
      int32_t len = a.seq_lens[b];
      s_pre[a.B + 1 + b] = len;
      run += kv_steps(a, len);
    }
  }
  if (tid == THREADS - 1) s_pre[a.B] = carry + incl;
  __syncthreads();
}

// A worker's view of one unit segment (a worker is one wave or one
// workgroup, depending on the kernel).
struct Segment {
  int b;          // sequence
  int k;          // key-value head
  int rb;         // query-row block
  int unit;       // (b * K + k) * RB + rb
  int seq_len;    // valid tokens
  int t_begin;    // first step of this segment (counted from the sequence's first token)
  int t_end;      // one past the last step
  int n_parts;    // workers sharing the unit (1: this one writes the output directly)
  int first_wg;   // first worker sharing the unit
};

// Workers' shares of the steps: equal, or (fast > 0) weighted. With two
// workgroups per CU (a full round of 2 x CUs) the first `fast` = CUs
// workgroups are each the older of a CU's pair, and the older one is served
// first (about 25% faster on the decode kernels, about 20% on the long-block
// kernel): its share is weighted wf against the younger one's ws. In launch
// order (per = 0) the fast workers are workers [0, fast); numbered XCD by
// XCD (worker_of, per = W / xcds workers per XCD) they are the first half of
// each XCD's block. On top of that, a worker's share is multiplied by xe on
// an even-numbered XCD and by xo on an odd-numbered one (the odd XCD of each
// pair streams a few percent slower; 1 : 1 when not weighted). Workgroup i
// runs on XCD i mod xcds with xcds even, so in launch order worker w's XCD
// has the parity of w, and in XCD order that of its block w / per.
struct Partition {
  int64_t total;  // steps over all units
  int w_eff;      // workers with work: min(W, total); each then has >= 1 step
  int64_t lo, hi; // this worker's flat step range
  int fast;       // workers with the larger share (0: equal shares)
  int per;        // > 0: fast workers are the first per / 2 of each block of per
  int wf, ws;     // share weights of the older and the younger workgroup
  int xe, xo;     // share factors on even- and odd-numbered XCDs
  int64_t wt;     // sum of the shares (w_eff when equal)
  int seg;        // virtual steps before each unit (see make_partition); 0: none

  // XCD factors of launch-order workers [0, n) (even ones xe, odd ones xo),
  // and its inverse: the largest n with xsum(n) <= v
  __host__ __device__ int64_t xsum(int64_t n) const { return (n + 1) / 2 * xe + n / 2 * xo; }
  __host__ __device__ int64_t xinv(int64_t v) const {
    const int64_t m = v / (xe + xo), r = v - m * (xe + xo);
    return 2 * m + (r >= xe ? 1 : 0);
  }
  __host__ __device__ int64_t share_prefix(int w) const {  // shares of workers [0, w)
    if (per) {
      const int h = per >> 1, r = w % per, blk = w / per;
      const int64_t be = (int64_t)h * (wf + ws) * xe, bo = (int64_t)h * (wf + ws) * xo;
      return (int64_t)(blk >> 1) * (be + bo) + (blk & 1 ? be : 0) +
             (int64_t)(blk & 1 ? xo : xe) * ((int64_t)(r < h ? r : h) * wf + (int64_t)(r > h ? r - h : 0) * ws);
    }
    if (!fast) return xsum(w);
    const int64_t sf = xsum(w < fast ? w : fast);
    return wf * sf + ws * (xsum(w) - sf);
  }
  // Worker w's range is [total * P(w) / wt, total * P(w + 1) / wt), P the
  // share prefix; the owner of step x is the largest w with P(w) <= u.
  __host__ __device__ int owner(int64_t x) const {  // worker whose range holds step x
    const int64_t u = ((x + 1) * wt - 1) / total;
    int64_t w;
    if (per) {
      const int h = per >> 1;
      const int64_t be = (int64_t)h * (wf + ws) * xe, bo = (int64_t)h * (wf + ws) * xo;
      const int64_t pr = u / (be + bo);
      int64_t rem = u - pr * (be + bo), blk = 2 * pr, xs = xe;
      if (rem >= be) {
        blk += 1;
        rem -= be;
        xs = xo;
      }
      const int64_t hf = (int64_t)h * wf * xs;
      w = blk * per + (rem < hf ? rem / (wf * xs) : h + (rem - hf) / (ws * xs));
    } else if (!fast) {
      w = xinv(u);
    } else {
      const int64_t sf = xsum(fast);
      w = u < wf * sf ? xinv(u / wf) : xinv(sf + (u - wf * sf) / ws);
    }
    return (int)(w < w_eff - 1 ? w : w_eff - 1);
  }
};

// The worker a workgroup plays. Workgroups are dealt to the XCDs round
// robin (workgroup i runs on XCD i mod xcds), each XCD with its own L2; with
// xcds > 0 (and W a multiple of it) the workers of one XCD are consecutive,
// so the consecutive row blocks of one (b, k), which read the same K and V
// rows, mostly share an L2.
__device__ __forceinline__ int worker_of(const AttnArgs& a, int wg) {
  if (a.xcds <= 0) return wg;
  const int per = a.W / a.xcds;
  return (wg % a.xcds) * per + wg / a.xcds;
}

// Worker w's partition of `total` steps over W workers, with the launch's
// weighting (fast_workers, xcds, the share weights and XCD factors as in
// AttnArgs). Host-callable for the checks of the test export.
__host__ __device__ inline Partition partition_of(int64_t total, int W, int fast_workers, int xcds,
                                                  int share_fast, int share_slow, int xcd_even,
                                                  int xcd_odd, int w) {
  Partition p;
  p.total = total;
  p.w_eff = (int)(p.total < (int64_t)W ? p.total : (int64_t)W);
  // weighted only with at least two steps per worker (and, below, only where
  // every weighted share keeps at least one step); numbered XCD by XCD, only
  // with every worker busy (the block structure)
  p.fast = fast_workers > 0 && fast_workers < p.w_eff && p.total >= 2 * (int64_t)p.w_eff
               ? fast_workers : 0;
  p.per = 0;
  if (p.fast && xcds > 0) {
    if (p.w_eff == W && W == 2 * fast_workers && fast_workers % xcds == 0)
      p.per = W / xcds;
    else
      p.fast = 0;
  }
  p.wf = share_fast;
  p.ws = share_slow;
  p.seg = 0;
  // the XCD factors only with the weighted shares of a full round (an even
  // number of fast workers keeps the parity pattern of launch order)
  const bool xw = p.fast && xcd_even > 0 && xcd_odd > 0 && (p.per || p.fast % 2 == 0);
  p.xe = xw ? xcd_even : 1;
  p.xo = xw ? xcd_odd : 1;
  p.wt = p.share_prefix(p.w_eff);
  // every worker keeps at least one step: otherwise equal shares
  const int64_t wmin = (int64_t)(p.wf < p.ws ? p.wf : p.ws) * (p.xe < p.xo ? p.xe : p.xo);
  if (p.fast && p.total * wmin < p.wt) {
    p.fast = p.per = 0;
    p.xe = p.xo = 1;
    p.wt = p.share_prefix(p.w_eff);
  }
  if (w < p.w_eff) {
    p.lo = p.total * p.share_prefix(w) / p.wt;
    p.hi = p.total * p.share_prefix(w + 1) / p.wt;
  } else {
    p.lo = p.hi = 0;
  }
  return p;
}

// The flat step a virtual step v stands for, with c > 0 virtual steps
// placed before each unit's steps: unit u ((b * K + k) * RB + rb, in flat
// order) then starts at virtual step (its first flat step) + c * u, and its
// c virtual steps stand for its first flat step. pre[b] (b <= B): the steps
// of one (b', k) summed over b' < b; us(b, rb): the steps of unit (b, k, rb).
template <typename UnitSteps>
__host__ __device__ inline int64_t flat_of_virtual(int B, int K, int RB, int64_t c, const int32_t* pre,
                                                   UnitSteps us, int64_t v) {
  const int64_t cu = c * K * RB;  // virtual steps of one sequence's units
  if (v >= (int64_t)pre[B] * K + cu * B) return (int64_t)pre[B] * K;
  // last b whose virtual start pre[b] * K + cu * b is <= v
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)pre[mid] * K + cu * mid <= v) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int tk = pre[b + 1] - pre[b];
  int64_t off = v - ((int64_t)pre[b] * K + cu * b);
  const int64_t span = tk + c * RB;  // virtual steps of one (b, k)
  const int64_t k = off / span;
  off -= k * span;
  int64_t flat = (int64_t)pre[b] * K + k * tk;
  for (int rb = 0; rb < RB; ++rb) {
    if (off < c) return flat;
    off -= c;
    const int n = us(b, rb);
    if (off < n) return flat + off;
    off -= n;
    flat += n;
  }
  return flat;
}

// Worker w's partition of `total` flat steps over W workers in equal shares
// of the steps plus c virtual steps before each of the B * K * RB units
// (flat_of_virtual), its range mapped back to flat steps. Host-callable for
// the checks of the test export.
template <typename UnitSteps>
__host__ __device__ inline Partition costed_partition(int64_t total, int B, int K, int RB, int c,
                                                      const int32_t* pre, UnitSteps us, int W, int w) {
  Partition p = partition_of(total + (int64_t)c * B * K * RB, W, 0, 0, 1, 1, 0, 0, w);
  p.seg = c;
  if (c > 0) {
    p.lo = flat_of_virtual(B, K, RB, c, pre, us, p.lo);
    p.hi = flat_of_virtual(B, K, RB, c, pre, us, p.hi);
  }
  return p;
}

// This worker's flat step range. With a.seg_steps = c > 0 the shares are
// taken of the virtual steps (c before each unit: the fixed cost of a
// segment, the waves' fold and the partial's stores, in steps), so a
// worker whose range enters more units gets fewer real steps; the range is
// the flat steps its virtual range stands for. Ranges stay contiguous and
// cover every flat step once; a worker whose virtual range lies within one
// unit's virtual steps gets none (costed_partition). Partition::owner takes
// virtual steps: flat step x of unit u is virtual step x + c * (u + 1).
// COSTED: equal shares with those virtual steps (the per-wave matrix-core
// kernel, one workgroup per CU in launch order; the compiler folds the
// equal shares into the owner lookups). Otherwise the launch's weighted
// shares of the flat steps alone (a.seg_steps is not read).
template <bool COSTED>
__device__ __forceinline__ Partition make_partition(const AttnArgs& a, const int32_t* s_pre,
                                                    int w) {
  const int64_t total = (int64_t)__builtin_amdgcn_readfirstlane(s_pre[a.B]) * a.K;
  if constexpr (!COSTED) {
    return partition_of(total, a.W, a.fast_workers, a.xcds, a.share_fast, a.share_slow,
                        a.xcd_even, a.xcd_odd, w);
  } else {
    const auto us = [&](int b, int rb) { return unit_steps(a, s_pre[a.B + 1 + b], rb); };
    return costed_partition(total, a.B, a.K, a.RB, a.seg_steps, s_pre, us, a.W, w);
  }
}

// Segment containing flat step x (x < p.total).
__device__ __forceinline__ Segment find_segment(const AttnArgs& a, const int32_t* s_pre,
                                                const Partition& p, int64_t x) {
  // first b with s_pre[b + 1] * K > x
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)s_pre[mid + 1] * a.K > x) hi = mid; else lo = mid + 1;
  }
  // every field is wave-uniform; readfirstlane keeps them in scalar registers
  Segment s;
  s.b = __builtin_amdgcn_readfirstlane(lo);
  const int p0 = __builtin_amdgcn_readfirstlane(s_pre[s.b]);
  const int tk = __builtin_amdgcn_readfirstlane(s_pre[s.b + 1]) - p0;  // steps of one (b, k)
  const int64_t base = (int64_t)p0 * a.K;
  int off = (int)(x - base);  // < tk * K
  s.k = off / tk;
  off -= s.k * tk;
  s.seq_len = __builtin_amdgcn_readfirstlane(s_pre[a.B + 1 + s.b]);
  // the row block: its units' steps run back to back (off < tk ends the walk)
  int rb = 0, tb = unit_steps(a, s.seq_len, 0);
  while (off >= tb) {
    off -= tb;
    ++rb;
    tb = unit_steps(a, s.seq_len, rb);
  }
  s.rb = __builtin_amdgcn_readfirstlane(rb);
  tb = __builtin_amdgcn_readfirstlane(tb);
  s.unit = (s.b * a.K + s.k) * a.RB + s.rb;
  s.t_begin = __builtin_amdgcn_readfirstlane(off);
  const int64_t room = p.hi - x;
  s.t_end = (int64_t)(tb - s.t_begin) < room ? tb : s.t_begin + (int)room;
  const int64_t vstart = x - s.t_begin + (int64_t)p.seg * (s.unit + 1);  // virtual
  s.first_wg = p.owner(vstart);
  s.n_parts = p.owner(vstart + tb - 1) - s.first_wg + 1;
  // step indices from here on count from the sequence's first token
  const int fs = unit_first_step(a, s.seq_len);
  s.t_begin += fs;
  s.t_end += fs;
  return s;
}

// ---------------------------------------------------------------- fused append

// The fused append's share of this workgroup: every new row that lies in one
// of its own steps, copied in 16-byte chunks to its logical position exactly
// as the separate append does (rows of an out-of-range block entry are
// skipped; sequences of invalid length own no steps). Each new row is read
// only by the workgroup owning its step (and the clamped reads past a
// sequence's end hit its last row, in the same step), so after this
// workgroup's stores are acknowledged and its waves have met, its own reads
// see them and no other workgroup reads them. Requires one row block per
// (b, k): with several, other workgroups would read the rows too.
template <int H, int NT, bool PAGED>
__device__ __forceinline__ void append_owned(const AttnArgs& a, const int32_t* s_pre, const Partition& part) {
  if (!a.k_new) return;
  constexpr int CPR = H / 8;  // 16-byte chunks per row
  for (int64_t x = part.lo; x < part.hi;) {
    const Segment g = find_segment(a, s_pre, part, x);
    x += g.t_end - g.t_begin;
    const int new0 = g.seq_len - a.T;
    const int lo = max(new0, g.t_begin * STEP);
    const int hi = min(g.seq_len, g.t_end * STEP);
    for (int e = threadIdx.x; e < (hi - lo) * CPR; e += NT) {
      const int pos = lo + e / CPR;
      const int ch = e - (e / CPR) * CPR;
      int64_t off;
      if constexpr (PAGED) {
        const int blk = a.table[(int64_t)g.b * a.max_blocks + (pos >> a.block_shift)];
        if ((unsigned)blk >= (unsigned)a.num_blocks) continue;
        off = (int64_t)blk * a.stride_seq + (int64_t)(pos & ((1 << a.block_shift) - 1)) * a.stride_tok;
      } else {
        off = (int64_t)g.b * a.stride_seq + (int64_t)pos * a.stride_tok;
      }
      off += (int64_t)g.k * a.stride_head + ch * 16;
      const int64_t src = (((int64_t)g.b * a.T + (pos - new0)) * a.K + g.k) * (H * 2) + ch * 16;
      *reinterpret_cast<uint4*>(a.k_store + off) = *reinterpret_cast<const uint4*>(a.k_new + src);
      *reinterpret_cast<uint4*>(a.v_store + off) = *reinterpret_cast<const uint4*>(a.v_new + src);
    }
  }
  wait_stores();
  __syncthreads();
}

// ---------------------------------------------------------------- outputs

__device__ __forceinline__ int64_t row_index(const AttnArgs& a, int b, int k, int r) {
  // query row r of unit (b, k) is (t, g) with r = t * G + g
  const int t = r / a.G;
  const int g = r - t * a.G;
  return ((int64_t)b * a.T + t) * a.N + (int64_t)k * a.G + g;
}

// Final write of one (row, h) element from base-2 stats.
__device__ __forceinline__ void write_final(const AttnArgs& a, int b, int k, int r, int H, int h,
                                            float o_sum, float m, float l) {
  const int64_t ri = row_index(a, b, k, r);
  store_out(a.out, ri * H + h, a.out_dtype, o_sum / l);
  if (h == 0 && a.lse) a.lse[ri] = (m + __log2f(l)) * LN2;
}

// NaN outputs for the rows of sequences with an invalid length. Units are
// dealt round-robin to all launched workgroups; lengths come from the LDS
// copy build_tile_prefix made (s_pre[B + 1 + b]), so no global load is
// waited for here.
template <int H>
__device__ __forceinline__ void fill_invalid(const AttnArgs& a, const int32_t* s_pre) {
  const float qnan = __int_as_float(0x7fc00000);
  const int units = a.B * a.K;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int b = u / a.K;
    if (seq_valid(s_pre[a.B + 1 + b], a.T, a.capacity)) continue;
    const int k = u - b * a.K;
    for (int e = threadIdx.x; e < a.R * H; e += THREADS) {
      const int r = e / H, h = e - (e / H) * H;
      const int64_t ri = row_index(a, b, k, r);
      store_out(a.out, ri * H + h, a.out_dtype, qnan);
      if (h == 0 && a.lse) a.lse[ri] = qnan;
    }
  }
}

// Finishing one unit segment whose per-wave states sit in LDS:
//   s_m[w * RMAX + r], s_l[w * RMAX + r], s_o[(w * RMAX + r) * H + h]
// for NW wave states (s_w: LDS for the per-row combination, [NW + 2][RMAX]). The waves' states are combined, then either the output
// is written (the segment is the whole unit: finish_direct) or a partial is
// stored (store_partial). A worker's shared units are counted together once
// its whole range is done (count_and_merge): the workgroup that counts a
// unit's last partial merges them all (merge_partials). Waiting for the
// partial stores and for the count's return only once per worker, at its
// end, keeps both latencies out of the middle of the range. (The kernels
// count the partial of a range's first segment, the later steps of a unit
// shared with the worker before, at once instead: the worker holding that
// unit's first steps, which it does last, then merges it, and no workgroup
// ends with two merges.) `bad` marks a
// segment that met an out-of-range block-table entry: its result is NaN.

// Per row r < rows: the largest of the NW waves' maxima, each wave's weight
// 2^(m_w - M) and the combined sum, into s_w ([NW + 2][RMAX] floats: weights,
// then M, then L). With one wave there is nothing to combine. Ends with a
// barrier when it writes.
template <int NW>
__device__ __forceinline__ void combine_rows(const AttnArgs& a, int rows, const float* s_m,
                                             const float* s_l, float* s_w) {
  if constexpr (NW > 1) {
    for (int r = threadIdx.x; r < rows; r += THREADS) {
      float M = NEG_BIG;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w * a.RMAX + r]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = __builtin_amdgcn_exp2f(s_m[w * a.RMAX + r] - M);
        s_w[w * a.RMAX + r] = wt;
        L += wt * s_l[w * a.RMAX + r];
      }
      s_w[NW * a.RMAX + r] = M;
      s_w[(NW + 1) * a.RMAX + r] = L;
    }
    __syncthreads();
  }
}

// Combined state of the NW waves for (row r, dim h), after combine_rows;
// rows of s_o are OST floats apart.
template <int H, int NW, int OST = H>
__device__ __forceinline__ void combine_waves(const AttnArgs& a, const float* s_m, const float* s_l,
                                              const float* s_o, const float* s_w, int r, int h,
                                              float& M, float& L, float& O) {
  if constexpr (NW == 1) {
    M = s_m[r];
    L = s_l[r];
    O = s_o[r * OST + h];
  } else {
    M = s_w[NW * a.RMAX + r];
    L = s_w[(NW + 1) * a.RMAX + r];
    O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) O += s_w[w * a.RMAX + r] * s_o[(w * a.RMAX + r) * OST + h];
  }
}

// The segment is its whole unit: write the output. Ends with a barrier, so
// LDS may be reused afterwards.
template <int H, int NW, int OST = H>
__device__ __forceinline__ void finish_direct(const AttnArgs& a, const Segment& s, const float* s_m,
                              const float* s_l, const float* s_o, float* s_w, bool bad) {
  const int rows = min(a.RMAX, a.R - s.rb * a.RMAX);
  const int row0 = s.rb * a.RMAX;
  const float qnan = __int_as_float(0x7fc00000);
  combine_rows<NW>(a, rows, s_m, s_l, s_w);
  for (int e = threadIdx.x; e < rows * H; e += THREADS) {
    const int r = e / H, h = e - (e / H) * H;
    float M, L, O;
    combine_waves<H, NW, OST>(a, s_m, s_l, s_o, s_w, r, h, M, L, O);
    if (bad) O = L = M = qnan;
    write_final(a, s.b, s.k, row0 + r, H, h, O, M, L);
  }
  __syncthreads();
}

// Store this worker's partial of the unit. The stores are device-coherent
// (they bypass this XCD's L2 copy); they are waited for in count_and_merge,
// before the partial is counted. Ends with a barrier, so LDS may be reused
// afterwards.
template <int H, int NW, int OST = H>
__device__ __forceinline__ void store_partial(const AttnArgs& a, const Segment& s, int worker, const float* s_m,
                              const float* s_l, const float* s_o, float* s_w, bool bad) {
  const int rows = min(a.RMAX, a.R - s.rb * a.RMAX);
  const float qnan = __int_as_float(0x7fc00000);
  const int slot = worker + s.unit;
  float* po = a.part_o + (int64_t)slot * a.RMAX * H;
  float* pml = a.part_ml + (int64_t)slot * a.RMAX * 2;
  combine_rows<NW>(a, rows, s_m, s_l, s_w);
  for (int e = threadIdx.x; e < rows * H; e += THREADS) {
    const int r = e / H, h = e - (e / H) * H;
    float M, L, O;
    combine_waves<H, NW, OST>(a, s_m, s_l, s_o, s_w, r, h, M, L, O);
    if (bad) O = L = M = qnan;
    store_coherent(po + r * H + h, O);
    if (h == 0) {
      store_coherent(pml + r * 2 + 0, M);
      store_coherent(pml + r * 2 + 1, L);
    }
  }
  __syncthreads();
}

// Count a stored partial (one thread, after its stores were acknowledged);
// true for the unit's last one.
//
// Publication. A partial is written with device-coherent stores (agent-scope
// atomic stores: on gfx950 they write through this XCD's L2 to the memory
// side, which every XCD reads coherently) and the storing waves wait until
// those stores are acknowledged (s_waitcnt vmcnt(0) counts a store as done
// only once the coherent write has completed) before a barrier and this
// count; the count itself is a device-scope atomic performed at the memory
// side, so it is ordered after the acknowledged partial. The workgroup whose
// count completes a unit takes a device-scope acquire fence and reads the
// partials with device-coherent loads. A release on every count (a write-back
// of the whole L2 per workgroup) measured 15% slower on batched decode, so
// the producer side relies on the acknowledgment instead.
__device__ __forceinline__ bool count_partial(const AttnArgs& a, const Segment& s) {
  const int prev = __hip_atomic_fetch_add(&a.counters[s.unit], 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
  return prev == s.n_parts - 1;
}

// Merge all partials of the unit and write the output; called by the
// workgroup that counted the last one, after its acquire fence. The count is
// reset for the next call.
//
// With LDS scratch for every partial's row statistics (n * rows * 2 floats
// within `cap`) and rows * H <= EPT * THREADS, the thread's EPT output
// elements are merged in passes of EP; a pass loads PJ partials' elements at
// once (one memory round trip per PJ partials, PJ * EP <= 32 registers), and
// the first of these loads is issued together with the statistics of all
// partials (into the scratch, each row's weights computed once). Otherwise
// the partials are folded in chunks of 8 whose loads are issued together,
// with an online rescale between chunks.
template <int H, int EPT>
__device__ __forceinline__ void merge_partials(const AttnArgs& a, const Segment& s, float* scratch, int cap) {
  const int rows = min(a.RMAX, a.R - s.rb * a.RMAX);
  const int row0 = s.rb * a.RMAX;
  constexpr int CH = 8;
  constexpr int EP = EPT < 16 ? EPT : 16;
  constexpr int PJ = 32 / EP > 16 ? 16 : 32 / EP;
  const int n = s.n_parts;
  auto slot_of = [&](int j) { return (int64_t)s.first_wg + j + s.unit; };
  if constexpr (EPT % 2 == 0) {
    // Two consecutive elements of a row per thread and load (8-byte
    // loads): passes of up to 16 such chunks, each loading PJ partials'
    // chunks at once (PJ * EP <= 32 chunks); the first pass's loads are
    // issued together with the statistics of all partials. Same summation
    // order as the element-wise form below.
    if (n * rows * 2 + 2 * rows <= cap && rows * H <= EPT * THREADS) {
      constexpr int E2 = EPT / 2;
      constexpr int EP = E2 < 16 ? E2 : 16;
      constexpr int PJ = 32 / EP > 16 ? 16 : 32 / EP;
      float* sw = scratch;                // [n][rows]: m, then the weight 2^(m - M)
      float* sl = scratch + n * rows;     // [n][rows]: l
      float* sM = scratch + 2 * n * rows; // [rows]: M
      float* sL = sM + rows;              // [rows]: L
      const int q_max = rows * H / 2 - 1;
      auto chunk = [&](int p0, int u) { return min((int)threadIdx.x + (p0 + u) * THREADS, q_max); };
      float2_t ov[PJ][EP];
      auto load_o = [&](int p0, int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < PJ; ++jj) {
          const float* po = a.part_o + slot_of(min(j0 + jj, n - 1)) * a.RMAX * H;
#pragma unroll
          for (int u = 0; u < EP; ++u) ov[jj][u] = load_coherent2(po + 2 * chunk(p0, u));
        }
      };
      load_o(0, 0);
      for (int e = threadIdx.x; e < n * rows; e += THREADS) {
        const int j = e / rows, r = e - (e / rows) * rows;
        const float2_t ml = load_coherent2(a.part_ml + slot_of(j) * a.RMAX * 2 + r * 2);
        sw[e] = ml.x;
        sl[e] = ml.y;
      }
      __syncthreads();
      for (int r = threadIdx.x; r < rows; r += THREADS) {
        float M = NEG_BIG;
        for (int j = 0; j < n; ++j) M = fmaxf(M, sw[j * rows + r]);
        float L = 0.f;
        for (int j = 0; j < n; ++j) {
          const float w = __builtin_amdgcn_exp2f(sw[j * rows + r] - M);
          sw[j * rows + r] = w;
          L += w * sl[j * rows + r];
        }
        sM[r] = M;
        sL[r] = L;
      }
      __syncthreads();
#pragma unroll
      for (int p0 = 0; p0 < E2; p0 += EP) {
        float2_t O[EP];
#pragma unroll
        for (int u = 0; u < EP; ++u) O[u] = (float2_t){0.f, 0.f};
        for (int j0 = 0; j0 < n; j0 += PJ) {
          if (p0 > 0 || j0 > 0) load_o(p0, j0);
#pragma unroll
          for (int jj = 0; jj < PJ; ++jj) {
            if (j0 + jj < n) {
#pragma unroll
              for (int u = 0; u < EP; ++u) O[u] += sw[(j0 + jj) * rows + 2 * chunk(p0, u) / H] * ov[jj][u];
            }
          }
        }
#pragma unroll
        for (int u = 0; u < EP; ++u) {
          const int q = threadIdx.x + (p0 + u) * THREADS;
          if (p0 + u < E2 && q <= q_max) {
            const int r = 2 * q / H, h = 2 * q - (2 * q / H) * H;
            const int64_t ri = row_index(a, s.b, s.k, row0 + r);
            const float L = sL[r];
            store_out2(a.out, ri * H + h, a.out_dtype, O[u].x / L, O[u].y / L);
            if (h == 0 && a.lse) a.lse[ri] = (sM[r] + __log2f(L)) * LN2;
          }
        }
      }
      __syncthreads();  // the scratch may be reused
      if (threadIdx.x == 0)
        __hip_atomic_store(&a.counters[s.unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
  if (n * rows * 2 + 2 * rows <= cap && rows * H <= EPT * THREADS) {
    float* sw = scratch;                // [n][rows]: m, then the weight 2^(m - M)
    float* sl = scratch + n * rows;     // [n][rows]: l
    float* sM = scratch + 2 * n * rows; // [rows]: M
    float* sL = sM + rows;              // [rows]: L
    // element u of pass p0: threadIdx.x + (p0 + u) * THREADS, clamped into
    // the unit (the duplicates are loaded and never stored)
    auto elem = [&](int p0, int u) { return min((int)threadIdx.x + (p0 + u) * THREADS, rows * H - 1); };
    float ov[PJ][EP];
    auto load_o = [&](int p0, int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int jj = 0; jj < PJ; ++jj) {
        const float* po = a.part_o + slot_of(min(j0 + jj, n - 1)) * a.RMAX * H;
#pragma unroll
        for (int u = 0; u < EP; ++u) ov[jj][u] = load_coherent(po + elem(p0, u));
      }
    };
    load_o(0, 0);
    for (int e = threadIdx.x; e < n * rows; e += THREADS) {
      const int j = e / rows, r = e - (e / rows) * rows;
      const float* ml = a.part_ml + slot_of(j) * a.RMAX * 2 + r * 2;
      sw[e] = load_coherent(ml);
      sl[e] = load_coherent(ml + 1);
    }
    __syncthreads();
    for (int r = threadIdx.x; r < rows; r += THREADS) {
      float M = NEG_BIG;
      for (int j = 0; j < n; ++j) M = fmaxf(M, sw[j * rows + r]);
      float L = 0.f;
      for (int j = 0; j < n; ++j) {
        const float w = __builtin_amdgcn_exp2f(sw[j * rows + r] - M);
        sw[j * rows + r] = w;
        L += w * sl[j * rows + r];
      }
      sM[r] = M;
      sL[r] = L;
    }
    __syncthreads();
#pragma unroll
    for (int p0 = 0; p0 < EPT; p0 += EP) {
      float O[EP];
#pragma unroll
      for (int u = 0; u < EP; ++u) O[u] = 0.f;
      for (int j0 = 0; j0 < n; j0 += PJ) {
        if (p0 > 0 || j0 > 0) load_o(p0, j0);
#pragma unroll
        for (int jj = 0; jj < PJ; ++jj) {
          if (j0 + jj < n) {
#pragma unroll
            for (int u = 0; u < EP; ++u) O[u] += sw[(j0 + jj) * rows + elem(p0, u) / H] * ov[jj][u];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < EP; ++u) {
        const int e = threadIdx.x + (p0 + u) * THREADS;
        if (p0 + u < EPT && e < rows * H) {
          const int r = e / H, h = e - (e / H) * H;
          write_final(a, s.b, s.k, row0 + r, H, h, O[u], sM[r], sL[r]);
        }
      }
    }
    __syncthreads();  // the scratch may be reused
  } else {
#pragma unroll 2
    for (int e = threadIdx.x; e < rows * H; e += THREADS) {
      const int r = e / H, h = e - (e / H) * H;
      float M = NEG_BIG, L = 0.f, O = 0.f;
      for (int base = 0; base < n; base += CH) {
        float mi[CH], li[CH], oi[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const bool ok = base + j < n;
          const int64_t sl = ok ? slot_of(base + j) : slot_of(0);
          const float* ml = a.part_ml + sl * a.RMAX * 2 + r * 2;
          mi[j] = load_coherent(ml);
          li[j] = load_coherent(ml + 1);
          oi[j] = load_coherent(a.part_o + (sl * a.RMAX + r) * H + h);
          if (!ok) {
            mi[j] = NEG_BIG;
            li[j] = 0.f;
            oi[j] = 0.f;
          }
        }
        float Mc = M;
#pragma unroll
        for (int j = 0; j < CH; ++j) Mc = fmaxf(Mc, mi[j]);
        const float keep = exp2f(M - Mc);
        L *= keep;
        O *= keep;
        M = Mc;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const float w = exp2f(mi[j] - M);
          L += w * li[j];
          O += w * oi[j];
        }
      }
      write_final(a, s.b, s.k, row0 + r, H, h, O, M, L);
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.counters[s.unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The units of a worker's range that it shares with other workers: only the
// first and the last segment of a range can be part of a shared unit (every
// segment in between is a whole unit).
struct SharedUnits {
  Segment s0, s1;
  int n = 0;
  __device__ void add(const Segment& s) {
    if (n == 0) s0 = s; else s1 = s;
    ++n;
  }
};

// Finish a segment: the output, or a partial to be counted at the worker's
// end. Ends with a barrier, so LDS may be reused afterwards.
template <int H, int NW, int OST = H>
__device__ __forceinline__ void finish_segment(const AttnArgs& a, const Segment& s, int worker, const float* s_m,
                               const float* s_l, const float* s_o, float* s_w, bool bad,
                               SharedUnits& sh) {
  if (s.n_parts == 1) {
    finish_direct<H, NW, OST>(a, s, s_m, s_l, s_o, s_w, bad);
  } else {
    store_partial<H, NW, OST>(a, s, worker, s_m, s_l, s_o, s_w, bad);
    sh.add(s);
  }
}

// At the end of a worker's range: once its partial stores are acknowledged,
// count them, then merge every unit whose last partial this worker counted.
// Needs s_flag[2] in LDS.
// scratch: LDS free at this point, `cap` floats; EPT: output elements per
// thread of a merge (rows per unit * H / THREADS, rounded up).
template <int H, int EPT>
__device__ __forceinline__ void count_and_merge(const AttnArgs& a, const SharedUnits& sh, int32_t* s_flag,
                                float* scratch, int cap) {
  if (sh.n == 0) return;
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool f0 = count_partial(a, sh.s0);
    const bool f1 = sh.n > 1 && count_partial(a, sh.s1);
    // the merger: acquire the other workgroups' partials (the barrier below
    // orders this before every thread's merge loads)
    if (f0 || f1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_flag[0] = f0;
    s_flag[1] = f1;
  }
  __syncthreads();
  if (s_flag[0]) merge_partials<H, EPT>(a, sh.s0, scratch, cap);
  if (s_flag[1]) merge_partials<H, EPT>(a, sh.s1, scratch, cap);
}

}  // namespace kvc
