// C entry points: argument checks, launch plan, dispatch.
//
// The plan never reads device data: sequence lengths and block tables stay on
// the device and the kernels divide the work among themselves from them
// ("Accelerating Sonar through speculation", section "Inference with
// speculative decoding": metadata is copied to GPU memory before the model
// runs, and syncing the GPU to the CPU on sequence lengths is the cost to
// avoid). The host only fixes the grid size and the workspace layout.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "kvc.h"
#include "kvc_internal.h"

// Scratch of kvc_attn_noalloc: the same layout as a caller's workspace
// (counters, then partials), one copy per device, held until the process
// ends. Host code never uses this name as an address (on the host it is a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device (noalloc_scratch below).
static __device__ __align__(256) char scratch[KVC_NOALLOC_SCRATCH_BYTES];

namespace {

using kvc::AttnArgs;
using kvc::CopyArgs;

constexpr int MAX_B = 4096;            // sequences per call (per-workgroup LDS prefix table)
// G * T up to this uses the vector-ALU kernel (its per-lane state grows with
// the rows); more rows go to the matrix cores.
constexpr int valu_max_rows(int H) { return H == 64 ? 8 : 4; }
constexpr int MFMA_MAX_NB = 4;         // 16-row blocks per matrix-core unit
// An automatic grid gives every unit a worker of its own. Units of at most
// SHORT_UNIT_STEPS 128-token steps are never split: a split adds a partial
// and a merge (a chain of memory round trips), which costs more than the
// shorter stream saves. Longer units are split as far as every worker keeps
// MIN_STEPS_PER_WORKER steps.
constexpr int SHORT_UNIT_STEPS = 4;
constexpr int MIN_STEPS_PER_WORKER = 2;
// An automatic grid is one round of workgroups: as many per CU as the
// kernel's register and LDS use lets reside (valu_workgroups_per_cu,
// mfma_workgroups_per_cu).
constexpr int DEFAULT_CUS = 256;
constexpr int DEFAULT_XCDS = 8;
// The workspace starts with a fixed-size array of per-unit counters. Only the
// counter atomics (and their reset to zero by the merging workgroup) ever
// write it, so it stays zero between calls whatever shapes they have; the
// partials that follow are scratch, always written before being read.
constexpr int64_t COUNTER_SLOTS = KVC_WORKSPACE_COUNTERS;

// A device attribute of the current device, cached per device (fallback
// when the query fails).
int device_attr(hipDeviceAttribute_t attr, int fallback, int (&cache)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return fallback;
  }
  if (cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, attr, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = fallback;
  }
  cache[dev] = n;
  return n;
}

int device_cu_count() {
  static int cached[64];
  return device_attr(hipDeviceAttributeMultiprocessorCount, DEFAULT_CUS, cached);
}

int device_xcd_count() {
  static int cached[64];
  return device_attr(hipDeviceAttributeNumberOfXccs, DEFAULT_XCDS, cached);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  bool mfma;
  bool wide;    // matrix cores, units of WIDE_ROWS rows sharing each tile over the waves
  int R, RB, RMAX, units;
  int W;        // workgroups launched
  int fast;     // workers given the larger share (see Partition), 0: equal shares
  int share_fast, share_slow;  // the shares' weights
  int xcd_even, xcd_odd;       // share factors by XCD parity (0: none)
  int xcds;     // workers numbered XCD by XCD (see worker_of), 0: in launch order
  int seg_steps;  // virtual steps charged per unit entered (see make_partition)
  int workers;  // independent workers: waves (vector-ALU kernel) or workgroups (matrix cores)
  size_t off_o, off_ml, bytes;
};

// Query-row blocks per (b, k) on the matrix cores for R rows: one block of
// up to 64 rows (the per-wave form); longer query blocks take blocks of
// WIDE_ROWS rows, whose waves share each K/V tile (each further row block
// re-reads the unit's K/V rows).
bool wide_rows(int R) { return (R + 15) / 16 > MFMA_MAX_NB; }
int row_blocks(int R) { return wide_rows(R) ? (R + kvc::WIDE_ROWS - 1) / kvc::WIDE_ROWS : 1; }

bool make_plan(int B, int T, int N, int K, int H, int max_seq_len, int num_wg, Plan* p) {
  if (B < 1 || T < 1 || T > KVC_MAX_T || N < 1 || K < 1 || N % K || (H != 64 && H != 128) ||
      max_seq_len < 1 || num_wg < 0 || B > MAX_B)
    return false;
  const int G = N / K;
  p->R = G * T;
  p->wide = false;
  if (p->R <= valu_max_rows(H)) {
    p->mfma = false;
    p->RB = 1;
    p->RMAX = p->R;
  } else {
    p->mfma = true;
    p->wide = wide_rows(p->R);
    p->RB = row_blocks(p->R);
    p->RMAX = p->wide ? kvc::WIDE_ROWS : (p->R + 15) / 16 * 16;
  }
  const int64_t units = (int64_t)B * K * p->RB;
  if (units > COUNTER_SLOTS) return false;
  p->units = (int)units;
  const int per_wg = 1;  // both kernels: one worker per workgroup
  p->fast = 0;
  if (num_wg > 0) {
    p->W = num_wg > (1 << 20) ? (1 << 20) : num_wg;
  } else {
    const int64_t steps_ub = units * ((max_seq_len + kvc::STEP - 1) / kvc::STEP);
    const int cus = device_cu_count();
    const int per_cu = p->wide   ? kvc::wide_workgroups_per_cu(B, H)
                       : p->mfma ? kvc::mfma_workgroups_per_cu(B, H, p->RMAX)
                                 : kvc::valu_workgroups_per_cu(B, H);
    const int64_t full = (int64_t)cus * per_cu;
    const int64_t unit_steps = (max_seq_len + kvc::STEP - 1) / kvc::STEP;
    int64_t want_workers = unit_steps <= SHORT_UNIT_STEPS
                               ? units
                               : (steps_ub + MIN_STEPS_PER_WORKER - 1) / MIN_STEPS_PER_WORKER;
    if (want_workers < units) want_workers = units;
    int64_t want = (want_workers + per_wg - 1) / per_wg;
    if (want > full) want = full;
    p->W = (int)(want < 1 ? 1 : want);
    // two per CU and a full round: the first `cus` workgroups are each the
    // older of a CU's pair
    p->fast = per_cu == 2 && p->W == full ? cus : 0;
  }
  // Several row blocks per (b, k) read the same K/V rows: number the
  // workers XCD by XCD so that consecutive row blocks mostly share an L2
  // (the weighted shares follow that numbering).
  const int xcds = device_xcd_count();
  p->xcds = p->mfma && p->RB > 1 && xcds > 1 && p->W % xcds == 0 ? xcds : 0;
  // the older workgroup of a CU's pair is about 25% faster on the decode
  // kernels, about 20% on the long-block kernel
  p->share_fast = p->wide ? 6 : 5;
  p->share_slow = p->wide ? 5 : 4;
  // the odd-numbered XCD of each pair streams about 6% slower
  p->xcd_even = xcds > 1 && xcds % 2 == 0 ? 16 : 0;
  p->xcd_odd = xcds > 1 && xcds % 2 == 0 ? 15 : 0;
  p->workers = p->W * per_wg;
  // The per-wave matrix-core kernel pays for each unit a workgroup enters
  // (the waves' fold, the partial's stores and count) about as much as for
  // 1 + R/8 of its steps (one workgroup per CU, 40 rows: about 12 us a
  // segment against 2.7 us a step; 64 rows with a draft tree: about 23
  // against 3.2), so its shares are taken with that many virtual steps per
  // unit (make_partition). The other kernels' segments cost too little
  // against their steps for it to pay.
  p->seg_steps = p->mfma && !p->wide ? 1 + p->R / 8 : 0;
  // (that kernel takes equal shares in launch order: make_partition<true>)
  if (p->mfma && !p->wide) p->fast = p->xcds = 0;
  const size_t slots = (size_t)p->workers + (size_t)p->units;
  p->off_ml = (size_t)COUNTER_SLOTS * sizeof(int32_t);
  p->off_o = p->off_ml + align_up(slots * p->RMAX * 2 * sizeof(float), 256);
  p->bytes = p->off_o + align_up(slots * p->RMAX * H * sizeof(float), 256);
  return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return ((1 << s) == v) ? s : -1;
}

// Shared cache checks; fills capacity (tokens) and block shift.
kvc_status check_cache(const kvc_cache* c, int K, int H, int* capacity, int* shift) {
  if (!c || !c->k || !c->v || c->reserved != 0) return KVC_ERR_INVALID;
  if (c->dtype != KVC_F16 && c->dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
  if (H != 64 && H != 128) return KVC_ERR_UNSUPPORTED;
  if (K < 1) return KVC_ERR_INVALID;
  if (!aligned16(c->k) || !aligned16(c->v)) return KVC_ERR_INVALID;
  if (c->stride_seq < 0 || c->stride_head < 0 || c->stride_tok < 0) return KVC_ERR_INVALID;
  if ((c->stride_seq % 8) || (c->stride_head % 8) || (c->stride_tok % 8)) return KVC_ERR_INVALID;
  if (c->block_table) {
    const int s = log2_exact(c->block_size);
    if (c->block_size < 1 || c->block_size > 4096 || s < 0) return KVC_ERR_INVALID;
    if (c->max_blocks_per_seq < 1 || c->num_blocks < 1) return KVC_ERR_INVALID;
    const int64_t cap = (int64_t)c->max_blocks_per_seq * c->block_size;
    *capacity = cap > INT32_MAX ? INT32_MAX : (int)cap;
    *shift = s;
  } else {
    if (c->capacity < 1) return KVC_ERR_INVALID;
    *capacity = c->capacity;
    *shift = 0;
  }
  return KVC_OK;
}

// Fills the copy arguments of an append (shared by kvc_append and the fused
// entry point's two-launch form).
void fill_copy_args(CopyArgs* a, const kvc_cache* c, int capacity, int shift, const void* k_new,
                    const void* v_new, int B, int T, int K, int H, const int32_t* seq_lens) {
  memset(a, 0, sizeof(*a));
  a->k = static_cast<char*>(c->k);
  a->v = static_cast<char*>(c->v);
  a->table = c->block_table;
  a->stride_seq = c->stride_seq * 2;
  a->stride_head = c->stride_head * 2;
  a->stride_tok = c->stride_tok * 2;
  a->capacity = capacity;
  a->block_shift = shift;
  a->max_blocks = c->block_table ? c->max_blocks_per_seq : 0;
  a->num_blocks = c->block_table ? c->num_blocks : 0;
  a->k_new = static_cast<const char*>(k_new);
  a->v_new = static_cast<const char*>(v_new);
  a->seq_lens = seq_lens;
  a->B = B;
  a->T = T;
  a->K = K;
  a->H = H;
}

// Attention, optionally preceded by the append of k_new / v_new (fused: one
// launch when every (b, k) is one unit, else an append launch first).
// The device address of this device's `scratch` array, taken once per
// device (with that device current); at that first use the counter region is
// cleared on `stream` (every completed call leaves it zero again).
struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[64];

hipError_t noalloc_scratch(void** out, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&] {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess) d.err = kvc::launch_zero(p, (size_t)COUNTER_SLOTS * sizeof(int32_t), stream);
    if (d.err == hipSuccess) d.ptr = p;
  });
  *out = d.ptr;
  return d.err;
}

// ws == nullptr with static_ws: the call runs in this device's `scratch`
// array (kvc_attn_noalloc), after the same checks.
kvc_status attn_common(const kvc_cache* c, const void* q, void* out, int out_dtype, float* lse,
                       int B, int T, int N, int K, int H, const int32_t* seq_lens, int max_seq_len,
                       float scale, int num_wg, void* ws, size_t ws_bytes, void* stream,
                       const kvc_attn_options* opts = nullptr, bool static_ws = false) {
  const void* k_new = opts ? opts->k_new : nullptr;
  const void* v_new = opts ? opts->v_new : nullptr;
  const int window = opts ? opts->window : 0;
  const uint32_t* tree = opts ? opts->tree_mask : nullptr;
  if (opts && (opts->reserved != 0 || window < 0)) return KVC_ERR_INVALID;
  int capacity = 0, shift = 0;
  const kvc_status st = check_cache(c, K, H, &capacity, &shift);
  if (st != KVC_OK) return st;
  if (B < 0 || T < 1 || T > KVC_MAX_T || N < 1 || N % K || num_wg < 0) return KVC_ERR_INVALID;
  if (tree && T > KVC_MAX_TREE_T) return KVC_ERR_INVALID;  // (T + 31) / 32 mask words per new token
  if (out_dtype != KVC_F16 && out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (max_seq_len < T || max_seq_len > capacity) return KVC_ERR_INVALID;
  if (!isfinite(scale)) return KVC_ERR_INVALID;
  if (B > MAX_B) return KVC_ERR_UNSUPPORTED;
  if (B == 0) return KVC_OK;  // nothing to read or write; empty buffers may be null
  if (!q || !out || !seq_lens) return KVC_ERR_INVALID;
  if (!aligned16(q) || !aligned16(out)) return KVC_ERR_INVALID;
  const bool fused = k_new != nullptr || v_new != nullptr;
  if (fused && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))) return KVC_ERR_INVALID;
  if ((int64_t)B * K * (N / K * T <= valu_max_rows(H) ? 1 : row_blocks(N / K * T)) > COUNTER_SLOTS)
    return KVC_ERR_UNSUPPORTED;
  // a window bounds the keys any call streams per unit: at most
  // window + T - 1 positions, starting anywhere inside a 128-token step
  int span = max_seq_len;
  if (window > 0) {
    const int64_t w = (int64_t)window + T - 1 + kvc::STEP;
    if (w < span) span = (int)w;
  }
  Plan p;
  if (!make_plan(B, T, N, K, H, span, num_wg, &p)) return KVC_ERR_INVALID;
  if (static_ws) {
    if (p.bytes > (size_t)KVC_NOALLOC_SCRATCH_BYTES) return KVC_ERR_WORKSPACE;
    if (noalloc_scratch(&ws, static_cast<hipStream_t>(stream)) != hipSuccess) return KVC_ERR_HIP;
    ws_bytes = KVC_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < p.bytes || !aligned16(ws)) return KVC_ERR_WORKSPACE;

  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.k = static_cast<const char*>(c->k);
  a.v = static_cast<const char*>(c->v);
  a.table = c->block_table;
  a.stride_seq = c->stride_seq * 2;
  a.stride_head = c->stride_head * 2;
  a.stride_tok = c->stride_tok * 2;
  a.capacity = capacity;
  a.block_shift = shift;
  a.max_blocks = c->block_table ? c->max_blocks_per_seq : 0;
  a.num_blocks = c->block_table ? c->num_blocks : 0;
  a.q = static_cast<const char*>(q);
  a.out = out;
  a.lse = lse;
  a.seq_lens = seq_lens;
  a.B = B;
  a.T = T;
  a.N = N;
  a.K = K;
  a.G = N / K;
  a.R = p.R;
  a.RB = p.RB;
  a.RMAX = p.RMAX;
  a.out_dtype = out_dtype;
  a.W = p.workers;
  a.fast_workers = p.fast;
  a.share_fast = p.share_fast;
  a.share_slow = p.share_slow;
  a.xcd_even = p.xcd_even;
  a.xcd_odd = p.xcd_odd;
  a.xcds = p.xcds;
  a.seg_steps = p.seg_steps;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.window = window;
  a.tree = tree;
  a.tree_words = (T + 31) / 32;
  char* w = static_cast<char*>(ws);
  a.counters = reinterpret_cast<int32_t*>(w);
  a.part_ml = reinterpret_cast<float*>(w + p.off_ml);
  a.part_o = reinterpret_cast<float*>(w + p.off_o);

  const bool bf = c->dtype == KVC_BF16;
  const bool paged = c->block_table != nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fused && p.RB == 1) {
    a.k_new = static_cast<const char*>(k_new);
    a.v_new = static_cast<const char*>(v_new);
    a.k_store = static_cast<char*>(c->k);
    a.v_store = static_cast<char*>(c->v);
  } else if (fused) {
    CopyArgs ca;
    fill_copy_args(&ca, c, capacity, shift, k_new, v_new, B, T, K, H, seq_lens);
    if (kvc::launch_append(ca, paged, s) != hipSuccess) return KVC_ERR_HIP;
  }
  const hipError_t e = p.wide   ? kvc::launch_attn_wide(a, bf, H, paged, s)
                       : p.mfma ? kvc::launch_attn_mfma(a, bf, H, paged, s)
                                : kvc::launch_attn_valu(a, bf, H, paged, s);
  return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

}  // namespace

extern "C" {

kvc_status kvc_append(const kvc_cache* cache, const void* k_new, const void* v_new, int B, int T,
                      int K, int H, const int32_t* seq_lens, void* stream) {
  int capacity = 0, shift = 0;
  const kvc_status st = check_cache(cache, K, H, &capacity, &shift);
  if (st != KVC_OK) return st;
  if (B < 0 || T < 1) return KVC_ERR_INVALID;
  if (B == 0) return KVC_OK;  // empty buffers may be null
  if (!k_new || !v_new || !seq_lens) return KVC_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVC_ERR_INVALID;
  CopyArgs a;
  fill_copy_args(&a, cache, capacity, shift, k_new, v_new, B, T, K, H, seq_lens);
  const hipError_t e = kvc::launch_append(a, cache->block_table != nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

kvc_status kvc_attn_decode(const kvc_cache* cache, const void* q, void* out, int out_dtype,
                           float* lse, int B, int N, int K, int H, const int32_t* seq_lens,
                           int max_seq_len, float scale, int num_workgroups, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return attn_common(cache, q, out, out_dtype, lse, B, 1, N, K, H, seq_lens, max_seq_len, scale,
                     num_workgroups, workspace, workspace_bytes, stream);
}

kvc_status kvc_attn_verify(const kvc_cache* cache, const void* q, void* out, int out_dtype,
                           float* lse, int B, int T, int N, int K, int H, const int32_t* seq_lens,
                           int max_seq_len, float scale, int num_workgroups, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return attn_common(cache, q, out, out_dtype, lse, B, T, N, K, H, seq_lens, max_seq_len, scale,
                     num_workgroups, workspace, workspace_bytes, stream);
}

kvc_status kvc_append_attend(const kvc_cache* cache, const void* k_new, const void* v_new,
                             const void* q, void* out, int out_dtype, float* lse, int B, int T,
                             int N, int K, int H, const int32_t* seq_lens, int max_seq_len,
                             float scale, int num_workgroups, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_ERR_INVALID;
  kvc_attn_options o;
  memset(&o, 0, sizeof(o));
  o.k_new = k_new;
  o.v_new = v_new;
  return attn_common(cache, q, out, out_dtype, lse, B, T, N, K, H, seq_lens, max_seq_len, scale,
                     num_workgroups, workspace, workspace_bytes, stream, &o);
}

kvc_status kvc_attn(const kvc_cache* cache, const kvc_attn_options* opts, const void* q, void* out,
                    int out_dtype, float* lse, int B, int T, int N, int K, int H,
                    const int32_t* seq_lens, int max_seq_len, float scale, int num_workgroups,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (opts && B > 0 && opts->tree_mask && ((uintptr_t)opts->tree_mask & 3u)) return KVC_ERR_INVALID;
  return attn_common(cache, q, out, out_dtype, lse, B, T, N, K, H, seq_lens, max_seq_len, scale,
                     num_workgroups, workspace, workspace_bytes, stream, opts);
}

kvc_status kvc_attn_noalloc(const kvc_cache* cache, const kvc_attn_options* opts, const void* q,
                            void* out, int out_dtype, float* lse, int B, int T, int N, int K, int H,
                            const int32_t* seq_lens, int max_seq_len, float scale,
                            int num_workgroups, void* stream) {
  if (opts && B > 0 && opts->tree_mask && ((uintptr_t)opts->tree_mask & 3u)) return KVC_ERR_INVALID;
  return attn_common(cache, q, out, out_dtype, lse, B, T, N, K, H, seq_lens, max_seq_len, scale,
                     num_workgroups, nullptr, 0, stream, opts, true);
}

size_t kvc_workspace_bytes(int B, int T, int N, int K, int H, int max_seq_len, int num_workgroups) {
  Plan p;
  if (!make_plan(B, T, N, K, H, max_seq_len, num_workgroups, &p)) return 0;
  return p.bytes;
}

const char* kvc_plan_kernel(int B, int T, int N, int K, int H, int max_seq_len, int num_workgroups) {
  Plan p;
  if (!make_plan(B, T, N, K, H, max_seq_len, num_workgroups, &p)) return nullptr;
  return p.wide ? "attn_wide_kernel" : p.mfma ? "attn_mfma_kernel" : "attn_valu_kernel";
}

const char* kvc_status_string(int status) {
  switch (status) {
    case KVC_OK: return "KVC_OK";
    case KVC_ERR_INVALID: return "KVC_ERR_INVALID: invalid argument";
    case KVC_ERR_UNSUPPORTED: return "KVC_ERR_UNSUPPORTED: unsupported head size, dtype or batch";
    case KVC_ERR_WORKSPACE: return "KVC_ERR_WORKSPACE: workspace missing or too small";
    case KVC_ERR_HIP: return "KVC_ERR_HIP: HIP runtime error at launch";
    default: return "unknown kvc_status";
  }
}

kvc_status kvc_gather(const kvc_cache* paged, void* dst_k, void* dst_v, int B, int K, int H,
                      const int32_t* seq_lens, int max_seq_len, void* stream) {
  int capacity = 0, shift = 0;
  const kvc_status st = check_cache(paged, K, H, &capacity, &shift);
  if (st != KVC_OK) return st;
  if (!paged->block_table || B < 0 || max_seq_len < 1) return KVC_ERR_INVALID;
  if (B == 0) return KVC_OK;  // empty buffers may be null
  if (!dst_k || !dst_v || !seq_lens) return KVC_ERR_INVALID;
  if (!aligned16(dst_k) || !aligned16(dst_v)) return KVC_ERR_INVALID;
  CopyArgs a;
  memset(&a, 0, sizeof(a));
  a.k = static_cast<char*>(paged->k);
  a.v = static_cast<char*>(paged->v);
  a.table = paged->block_table;
  a.stride_seq = paged->stride_seq * 2;
  a.stride_head = paged->stride_head * 2;
  a.stride_tok = paged->stride_tok * 2;
  a.capacity = capacity;
  a.block_shift = shift;
  a.max_blocks = paged->max_blocks_per_seq;
  a.num_blocks = paged->num_blocks;
  a.dst_k = static_cast<char*>(dst_k);
  a.dst_v = static_cast<char*>(dst_v);
  a.seq_lens = seq_lens;
  a.B = B;
  a.K = K;
  a.H = H;
  a.max_seq_len = max_seq_len;
  const hipError_t e = kvc::launch_gather(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

kvc_status kvc_partition_ranges(int64_t total, int W, int fast_workers, int xcds, int share_fast,
                                int share_slow, int xcd_even, int xcd_odd, int64_t* lo_hi,
                                int32_t* owners) {
  if (total < 0 || total > ((int64_t)1 << 32) || W < 1 || W > (1 << 20) || fast_workers < 0 ||
      xcds < 0 || share_fast < 1 || share_fast > 16 || share_slow < 1 || share_slow > 16 ||
      xcd_even < 0 || xcd_even > 64 || xcd_odd < 0 || xcd_odd > 64 || !lo_hi)
    return KVC_ERR_INVALID;
  for (int w = 0; w < W; ++w) {
    const kvc::Partition p = kvc::partition_of(total, W, fast_workers, xcds, share_fast, share_slow,
                                               xcd_even, xcd_odd, w);
    lo_hi[2 * w] = p.lo;
    lo_hi[2 * w + 1] = p.hi;
  }
  if (owners && total > 0) {
    const kvc::Partition p = kvc::partition_of(total, W, fast_workers, xcds, share_fast, share_slow,
                                               xcd_even, xcd_odd, 0);
    for (int64_t x = 0; x < total; ++x) owners[x] = p.owner(x);
  }
  return KVC_OK;
}

kvc_status kvc_partition_ranges_costed(int B, int K, int RB, const int32_t* unit_steps, int W,
                                       int seg_steps, int64_t* lo_hi, int32_t* owners) {
  if (B < 1 || B > (1 << 16) || K < 1 || K > 1024 || RB < 1 || RB > 64 || !unit_steps || W < 1 ||
      W > (1 << 20) || seg_steps < 0 || seg_steps > 64 || !lo_hi)
    return KVC_ERR_INVALID;
  std::vector<int32_t> pre((size_t)B + 1);
  int64_t run = 0;
  for (int b = 0; b < B; ++b) {
    pre[b] = (int32_t)run;
    for (int rb = 0; rb < RB; ++rb) {
      const int32_t n = unit_steps[(int64_t)b * RB + rb];
      if (n < 0 || n > (1 << 20)) return KVC_ERR_INVALID;
      run += n;
    }
    if (run * K > ((int64_t)1 << 32)) return KVC_ERR_INVALID;
  }
  pre[B] = (int32_t)run;
  const int64_t total = run * K;
  const auto us = [&](int b, int rb) { return unit_steps[(int64_t)b * RB + rb]; };
  for (int w = 0; w < W; ++w) {
    const kvc::Partition p = kvc::costed_partition(total, B, K, RB, seg_steps, pre.data(), us, W, w);
    lo_hi[2 * w] = p.lo;
    lo_hi[2 * w + 1] = p.hi;
  }
  if (owners && total > 0) {
    // the lookup the kernel makes: flat step x of unit u at virtual x + c (u + 1)
    const kvc::Partition p = kvc::costed_partition(total, B, K, RB, seg_steps, pre.data(), us, W, 0);
    int64_t x = 0, u = 0;
    for (int b = 0; b < B; ++b)
      for (int k = 0; k < K; ++k)
        for (int rb = 0; rb < RB; ++rb, ++u)
          for (int i = 0; i < us(b, rb); ++i, ++x) owners[x] = p.owner(x + (int64_t)seg_steps * (u + 1));
  }
  return KVC_OK;
}

}  // extern "C"
