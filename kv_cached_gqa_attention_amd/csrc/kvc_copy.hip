// Cache writes and the paged-to-contiguous gather.
//
// Append: every new key and value row goes to its logical position in the
// cache ("Making inference cheap: KV cache, batching and quantization": the
// cache is extended by one row per layer and key-value head per generated
// token; "Accelerating Sonar through speculation", section "Single-token MTP
// schedule": a kernel places the next target tokens at their positions, so
// no GPU-to-CPU synchronisation is needed). With a block table the position
// goes through the logical-to-physical block map of "CS336, lectures 10 and
// 12", section "PagedAttention".
//
// One thread moves one 16-byte chunk of a K row and the matching chunk of the
// V row; consecutive threads cover consecutive chunks, so each row is one
// coalesced run. Bytes are copied unchanged.
#include "kvc_internal.h"

namespace kvc {

template <bool PAGED>
__global__ __launch_bounds__(256) void append_kernel(CopyArgs a) {
  const int cpr = a.H / 8;  // 16-byte chunks per row (2-byte elements)
  const int64_t total = (int64_t)a.B * a.T * a.K * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int ch = (int)(idx % cpr);
    int64_t rest = idx / cpr;
    const int k = (int)(rest % a.K);
    rest /= a.K;
    const int t = (int)(rest % a.T);
    const int b = (int)(rest / a.T);
    const int len = a.seq_lens[b];
    if (len < a.T || len > a.capacity) continue;
    const int pos = len - a.T + t;
    int64_t off;
    if constexpr (PAGED) {
      const int blk = a.table[(int64_t)b * a.max_blocks + (pos >> a.block_shift)];
      if ((unsigned)blk >= (unsigned)a.num_blocks) continue;
      off = (int64_t)blk * a.stride_seq + (int64_t)(pos & ((1 << a.block_shift) - 1)) * a.stride_tok;
    } else {
      off = (int64_t)b * a.stride_seq + (int64_t)pos * a.stride_tok;
    }
    off += (int64_t)k * a.stride_head + ch * 16;
    const int64_t src = (((int64_t)b * a.T + t) * a.K + k) * (a.H * 2) + ch * 16;
    *reinterpret_cast<uint4*>(a.k + off) = *reinterpret_cast<const uint4*>(a.k_new + src);
    *reinterpret_cast<uint4*>(a.v + off) = *reinterpret_cast<const uint4*>(a.v_new + src);
  }
}

__global__ __launch_bounds__(256) void gather_kernel(CopyArgs a) {
  const int cpr = a.H / 8;
  const int64_t total = (int64_t)a.B * a.K * a.max_seq_len * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int ch = (int)(idx % cpr);
    int64_t rest = idx / cpr;
    const int tok = (int)(rest % a.max_seq_len);
    rest /= a.max_seq_len;
    const int k = (int)(rest % a.K);
    const int b = (int)(rest / a.K);
    const int len = a.seq_lens[b];
    if (len < 0 || len > a.max_seq_len || len > a.capacity || tok >= len) continue;
    const int blk = a.table[(int64_t)b * a.max_blocks + (tok >> a.block_shift)];
    if ((unsigned)blk >= (unsigned)a.num_blocks) continue;
    const int64_t off = (int64_t)blk * a.stride_seq + (int64_t)k * a.stride_head +
                        (int64_t)(tok & ((1 << a.block_shift) - 1)) * a.stride_tok + ch * 16;
    const int64_t dst = (((int64_t)b * a.K + k) * a.max_seq_len + tok) * (a.H * 2) + ch * 16;
    *reinterpret_cast<uint4*>(a.dst_k + dst) = *reinterpret_cast<const uint4*>(a.k + off);
    *reinterpret_cast<uint4*>(a.dst_v + dst) = *reinterpret_cast<const uint4*>(a.v + off);
  }
}

// Zero `n16` 16-byte words at p (vector stores).
__global__ __launch_bounds__(256) void zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

static unsigned grid_for(int64_t work) {
  int64_t blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return (unsigned)(blocks < 1 ? 1 : blocks);
}

hipError_t launch_append(const CopyArgs& a, bool paged, hipStream_t stream) {
  const unsigned grid = grid_for((int64_t)a.B * a.T * a.K * (a.H / 8));
  if (paged)
    hipLaunchKernelGGL(append_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n16)), dim3(256), 0, stream, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_gather(const CopyArgs& a, hipStream_t stream) {
  const unsigned grid = grid_for((int64_t)a.B * a.K * a.max_seq_len * (a.H / 8));
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvc
