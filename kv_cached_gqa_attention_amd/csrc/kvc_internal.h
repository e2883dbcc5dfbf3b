// Host-side declarations shared by the C entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_device.h"

namespace kvc {

// Cache description with byte strides, as the copy kernels take it.
struct CopyArgs {
  char* k;
  char* v;
  const int32_t* table;
  int64_t stride_seq, stride_head, stride_tok;  // bytes
  int32_t capacity, block_shift, max_blocks, num_blocks;
  const char* k_new;  // append: [B, T, K, H]
  const char* v_new;
  char* dst_k;        // gather: [B, K, max_seq_len, H]
  char* dst_v;
  const int32_t* seq_lens;
  int32_t B, T, K, H, max_seq_len;
};

hipError_t launch_append(const CopyArgs& a, bool paged, hipStream_t stream);
hipError_t launch_gather(const CopyArgs& a, hipStream_t stream);
// Zero `bytes` (a multiple of 16) at the 16-byte aligned device address p.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_attn_valu(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream);
// Workgroups of the vector-ALU kernel that fit one CU's LDS for B sequences.
int valu_workgroups_per_cu(int B, int H);
// Workgroups of the matrix-core kernel per CU (one: a wave per SIMD).
int mfma_workgroups_per_cu(int B, int H, int RMAX);
hipError_t launch_attn_mfma(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream);
// Long query blocks: units of WIDE_ROWS rows whose four waves share each K/V tile.
constexpr int WIDE_ROWS = 128;
int wide_workgroups_per_cu(int B, int H);
hipError_t launch_attn_wide(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream);

}  // namespace kvc
