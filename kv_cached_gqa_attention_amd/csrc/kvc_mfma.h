// Matrix-core building blocks shared by the attention kernels that run
// q.k and p.v on v_mfma_f32_16x16x32_{bf16,f16}: the instruction, the split
// of probability weights into a 16-bit high part and a 16-bit remainder, and
// the transposed LDS read that feeds V^T.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

template <bool BF>
__device__ __forceinline__ floatx4 mfma16(uint4 a, uint4 b, floatx4 c) {
  if constexpr (BF) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Two probability weights e0, e1 (finite, >= 0) as a packed 16-bit high
// part and a packed 16-bit remainder, hi + lo = e to about 2^-16 relative.
// bf16: the high part is e with its low 16 bits cut (exact to take away, so
// the remainder e - hi is exact in fp32), the remainder is cut the same way;
// each pair is packed by one byte permute. f16: round-toward-zero packs.
template <bool BF>
__device__ __forceinline__ void split_pair(float e0, float e1, uint32_t& hi, uint32_t& lo) {
  if constexpr (BF) {
    const uint32_t u0 = __float_as_uint(e0), u1 = __float_as_uint(e1);
    // bytes 2,3 of u0 then bytes 2,3 of u1 (v_perm_b32: bytes 0-3 index S1, 4-7 S0)
    hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
    const float r0 = e0 - __uint_as_float(u0 & 0xffff0000u);
    const float r1 = e1 - __uint_as_float(u1 & 0xffff0000u);
    lo = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
  } else {
    const auto h = __builtin_amdgcn_cvt_pkrtz(e0, e1);
    hi = __builtin_bit_cast(uint32_t, h);
    const auto l = __builtin_amdgcn_cvt_pkrtz(e0 - (float)h[0], e1 - (float)h[1]);
    lo = __builtin_bit_cast(uint32_t, l);
  }
}

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

typedef __attribute__((address_space(3))) char lds_char;

// ds_read_b64_tr_b16 at p: within each 16-lane group, lane i's element j is
// 16-bit element (i % 4) of the 8 bytes that lane 4 j + i / 4 of the group
// addresses (layout checked on the GPU).
__device__ __forceinline__ uint2 read_tr16(const lds_char* p) {
  const v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)p);
  return __builtin_bit_cast(uint2, r);
}

}  // namespace kvc
