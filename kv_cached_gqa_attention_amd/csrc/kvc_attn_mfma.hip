// Split-KV attention on the matrix cores, for units whose G * T query rows
// make q.k and p.v real dense contractions (the speculative verify pass:
// "Accelerating Sonar through speculation", section "Speculative decoding",
// scores n drafted tokens in one target pass; with T = n + 1 tokens and G
// query heads per key-value head, each K/V row serves G * T query rows).
//
// Per 32-token tile and wave (v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulate):
//   S^T [32 tok x 16 q] = K [32 tok x H] . Q^T [H x 16 q]      per 16 query rows
//   O^T [H x 16 q]     += V^T [H x 32 tok] . P^T [32 tok x 16 q]
// Computing the transposed score block puts a query row in a lane column, so
// its running max needs only two cross-lane steps, and P^T leaves the
// accumulators already in the B-operand layout of the p.v product (the
// token-to-k-slot map is chosen to make that true). V^T needs each lane to
// hold 8 tokens of one h: eight lanes load 8 token rows and swap 16-bit
// elements with an 8 x 8 register transpose (swizzle + DPP).
// p is split into a 16-bit high part and a 16-bit remainder, each multiplied
// by V on the matrix cores, so p.v keeps about 16 bits of p (within 2^-16
// relative, far inside the 2e-3 gate).
#include "kvc_device.h"
#include "kvc_internal.h"

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

__device__ __forceinline__ uint32_t swz_xor4(uint32_t x) {
  // ds_swizzle bit-mask mode: and 0x1f, or 0, xor 4 (within 32-lane halves)
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x101F);
}

// 8 x 8 transpose of 16-bit elements across the 8 lanes of an aligned lane
// octet: lane i holds x_i[0..7] (element 2w in the low half of word w), and
// receives y_i[j] = x_j[i]. Block swaps of 4, 2, then 1 element(s).
__device__ __forceinline__ uint4 transpose8(uint4 v, int i8) {
  // Per-lane choices are selects, not branches (every lane runs both sides
  // of a divergent branch anyway).
  uint32_t x0 = v.x, x1 = v.y, x2 = v.z, x3 = v.w;
  const bool b2 = (i8 & 4) != 0, b1 = (i8 & 2) != 0, b0 = (i8 & 1) != 0;
  uint32_t r0 = swz_xor4(b2 ? x0 : x2), r1 = swz_xor4(b2 ? x1 : x3);
  x0 = b2 ? r0 : x0;
  x1 = b2 ? r1 : x1;
  x2 = b2 ? x2 : r0;
  x3 = b2 ? x3 : r1;
  r0 = dpp_u<DPP_QUAD_XOR2>(b1 ? x0 : x1);
  r1 = dpp_u<DPP_QUAD_XOR2>(b1 ? x2 : x3);
  x0 = b1 ? r0 : x0;
  x2 = b1 ? r1 : x2;
  x1 = b1 ? x1 : r0;
  x3 = b1 ? x3 : r1;
  const uint32_t p0 = dpp_u<DPP_QUAD_XOR1>(x0), p1 = dpp_u<DPP_QUAD_XOR1>(x1);
  const uint32_t p2 = dpp_u<DPP_QUAD_XOR1>(x2), p3 = dpp_u<DPP_QUAD_XOR1>(x3);
  // v_perm_b32(S0 = own word, S1 = partner's word): bytes 0-3 index S1,
  // 4-7 index S0. Odd lanes keep their high half and take the partner's
  // high half as low half ([p2 p3 x2 x3]); even lanes keep their low half
  // and take the partner's low half as high half ([x0 x1 p0 p1]).
  const uint32_t sel = b0 ? 0x07060302u : 0x01000504u;
  x0 = __builtin_amdgcn_perm(x0, p0, sel);
  x1 = __builtin_amdgcn_perm(x1, p1, sel);
  x2 = __builtin_amdgcn_perm(x2, p2, sel);
  x3 = __builtin_amdgcn_perm(x3, p3, sel);
  return make_uint4(x0, x1, x2, x3);
}

// MASKED: a window or draft-tree mask is in use (the general per-key test);
// otherwise the causal test alone.
template <bool BF, int H, int NB, bool PAGED, bool MASKED>
__global__ __launch_bounds__(THREADS) void attn_mfma_kernel(AttnArgs a) {
  constexpr int RMAX = NB * 16;  // query rows per unit (row block)
  constexpr int KS = H / 32;     // k-steps of S^T over h
  constexpr int MH = H / 16;     // 16-row h blocks of O^T

  extern __shared__ int32_t s_pre[];  // [2B + 1]
  __shared__ float s_m[RMAX], s_l[RMAX];
  __shared__ float s_o[RMAX * H];
  __shared__ int32_t s_wave[WAVES], s_bad[WAVES], s_flag[2];

  build_tile_prefix(a, s_pre, s_wave);
  fill_invalid<H>(a);
  const Partition part = make_partition(a, s_pre, blockIdx.x);
  append_owned<H, THREADS, PAGED>(a, s_pre, part);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int c = lane & 15;   // column (query row) / A-row (token or h) within a 16 block
  const int g = lane >> 4;   // k-slot group
  const int i8 = lane & 7;   // lane within its transpose octet
  const int hb = c >> 3;     // which 8 of the 16 h of a block this octet loads
  // token of k-slot (g, j): j < 4 -> 4g + j ; j >= 4 -> 16 + 4g + (j - 4)
  const int vtok = (i8 < 4) ? (4 * g + i8) : (16 + 4 * g + i8 - 4);

  SharedUnits shared;
  for (int64_t x = part.lo; x < part.hi;) {
    const Segment s = find_segment(a, s_pre, part, x);
    x += s.t_end - s.t_begin;

    // Q^T fragments (B operand): query row rb*RMAX + 16 nb + c, h = 32 ks + 8 g + j.
    uint4 qf[NB][KS];
    int tq[NB];         // new-token index of this lane's query column
    uint32_t tw[NB];    // its tree word
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int rr = s.rb * RMAX + nb * 16 + c;
      if (rr < a.R) {
        const char* qrow = a.q + row_index(a, s.b, s.k, rr) * (H * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[nb][ks] = load16(qrow + (ks * 32 + g * 8) * 2);
        tq[nb] = rr / a.G;
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[nb][ks] = make_uint4(0, 0, 0, 0);
        tq[nb] = a.T - 1;  // padding column: any valid row, discarded
      }
      tw[nb] = MASKED && a.tree ? a.tree[(int64_t)s.b * a.T + tq[nb]] : 0u;
    }

    const char* kb = a.k + (int64_t)s.k * a.stride_head + (PAGED ? 0 : (int64_t)s.b * a.stride_seq);
    const char* vb = a.v + (int64_t)s.k * a.stride_head + (PAGED ? 0 : (int64_t)s.b * a.stride_seq);
    const int32_t* trow = PAGED ? a.table + (int64_t)s.b * a.max_blocks : nullptr;
    const int bmask = (1 << a.block_shift) - 1;
    bool bad = false;
    const int vis0 = MASKED ? first_visible(a, s.seq_len) : 0;
    auto row_off = [&](int tok) -> int64_t {
      tok = min(tok, s.seq_len - 1);
      if constexpr (MASKED) tok = max(tok, vis0);
      if constexpr (PAGED) {
        int blk = trow[tok >> a.block_shift];
        if ((unsigned)blk >= (unsigned)a.num_blocks) {
          bad = true;
          blk = 0;
        }
        return (int64_t)blk * a.stride_seq + (int64_t)(tok & bmask) * a.stride_tok;
      } else {
        return (int64_t)tok * a.stride_tok;
      }
    };

    uint4 kf[2][KS], vf[MH];
    floatx4 ot[MH][NB];
#pragma unroll
    for (int mh = 0; mh < MH; ++mh)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ot[mh][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m[NB], l[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m[nb] = NEG_BIG;
      l[nb] = 0.f;
    }

    auto load_k = [&](int tile) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int64_t off = row_off(tile * TILE + mb * 16 + c);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[mb][ks] = load16(kb + off + (ks * 32 + g * 8) * 2);
      }
    };
    auto load_v = [&](int tile) {
      const int64_t offv = row_off(tile * TILE + vtok);
#pragma unroll
      for (int mh = 0; mh < MH; ++mh) vf[mh] = load16(vb + offv + (mh * 16 + hb * 8) * 2);
    };
    // Work comes in steps of one tile per wave, so the four waves have equal
    // work; tiles past the unit's end are masked (their loads are clamped).
    load_k(s.t_begin * WAVES + wave);
    __builtin_amdgcn_sched_barrier(0);
    load_v(s.t_begin * WAVES + wave);
    __builtin_amdgcn_sched_barrier(0);

    for (int sp = s.t_begin; sp < s.t_end; ++sp) {
      const int ti = sp * WAVES + wave;
      // ---- S^T = K . Q^T
      floatx4 st[2][NB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16<BF>(kf[mb][ks], qf[nb][ks], acc);
          st[mb][nb] = acc;
        }

      // ---- next tile's K (past the segment: this tile again, cached)
      const int tn = min(sp + 1, s.t_end - 1) * WAVES + wave;
      load_k(tn);

      // ---- scale, mask, online softmax (one query row per lane column)
      const int tok0 = ti * TILE;
      const int new0 = s.seq_len - a.T;
      // tiles wholly inside [new0 + 1 (new0 with a tree), seq_len - window)
      // are visible to every query
      const bool edge = tok0 + TILE > (MASKED && a.tree ? new0 : new0 + 1) ||
                        (MASKED && a.window > 0 && tok0 < s.seq_len - a.window);
      uint4 phi[NB], plo[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float p[2][4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = st[mb][nb][i] * a.scale_log2;
            const int tok = tok0 + mb * 16 + 4 * g + i;
            if (edge && !(MASKED ? key_visible(a, tok, new0, tq[nb], tw[nb]) : tok <= new0 + tq[nb]))
              v = -__builtin_inff();
            p[mb][i] = v;
          }
        float mt = p[0][0];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mt = fmaxf(mt, p[mb][i]);
        mt = fmaxf(mt, shfl_xor_f(mt, 16));
        mt = fmaxf(mt, shfl_xor_f(mt, 32));
        if (__builtin_amdgcn_ballot_w64(mt > m[nb] + RESCALE_MARGIN) != 0ull) {
          const float mn = mt > m[nb] + RESCALE_MARGIN ? mt : m[nb];
          const float alpha = __builtin_amdgcn_exp2f(m[nb] - mn);
          l[nb] *= alpha;
#pragma unroll
          for (int mh = 0; mh < MH; ++mh) ot[mh][nb] *= alpha;
          m[nb] = mn;
        }
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float e0 = __builtin_amdgcn_exp2f(p[mb][i] - m[nb]);
            const float e1 = __builtin_amdgcn_exp2f(p[mb][i + 1] - m[nb]);
            l[nb] += e0 + e1;
            split_pair<BF>(e0, e1, hw[mb * 2 + i / 2], lw[mb * 2 + i / 2]);
          }
        phi[nb] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        plo[nb] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }

      // ---- O^T += V^T . P^T
#pragma unroll
      for (int mh = 0; mh < MH; ++mh) {
        const uint4 vt = transpose8(vf[mh], i8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          ot[mh][nb] = mfma16<BF>(vt, phi[nb], ot[mh][nb]);
          ot[mh][nb] = mfma16<BF>(vt, plo[nb], ot[mh][nb]);
        }
      }

      // ---- next tile's V
      load_v(tn);
    }

    // ---- per-column totals of l (lanes of one column hold different tokens)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      l[nb] += shfl_xor_f(l[nb], 16);
      l[nb] += shfl_xor_f(l[nb], 32);
    }
    {
      const unsigned long long anybad = __ballot(bad);
      if (lane == 0) s_bad[wave] = anybad != 0ull;
    }
    // ---- fold the four waves into one state in LDS, one wave at a time
    for (int w = 0; w < WAVES; ++w) {
      if (wave == w) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = nb * 16 + c;
          float sp = 0.f, sw = 1.f, M = m[nb];
          if (w > 0) {
            const float mp = s_m[col];
            M = fmaxf(mp, m[nb]);
            sp = __builtin_amdgcn_exp2f(mp - M);
            sw = __builtin_amdgcn_exp2f(m[nb] - M);
          }
#pragma unroll
          for (int mh = 0; mh < MH; ++mh)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float* dst = &s_o[col * H + mh * 16 + 4 * g + i];
              *dst = (w > 0 ? *dst * sp : 0.f) + ot[mh][nb][i] * sw;
            }
          if (g == 0) {
            s_l[col] = (w > 0 ? s_l[col] * sp : 0.f) + l[nb] * sw;
            s_m[col] = M;
          }
        }
      }
      __syncthreads();
    }
    bool segbad = false;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) segbad |= s_bad[w] != 0;
    finish_segment<H, 1>(a, s, blockIdx.x, s_m, s_l, s_o, s_m, segbad, shared);
  }
  count_and_merge<H>(a, shared, s_flag);
}

// ---------------------------------------------------------------- launch

template <bool BF, int H, int NB, bool PAGED, bool MASKED>
static hipError_t launch_mfma_t(const AttnArgs& a, hipStream_t stream) {
  const size_t shmem = (size_t)(2 * a.B + 1) * sizeof(int32_t);
  // one worker per workgroup
  hipLaunchKernelGGL((attn_mfma_kernel<BF, H, NB, PAGED, MASKED>), dim3(a.W), dim3(THREADS), shmem,
                     stream, a);
  return hipGetLastError();
}

template <bool BF, int H, bool PAGED, bool MASKED>
static hipError_t launch_mfma_nb(const AttnArgs& a, hipStream_t stream) {
  switch (a.RMAX / 16) {
    case 1: return launch_mfma_t<BF, H, 1, PAGED, MASKED>(a, stream);
    case 2: return launch_mfma_t<BF, H, 2, PAGED, MASKED>(a, stream);
    case 3: return launch_mfma_t<BF, H, 3, PAGED, MASKED>(a, stream);
    case 4: return launch_mfma_t<BF, H, 4, PAGED, MASKED>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool MASKED>
static hipError_t launch_mfma_m(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  if (bf16) {
    if (H == 64)
      return paged ? launch_mfma_nb<true, 64, true, MASKED>(a, stream)
                   : launch_mfma_nb<true, 64, false, MASKED>(a, stream);
    return paged ? launch_mfma_nb<true, 128, true, MASKED>(a, stream)
                 : launch_mfma_nb<true, 128, false, MASKED>(a, stream);
  }
  if (H == 64)
    return paged ? launch_mfma_nb<false, 64, true, MASKED>(a, stream)
                 : launch_mfma_nb<false, 64, false, MASKED>(a, stream);
  return paged ? launch_mfma_nb<false, 128, true, MASKED>(a, stream)
               : launch_mfma_nb<false, 128, false, MASKED>(a, stream);
}

hipError_t launch_attn_mfma(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  const bool masked = a.window > 0 || a.tree != nullptr;
  return masked ? launch_mfma_m<true>(a, bf16, H, paged, stream)
                : launch_mfma_m<false>(a, bf16, H, paged, stream);
}

}  // namespace kvc
