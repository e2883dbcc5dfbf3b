// Split-KV attention on the vector ALUs, for units with few query rows
// (R = G * T <= 8: single-token decode with GQA groups up to 8, or short
// verify blocks of small groups).
//
// What it computes is the cached attention of "Making inference cheap: KV
// cache, batching and quantization" (the new token's query against every
// stored key, one 1 x n score row) with grouped heads ("CS336, lectures 10
// and 12", section "Reducing the KV cache"). Decode attention moves about one
// byte per flop ("Arithmetic intensity of inference": intensity S/(S+1) < 1
// without grouping, G * T flop per byte with it), so the kernel is built to
// stream K and V once at full HBM rate:
//
//  * A row of K (or V) is H 16-bit values. LPR lanes share one row, each
//    holding DPL = H / LPR dims as 16-byte loads, so one wave instruction
//    reads 64 / LPR whole rows (full 128-byte lines).
//  * Every lane keeps all R query rows of the unit in registers (packed
//    16-bit pairs), so each K/V row fetched from HBM is used by all G heads
//    of its group (and all T block tokens) straight from registers.
//  * q.k uses v_dot2_f32_{bf16,f16}: two 16-bit products accumulated in fp32
//    per instruction, no conversion; the LPR partial sums are reduced with
//    DPP row operations.
//  * Softmax is the online form in fp32, per lane group; the p.v update
//    widens V to fp32 (exact) and accumulates in fp32.
//  * Loads are software-pipelined: the next tile's K is requested right
//    after the current q.k, its V right after the current p.v.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

template <bool BF, int H, int R, int LPR, bool PAGED>
__global__ __launch_bounds__(THREADS) void attn_valu_kernel(AttnArgs a) {
  constexpr int DPL = H / LPR;         // dims per lane: 8 or 16
  constexpr int NCH = DPL / 8;         // 16-byte chunks per lane per row
  constexpr int NW32 = DPL / 2;        // packed 32-bit words per lane per row
  constexpr int GROUPS = 64 / LPR;     // rows per wave instruction
  constexpr int RPG = TILE / GROUPS;   // tokens per lane group per tile
  constexpr int SLICE = H / NCH;       // elements covered by one chunk across the group
  static_assert(DPL == 8 || DPL == 16, "8 or 16 dims per lane");

  extern __shared__ int32_t s_pre[];   // [B + 1]
  __shared__ float s_m[WAVES * R], s_l[WAVES * R];
  __shared__ float s_o[WAVES * R * H];
  __shared__ int32_t s_wave[WAVES], s_bad[WAVES], s_flag[1];

  build_tile_prefix(a, s_pre, s_wave);
  fill_invalid<H>(a);
  const Partition part = make_partition(a, s_pre);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / LPR;
  const int li = lane % LPR;

  for (int64_t x = part.lo; x < part.hi;) {
    const Segment s = find_segment(a, s_pre, part, x);
    x += s.t_end - s.t_begin;

    // Query rows of the unit, packed, this lane's dims.
    uint32_t qp[R][NW32];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const char* qrow = a.q + row_index(a, s.b, s.k, r) * (H * 2);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4 v = load16(qrow + c * SLICE * 2 + li * 16);
        qp[r][c * 4 + 0] = v.x;
        qp[r][c * 4 + 1] = v.y;
        qp[r][c * 4 + 2] = v.z;
        qp[r][c * 4 + 3] = v.w;
      }
    }
    // Row r = t * G + g sees keys j < seq_len - T + t + 1; only tiles that
    // reach past vis_min need the mask.
    const int vis_min = s.seq_len - a.T + 1;

    const char* kb = a.k + (int64_t)s.k * a.stride_head + (PAGED ? 0 : (int64_t)s.b * a.stride_seq);
    const char* vb = a.v + (int64_t)s.k * a.stride_head + (PAGED ? 0 : (int64_t)s.b * a.stride_seq);
    const int32_t* trow = PAGED ? a.table + (int64_t)s.b * a.max_blocks : nullptr;
    const int bmask = (1 << a.block_shift) - 1;
    const int lane_off = li * 16;  // byte offset of this lane's first 8 dims
    bool bad = false;

    // Byte offset of token `tok` (clamped to the last valid row) within head k.
    auto row_off = [&](int tok) -> int64_t {
      tok = min(tok, s.seq_len - 1);
      if constexpr (PAGED) {
        int blk = trow[tok >> a.block_shift];
        if ((unsigned)blk >= (unsigned)a.num_blocks) {
          bad = true;
          blk = 0;
        }
        return (int64_t)blk * a.stride_seq + (int64_t)(tok & bmask) * a.stride_tok + lane_off;
      } else {
        return (int64_t)tok * a.stride_tok + lane_off;
      }
    };
    auto load_rows = [&](const char* base, int tile, uint4 (&dst)[RPG][NCH]) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const char* p = base + row_off(tile * TILE + grp + GROUPS * i);
#pragma unroll
        for (int c = 0; c < NCH; ++c) dst[i][c] = load16(p + c * SLICE * 2);
      }
    };

    float m[R], l[R], o[R][DPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      m[r] = NEG_BIG;
      l[r] = 0.f;
#pragma unroll
      for (int d = 0; d < DPL; ++d) o[r][d] = 0.f;
    }

    // First tile: issued unconditionally (a wave without tiles in this
    // segment re-reads its last one and never uses it) and in the loop's
    // order, all K rows then all V rows, so that every path into the loop
    // leaves the same loads in flight and q.k waits only for K.
    uint4 kr[RPG][NCH], vr[RPG][NCH];
    int ti = s.t_begin + wave;
    {
      const int t0 = min(ti, s.t_end - 1);
      load_rows(kb, t0, kr);
      __builtin_amdgcn_sched_barrier(0);
      load_rows(vb, t0, vr);
      __builtin_amdgcn_sched_barrier(0);
    }

    for (; ti < s.t_end; ti += WAVES) {
      // ---- scores (base 2)
      float sc[R][RPG];
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            acc = dot2<BF>(kr[i][c].x, qp[r][c * 4 + 0], acc);
            acc = dot2<BF>(kr[i][c].y, qp[r][c * 4 + 1], acc);
            acc = dot2<BF>(kr[i][c].z, qp[r][c * 4 + 2], acc);
            acc = dot2<BF>(kr[i][c].w, qp[r][c * 4 + 3], acc);
          }
          sc[r][i] = acc;
        }
      }
      // ---- next tile's K goes out as soon as this tile's K is consumed.
      // The prefetch is unconditional (no register copies for a conditional
      // load); past the segment it re-reads the segment's last tile, which
      // this workgroup has just brought into the cache.
      const int tn = min(ti + WAVES, s.t_end - 1);
      load_rows(kb, tn, kr);
#pragma unroll
      for (int i = 0; i < RPG; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r][i] = group_sum<LPR>(sc[r][i]) * a.scale_log2;

      // ---- causal / length mask (only the last tiles of a sequence)
      const int tok0 = ti * TILE;
      if (tok0 + TILE > vis_min) {
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          const int tok = tok0 + grp + GROUPS * i;
#pragma unroll
          for (int r = 0; r < R; ++r)
            if (tok >= vis_min + r / a.G) sc[r][i] = -__builtin_inff();
        }
      }

      // ---- online softmax; the rescale runs only when some row's max grew
      float mn[R];
      bool grew = false;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float mt = sc[r][0];
#pragma unroll
        for (int i = 1; i < RPG; ++i) mt = fmaxf(mt, sc[r][i]);
        mn[r] = fmaxf(m[r], mt);
        grew |= mn[r] > m[r];
      }
      if (__builtin_amdgcn_ballot_w64(grew) != 0ull) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float alpha = __builtin_amdgcn_exp2f(m[r] - mn[r]);
          l[r] *= alpha;
#pragma unroll
          for (int d = 0; d < DPL; ++d) o[r][d] *= alpha;
          m[r] = mn[r];
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          const float p = __builtin_amdgcn_exp2f(sc[r][i] - m[r]);
          sc[r][i] = p;
          l[r] += p;
        }
      }

      // ---- p.v
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint32_t w4[4] = {vr[i][c].x, vr[i][c].y, vr[i][c].z, vr[i][c].w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float v0 = lo_f<BF>(w4[w]);
            const float v1 = hi_f<BF>(w4[w]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              o[r][c * 8 + 2 * w] = fmaf(sc[r][i], v0, o[r][c * 8 + 2 * w]);
              o[r][c * 8 + 2 * w + 1] = fmaf(sc[r][i], v1, o[r][c * 8 + 2 * w + 1]);
            }
          }
        }
      }
      // ---- next tile's V
      load_rows(vb, tn, vr);
    }

    // ---- combine the lane groups of this wave
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float M = m[r];
#pragma unroll
      for (int msk = LPR; msk < 64; msk <<= 1) M = fmaxf(M, shfl_xor_f(M, msk));
      const float scl = __builtin_amdgcn_exp2f(m[r] - M);
      float L = l[r] * scl;
#pragma unroll
      for (int msk = LPR; msk < 64; msk <<= 1) L += shfl_xor_f(L, msk);
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        float od = o[r][d] * scl;
#pragma unroll
        for (int msk = LPR; msk < 64; msk <<= 1) od += shfl_xor_f(od, msk);
        o[r][d] = od;
      }
      if (grp == 0) {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) s_o[(wave * R + r) * H + c * SLICE + li * 8 + e] = o[r][c * 8 + e];
      }
      if (lane == 0) {
        s_m[wave * R + r] = M;
        s_l[wave * R + r] = L;
      }
    }
    {
      const unsigned long long anybad = __ballot(bad);
      if (lane == 0) s_bad[wave] = anybad != 0ull;
    }
    __syncthreads();
    bool segbad = false;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) segbad |= s_bad[w] != 0;
    finish_segment<H, WAVES>(a, s, s_m, s_l, s_o, segbad, s_flag);
  }
}

// ---------------------------------------------------------------- launch

template <bool BF, int H, int R, bool PAGED>
static hipError_t launch_valu_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int LPR = (H == 64) ? 8 : (R <= 4 ? 8 : 16);
  const size_t shmem = (size_t)(a.B + 1) * sizeof(int32_t);
  hipLaunchKernelGGL((attn_valu_kernel<BF, H, R, LPR, PAGED>), dim3(a.W), dim3(THREADS), shmem,
                     stream, a);
  return hipGetLastError();
}

template <bool BF, int H, bool PAGED>
static hipError_t launch_valu_r(const AttnArgs& a, hipStream_t stream) {
  switch (a.R) {
    case 1: return launch_valu_t<BF, H, 1, PAGED>(a, stream);
    case 2: return launch_valu_t<BF, H, 2, PAGED>(a, stream);
    case 3: return launch_valu_t<BF, H, 3, PAGED>(a, stream);
    case 4: return launch_valu_t<BF, H, 4, PAGED>(a, stream);
    case 5: return launch_valu_t<BF, H, 5, PAGED>(a, stream);
    case 6: return launch_valu_t<BF, H, 6, PAGED>(a, stream);
    case 7: return launch_valu_t<BF, H, 7, PAGED>(a, stream);
    case 8: return launch_valu_t<BF, H, 8, PAGED>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_valu(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  if (bf16) {
    if (H == 64) return paged ? launch_valu_r<true, 64, true>(a, stream) : launch_valu_r<true, 64, false>(a, stream);
    return paged ? launch_valu_r<true, 128, true>(a, stream) : launch_valu_r<true, 128, false>(a, stream);
  }
  if (H == 64) return paged ? launch_valu_r<false, 64, true>(a, stream) : launch_valu_r<false, 64, false>(a, stream);
  return paged ? launch_valu_r<false, 128, true>(a, stream) : launch_valu_r<false, 128, false>(a, stream);
}

}  // namespace kvc
