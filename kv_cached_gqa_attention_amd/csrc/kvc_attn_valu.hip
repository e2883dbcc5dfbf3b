// Split-KV attention on the vector ALUs, for units with few query rows
// (R = G * T <= 4 at head size 128, <= 8 at head size 64: single-token
// decode with small GQA groups, or short verify blocks of small groups).
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
//  * A workgroup owns a contiguous range of tiles; its four waves take
//    alternate tiles, so together they stream one contiguous window (worth
//    about 15% of bandwidth over four far-apart streams). At a unit boundary
//    the waves park their states in LDS, combine, and publish a partial; the
//    next unit's first tiles are requested before that, so the stream does
//    not drain at the boundary. Work is counted in steps of one tile per
//    wave, so the four waves always have equal work.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

// MASKED: a window or draft-tree mask is in use (the general per-key test);
// otherwise the causal test alone, which keeps the loop leaner.
template <bool BF, int H, int R, int LPR, bool PAGED, int WPE, bool MASKED>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attn_valu_kernel(AttnArgs a) {
  constexpr int DPL = H / LPR;         // dims per lane: 8 or 16
  constexpr int NCH = DPL / 8;         // 16-byte chunks per lane per row
  constexpr int GROUPS = 64 / LPR;     // rows per wave instruction
  constexpr int RPG = TILE / GROUPS;   // tokens per lane group per tile
  constexpr int SLICE = H / NCH;       // elements covered by one chunk across the group
  static_assert(DPL == 8 || DPL == 16, "8 or 16 dims per lane");

  extern __shared__ int32_t s_pre[];   // [2B + 1]
  __shared__ float s_m[WAVES * R], s_l[WAVES * R];
  __shared__ float s_o[WAVES * R * H];
  __shared__ float s_w[(WAVES + 2) * R];
  __shared__ int32_t s_wave[WAVES], s_bad[WAVES], s_flag[2];

  build_tile_prefix(a, s_pre, s_wave);
  fill_invalid<H>(a);
  const Partition part = make_partition(a, s_pre, blockIdx.x);
  append_owned<H, THREADS, PAGED>(a, s_pre, part);
  if (part.lo >= part.hi) return;  // the whole workgroup: no barrier is skipped

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int grp = lane / LPR;
  const int li = lane % LPR;
  const int lane_off = li * 16;  // byte offset of this lane's first 8 dims in a row
  const int bmask = (1 << a.block_shift) - 1;

  auto kbase = [&](const Segment& g) {
    return a.k + (int64_t)g.k * a.stride_head + (PAGED ? 0 : (int64_t)g.b * a.stride_seq);
  };
  auto vbase = [&](const Segment& g) {
    return a.v + (int64_t)g.k * a.stride_head + (PAGED ? 0 : (int64_t)g.b * a.stride_seq);
  };
  // Byte offset of token `tok` of sequence g.b (clamped to its last valid
  // row, and under a window to its first visible one); an out-of-range block
  // entry reads block 0 and flags the unit.
  auto row_off = [&](const Segment& g, int tok, bool& bad) -> int64_t {
    tok = min(tok, g.seq_len - 1);
    if constexpr (MASKED) tok = max(tok, first_visible(a, g.seq_len));
    if constexpr (PAGED) {
      int blk = a.table[(int64_t)g.b * a.max_blocks + (tok >> a.block_shift)];
      if ((unsigned)blk >= (unsigned)a.num_blocks) {
        bad = true;
        blk = 0;
      }
      return (int64_t)blk * a.stride_seq + (int64_t)(tok & bmask) * a.stride_tok + lane_off;
    } else {
      return (int64_t)tok * a.stride_tok + lane_off;
    }
  };
  auto load_rows = [&](const char* base, const Segment& g, int tile, uint4 (&dst)[RPG][NCH],
                       bool& bad) {
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const char* p = base + row_off(g, tile * TILE + grp + GROUPS * i, bad);
#pragma unroll
      for (int c = 0; c < NCH; ++c) dst[i][c] = load16(p + c * SLICE * 2);
    }
  };
  Segment cur = find_segment(a, s_pre, part, part.lo);
  int64_t x_next = part.lo + (cur.t_end - cur.t_begin);

  // A unit's query rows, this lane's dims. They are loaded again with every
  // K prefetch (the rows of the unit the prefetched tile belongs to; they
  // stay in L1), so the query loads are never newer than the tile loads and
  // waiting for them never waits for a tile prefetch. At a unit switch this
  // brings in the next unit's rows during the publish of the current one.
  uint4 qreg[R][NCH];
  auto load_q = [&](const Segment& g) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const char* qrow = a.q + row_index(a, g.b, g.k, r) * (H * 2);
#pragma unroll
      for (int c = 0; c < NCH; ++c) qreg[r][c] = load16(qrow + c * SLICE * 2 + li * 16);
    }
  };
  load_q(cur);
  bool bad_cur = false, bad_nxt = false;
  uint4 kr[RPG][NCH], vr[RPG][NCH];
  load_rows(kbase(cur), cur, cur.t_begin * WAVES + wave, kr, bad_cur);
  __builtin_amdgcn_sched_barrier(0);
  load_rows(vbase(cur), cur, cur.t_begin * WAVES + wave, vr, bad_cur);
  __builtin_amdgcn_sched_barrier(0);

  SharedUnits shared;
  while (true) {
    const bool has_next = x_next < part.hi;
    const Segment nxt = has_next ? find_segment(a, s_pre, part, x_next) : cur;
    // Row r = t * G + g is new token t. Tiles wholly inside [mask_lo,
    // mask_hi) are visible to every row; others take the per-key test
    // (causal or tree rule among the new rows, window at the start).
    const int new0 = cur.seq_len - a.T;
    const int mask_hi = MASKED && a.tree ? new0 : new0 + 1;
    const int mask_lo = MASKED && a.window > 0 ? cur.seq_len - a.window : INT_MIN;
    uint32_t tword[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      tword[r] = MASKED && a.tree ? a.tree[(int64_t)cur.b * a.T + r / a.G] : 0u;

    float m[R], l[R], o[R][DPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      m[r] = NEG_BIG;
      l[r] = 0.f;
#pragma unroll
      for (int d = 0; d < DPL; ++d) o[r][d] = 0.f;
    }
    for (int st = cur.t_begin; st < cur.t_end; ++st) {
      const int ti = st * WAVES + wave;  // this wave's tile of step st
      // ---- scores (base 2)
      float sc[R][RPG];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint4 q4[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) q4[c] = qreg[r][c];
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            acc = dot2<BF>(kr[i][c].x, q4[c].x, acc);
            acc = dot2<BF>(kr[i][c].y, q4[c].y, acc);
            acc = dot2<BF>(kr[i][c].z, q4[c].z, acc);
            acc = dot2<BF>(kr[i][c].w, q4[c].w, acc);
          }
          sc[r][i] = acc;
        }
      }
      // ---- this wave's next tile: in the next step of this unit, else in
      // the next unit's first step, else this tile again (cached). Loads are
      // unconditional: a conditional load costs register copies.
      const bool hop = has_next && st + 1 == cur.t_end;
      const Segment& ng = hop ? nxt : cur;
      const int tn = (hop ? nxt.t_begin : min(st + 1, cur.t_end - 1)) * WAVES + wave;
      const char* nkb = hop ? kbase(nxt) : kbase(cur);
      const char* nvb = hop ? vbase(nxt) : vbase(cur);
      bool nbad = false;
      load_q(ng);
      load_rows(nkb, ng, tn, kr, nbad);
#pragma unroll
      for (int i = 0; i < RPG; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r][i] = group_sum<LPR>(sc[r][i]) * a.scale_log2;

      // ---- mask (only a unit's first and last tiles)
      const int tok0 = ti * TILE;
      if (tok0 + TILE > mask_hi || tok0 < mask_lo) {
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          const int tok = tok0 + grp + GROUPS * i;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const bool ok = MASKED ? key_visible(a, tok, new0, r / a.G, tword[r])
                                   : tok <= new0 + r / a.G;
            if (!ok) sc[r][i] = -__builtin_inff();
          }
        }
      }

      // ---- online softmax; the rescale runs only when some row's max grew
      // past the margin
      float mn[R];
      bool grew = false;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float mt = sc[r][0];
#pragma unroll
        for (int i = 1; i < RPG; ++i) mt = fmaxf(mt, sc[r][i]);
        const bool up = mt > m[r] + RESCALE_MARGIN;
        mn[r] = up ? mt : m[r];
        grew |= up;
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
      load_rows(nvb, ng, tn, vr, nbad);
      if (hop) bad_nxt |= nbad; else bad_cur |= nbad;
    }

    // ---- combine this wave's lane groups, park the wave's state in LDS
#pragma unroll
    for (int r = 0; r < R; ++r) {
      static_assert(LPR == 8, "lane groups of 8: the reductions run over 8 groups");
      const float mr = max_groups8(m[r]);
      const float scl = __builtin_amdgcn_exp2f(m[r] - mr);
      const float lr = sum_groups8(l[r] * scl);
#pragma unroll
      for (int d = 0; d < DPL; ++d) o[r][d] = sum_groups8(o[r][d] * scl);
      // lane group g parks rows g, g + GROUPS, ...
      if (r % GROUPS == grp) {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) s_o[(wave * R + r) * H + c * SLICE + li * 8 + e] = o[r][c * 8 + e];
      }
      if (lane == 0) {
        s_m[wave * R + r] = mr;
        s_l[wave * R + r] = lr;
      }
    }
    {
      const unsigned long long anybad = __builtin_amdgcn_ballot_w64(bad_cur);
      if (lane == 0) s_bad[wave] = anybad != 0ull;
    }
    __syncthreads();
    bool segbad = false;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) segbad |= s_bad[w] != 0;
    // The next unit's first tiles are in flight while the workgroup combines
    // and writes this one.
    finish_segment<H, WAVES>(a, cur, blockIdx.x, s_m, s_l, s_o, s_w, segbad, shared);

    if (!has_next) break;
    cur = nxt;
    x_next += nxt.t_end - nxt.t_begin;
    bad_cur = bad_nxt;
    bad_nxt = false;
  }
  count_and_merge<H>(a, shared, s_flag);
}

// ---------------------------------------------------------------- launch

template <bool BF, int H, int R, bool PAGED, bool MASKED>
static hipError_t launch_valu_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int LPR = 8;
  // Two waves per SIMD (at most 256 registers per lane) wherever the loop
  // fits without spilling: every shape except H = 128 with more than four
  // rows, which goes to the matrix cores anyway.
  constexpr int WPE = (H == 128 && R <= 4) || H == 64 ? 2 : 1;
  const size_t shmem = (size_t)(2 * a.B + 1) * sizeof(int32_t);
  // one worker per workgroup; its waves interleave the tiles
  hipLaunchKernelGGL((attn_valu_kernel<BF, H, R, LPR, PAGED, WPE, MASKED>), dim3(a.W), dim3(THREADS),
                     shmem, stream, a);
  return hipGetLastError();
}

template <bool BF, int H, bool PAGED, bool MASKED>
static hipError_t launch_valu_r(const AttnArgs& a, hipStream_t stream) {
  switch (a.R) {
    case 1: return launch_valu_t<BF, H, 1, PAGED, MASKED>(a, stream);
    case 2: return launch_valu_t<BF, H, 2, PAGED, MASKED>(a, stream);
    case 3: return launch_valu_t<BF, H, 3, PAGED, MASKED>(a, stream);
    case 4: return launch_valu_t<BF, H, 4, PAGED, MASKED>(a, stream);
    default: break;
  }
  if constexpr (H == 64) {
    switch (a.R) {
      case 5: return launch_valu_t<BF, H, 5, PAGED, MASKED>(a, stream);
      case 6: return launch_valu_t<BF, H, 6, PAGED, MASKED>(a, stream);
      case 7: return launch_valu_t<BF, H, 7, PAGED, MASKED>(a, stream);
      case 8: return launch_valu_t<BF, H, 8, PAGED, MASKED>(a, stream);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <bool MASKED>
static hipError_t launch_valu_m(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  if (bf16) {
    if (H == 64)
      return paged ? launch_valu_r<true, 64, true, MASKED>(a, stream)
                   : launch_valu_r<true, 64, false, MASKED>(a, stream);
    return paged ? launch_valu_r<true, 128, true, MASKED>(a, stream)
                 : launch_valu_r<true, 128, false, MASKED>(a, stream);
  }
  if (H == 64)
    return paged ? launch_valu_r<false, 64, true, MASKED>(a, stream)
                 : launch_valu_r<false, 64, false, MASKED>(a, stream);
  return paged ? launch_valu_r<false, 128, true, MASKED>(a, stream)
               : launch_valu_r<false, 128, false, MASKED>(a, stream);
}

hipError_t launch_attn_valu(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  const bool masked = a.window > 0 || a.tree != nullptr;
  return masked ? launch_valu_m<true>(a, bf16, H, paged, stream)
                : launch_valu_m<false>(a, bf16, H, paged, stream);
}

}  // namespace kvc
