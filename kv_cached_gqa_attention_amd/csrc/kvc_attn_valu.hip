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
//  * Tiles go from HBM straight into LDS (kvc_dma.h): each wave owns two
//    slots, [K tile + the unit's query rows] and [V tile]. While it computes
//    on one, the other's next tile is in flight (the next step's K while it
//    works on V, and so on, across unit boundaries). Nothing in flight
//    occupies registers; two workgroups share a CU, so two waves share each
//    SIMD and one's LDS waits hide under the other's arithmetic.
//  * A row of K (or V) is H 16-bit values. LPR = 8 lanes share one row, each
//    reading DPL = H / 8 dims from LDS as 16-byte reads; rows of odd index
//    have their two halves swapped so the eight rows of one read hit
//    distinct banks.
//  * Every lane reads all R query rows of the unit, so each K/V row fetched
//    from HBM is used by all G heads of its group (and all T block tokens).
//  * q.k uses v_dot2_f32_{bf16,f16}: two 16-bit products accumulated in fp32
//    per instruction, no conversion; the LPR partial sums are reduced with
//    DPP row operations.
//  * Softmax is the online form in fp32, per lane group; the p.v update
//    widens V to fp32 (exact) and accumulates in fp32.
//  * A workgroup owns a contiguous range of steps; its four waves take
//    alternate tiles, so together they stream one contiguous window. At a
//    unit boundary the waves combine their states in LDS and publish the
//    unit's output or a partial, while the next unit's tiles are in flight.
#include "kvc_device.h"
#include "kvc_dma.h"
#include "kvc_internal.h"

namespace kvc {

// LDS bytes of a wave's two slots: [K tile, 1 KB of query rows], [V tile].
// (With the prefix table of up to ~470 sequences, two workgroups fit a CU.)
template <int H>
constexpr int valu_wave_bytes() { return 2 * TILE * H * 2 + 1024; }
template <int H>
constexpr int valu_ring_bytes() { return WAVES * valu_wave_bytes<H>(); }

// MASKED: a window or draft-tree mask is in use (the general per-key test);
// otherwise the causal test alone, which keeps the loop leaner.
template <bool BF, int H, int R, bool PAGED, bool MASKED>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_valu_kernel(AttnArgs a) {
  constexpr int LPR = 8;
  constexpr int DPL = H / LPR;         // dims per lane: 8 or 16
  constexpr int NCH = DPL / 8;         // 16-byte chunks per lane per row
  constexpr int GROUPS = 64 / LPR;     // rows per wave read
  constexpr int RPG = TILE / GROUPS;   // tokens per lane group per tile
  constexpr int SLICE = H / NCH;       // elements covered by one chunk across the group
  constexpr int ROWB = H * 2;
  constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
  constexpr int NI = TILE * CPR / 64;  // copy instructions per tile
  constexpr int TILEB = TILE * ROWB;
  constexpr int VSLOT = TILEB + 1024;  // the V slot's offset
  static_assert(DPL == 8 || DPL == 16, "8 or 16 dims per lane");
  static_assert(R * ROWB <= 1024, "the query rows fit one copy");

  extern __shared__ __attribute__((aligned(16))) int32_t s_pre[];  // [2B + 1], then the rings
  __shared__ float s_m[WAVES * R], s_l[WAVES * R];
  __shared__ float s_o[WAVES * R * H];
  __shared__ float s_w[(WAVES + 2) * R];
  __shared__ int32_t s_wave[WAVES], s_bad[WAVES], s_flag[2];

  build_tile_prefix(a, s_pre, s_wave);
  fill_invalid<H>(a, s_pre);
  const int worker = worker_of(a, blockIdx.x);
  const Partition part = make_partition<false>(a, s_pre, worker);
  append_owned<H, THREADS, PAGED>(a, s_pre, part);
  if (part.lo >= part.hi) return;  // the whole workgroup: no barrier is skipped

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int grp = lane / LPR;
  const int li = lane % LPR;
  char* ring = reinterpret_cast<char*>(s_pre) + prefix_bytes(a.B) + wave * valu_wave_bytes<H>();
  const uint32_t ring_lds = lds_addr(ring);

  // Swizzle of 16-byte chunk positions: odd rows swap their halves (H = 128).
  auto swz = [](int r) { return H == 128 ? (r & 1) << 3 : 0; };
  // This lane's LDS offsets of its chunks c of row grp (add ROWB * GROUPS * i
  // for row grp + GROUPS * i).
  int koff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) koff[c] = grp * ROWB + 16 * ((li + 8 * c) ^ swz(grp));

  // Copy issue: K half of step x = [K tile, query rows], V half = [V tile].
  uint32_t lvoff[NI];
  tile_lane_offsets<H>(a, lane, swz, lvoff);
  // the unit's R query rows, row-major after the K tile: this lane's 16 bytes
  uint32_t qoff;
  {
    const int rq = min(lane * 16 / ROWB, R - 1);
    const int t = rq / a.G;
    qoff = (uint32_t)(((int64_t)t * a.N + (rq - t * a.G)) * ROWB + (lane * 16) % ROWB);
  }
  // Bad-entry flags of the segment computed and of the next one (the copies
  // run one step ahead), indexed by segment ordinal parity.
  bool bad2[2] = {false, false};
  auto issue_k = [&](const StepCursor& c) __attribute__((always_inline)) {
    bool bad = false;
    copy_tile<H, PAGED, MASKED>(a, c.s, c.kb, c.tok0, ring_lds, lane, swz, lvoff, bad);
    dma16(a.q + row_index(a, c.s.b, c.s.k, 0) * ROWB, qoff, ring_lds + TILEB);
    bad2[c.ord & 1] |= bad;
  };
  auto issue_v = [&](const StepCursor& c) __attribute__((always_inline)) {
    bool bad = false;
    copy_tile<H, PAGED, MASKED>(a, c.s, c.vb, c.tok0, ring_lds + VSLOT, lane, swz, lvoff, bad);
    bad2[c.ord & 1] |= bad;
  };

  StepCursor cs, cn;  // the step computed, the next one (whose copies are issued)
  cs.begin(a, s_pre, part, part.lo, wave);
  cn = cs;
  issue_k(cn);
  issue_v(cn);
  cn.advance(a, s_pre, part);

  SharedUnits shared;
  Segment early;             // a unit whose early part was counted last
  bool early_merge = false;  // (uniform)
  while (true) {
    // ---- a new segment: its masks and state
    const Segment g = cs.s;
    const int new0 = g.seq_len - a.T;
    const int mask_hi = MASKED && a.tree ? new0 : new0 + 1;
    const int mask_lo = MASKED && a.window > 0 ? g.seq_len - a.window : INT_MIN;
    uint32_t tword[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      // (here T <= R <= 8: every new token's bit is in word 0 of its row)
      tword[r] = MASKED && a.tree ? load_uniform(a.tree, ((int64_t)g.b * a.T + r / a.G) * a.tree_words) : 0u;

    float m[R], l[R], o[R][DPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      m[r] = NEG_BIG;
      l[r] = 0.f;
#pragma unroll
      for (int d = 0; d < DPL; ++d) o[r][d] = 0.f;
    }
    for (;;) {
      const int64_t x = cs.x;
      const bool more = x + 1 < part.hi;
      // The two workgroups of a CU (i and i + W / 2 in an automatic grid)
      // take turns at the higher wave priority, step by step: the hardware
      // otherwise serves the older one first throughout.
      if ((x + (blockIdx.x >= gridDim.x / 2 ? 1 : 0)) & 1)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
      const char* kslot = ring;
      const char* vslot = ring + VSLOT;
      // ---- K half of step x: the one later copy is its V half
      wait_vm<NI>();
      uint4 qreg[R][NCH], kr[RPG][NCH];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          qreg[r][c] = *reinterpret_cast<const uint4*>(kslot + TILEB + r * ROWB + (c * SLICE + li * 8) * 2);
#pragma unroll
      for (int i = 0; i < RPG; ++i)
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          kr[i][c] = *reinterpret_cast<const uint4*>(kslot + koff[c] + i * GROUPS * ROWB);
      // ---- scores (base 2)
      float sc[R][RPG];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            acc = dot2<BF>(kr[i][c].x, qreg[r][c].x, acc);
            acc = dot2<BF>(kr[i][c].y, qreg[r][c].y, acc);
            acc = dot2<BF>(kr[i][c].z, qreg[r][c].z, acc);
            acc = dot2<BF>(kr[i][c].w, qreg[r][c].w, acc);
          }
          sc[r][i] = acc;
        }
      // ---- the K slot is free: the next step's K half goes there
      wait_lds();
      if (more) issue_k(cn);
      // the lane groups' sums, one reduction step over every score at a time
      // (the steps of one score depend on each other; those of different
      // scores do not)
#pragma unroll
      for (int i = 0; i < RPG; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r][i] += dpp_f<DPP_QUAD_XOR1>(sc[r][i]);
#pragma unroll
      for (int i = 0; i < RPG; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r][i] += dpp_f<DPP_QUAD_XOR2>(sc[r][i]);
#pragma unroll
      for (int i = 0; i < RPG; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r][i] = (sc[r][i] + dpp_f<DPP_ROW_HALF_MIRROR>(sc[r][i])) * a.scale_log2;

      // ---- mask (only a unit's first and last tiles; the empty asm keeps
      // the compiler from turning the branch into selects on every tile)
      const int tok0 = cs.tok0;
      if (tok0 + TILE > mask_hi || tok0 < mask_lo) {
        asm volatile("");
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

      // ---- V half of step x: later copies are the next step's K half
      if (more) wait_vm<NI + 1>(); else wait_vm<0>();
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint4 vr = *reinterpret_cast<const uint4*>(vslot + koff[c] + i * GROUPS * ROWB);
          const uint32_t w4[4] = {vr.x, vr.y, vr.z, vr.w};
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
      // ---- the V slot is free: the next step's V half goes there
      wait_lds();
      if (more) {
        issue_v(cn);
        cn.advance(a, s_pre, part);
      }
      if (x + 1 == cs.end) break;  // segment done (also at the range's end)
      cs.advance(a, s_pre, part);
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
      const bool bad = bad2[cs.ord & 1];
      bad2[cs.ord & 1] = false;
      const unsigned long long anybad = __builtin_amdgcn_ballot_w64(bad);
      if (lane == 0) s_bad[wave] = anybad != 0ull;
    }
    __syncthreads();
    bool segbad = false;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) segbad |= s_bad[w] != 0;
    if (g.n_parts > 1 && cs.ord == 0 && cs.x + 1 < part.hi) {
      // The range's first segment, not its last: the later steps of a unit
      // shared with the worker before, done early. Its partial is counted
      // now (the wait drains the next segment's copies in flight, once per
      // range), so that the worker holding the unit's first steps merges it;
      // if this count is the last (rare), the merge waits for the range's end.
      store_partial<H, WAVES>(a, g, worker, s_m, s_l, s_o, s_w, segbad);
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0) {
        const bool f = count_partial(a, g);
        if (f) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_flag[0] = f;
      }
      __syncthreads();
      if (s_flag[0]) {
        early_merge = true;
        early = g;
      }
    } else {
      finish_segment<H, WAVES>(a, g, worker, s_m, s_l, s_o, s_w, segbad, shared);
    }

    if (cs.x + 1 >= part.hi) break;
    cs.advance(a, s_pre, part);
  }
  // every copy has landed and every slot has been read: the slots are free
  __syncthreads();
  count_and_merge<H, (R * H + THREADS - 1) / THREADS>(a, shared, s_flag,
                     reinterpret_cast<float*>(reinterpret_cast<char*>(s_pre) + prefix_bytes(a.B)),
                     valu_ring_bytes<H>() / 4);
  if (early_merge)
    merge_partials<H, (R * H + THREADS - 1) / THREADS>(a, early,
                     reinterpret_cast<float*>(reinterpret_cast<char*>(s_pre) + prefix_bytes(a.B)),
                     valu_ring_bytes<H>() / 4);
}

// ---------------------------------------------------------------- launch

template <bool BF, int H, int R, bool PAGED, bool MASKED>
static hipError_t launch_valu_t(const AttnArgs& a, hipStream_t stream) {
  const auto kern = attn_valu_kernel<BF, H, R, PAGED, MASKED>;
  const size_t shmem = prefix_bytes(a.B) + valu_ring_bytes<H>();
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(prefix_bytes(4096) + valu_ring_bytes<H>()));
  if (attr != hipSuccess) return attr;
  // one worker per workgroup, one workgroup per CU; its waves interleave the tiles
  hipLaunchKernelGGL(kern, dim3(a.W), dim3(THREADS), shmem, stream, a);
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

int valu_workgroups_per_cu(int B, int H) {
  // static LDS (the waves' parked states, R * H <= 512 floats each, and
  // under 1 KB of row statistics and flags) + prefix table + slots, against
  // 160 KB
  constexpr size_t LDS_PER_CU = 160 * 1024;
  const size_t stat = (size_t)WAVES * 512 * 4 + 1024;
  const size_t per_wg = stat + prefix_bytes(B) + (H == 64 ? valu_ring_bytes<64>() : valu_ring_bytes<128>());
  return per_wg * 2 <= LDS_PER_CU ? 2 : 1;
}

hipError_t launch_attn_valu(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  const bool masked = a.window > 0 || a.tree != nullptr;
  return masked ? launch_valu_m<true>(a, bf16, H, paged, stream)
                : launch_valu_m<false>(a, bf16, H, paged, stream);
}

}  // namespace kvc
