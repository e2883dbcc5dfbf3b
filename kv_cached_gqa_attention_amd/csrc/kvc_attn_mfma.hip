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
// token-to-k-slot map is chosen to make that true).
//
// K and V tiles go from HBM straight into LDS (kvc_dma.h): each wave runs a
// ring of two or three tile slots (three when the workgroup's LDS allows),
// K and V tiles alternating, and keeps all but one slot in flight while it
// computes on the other, across unit boundaries. The slots' 16-byte chunks
// are XOR-swizzled per row so that the A-operand reads are free of bank
// conflicts: K rows are read 16 bytes per lane (one row per lane of a
// 16-lane group), and V^T comes from ds_read_b64_tr_b16, which hands each
// lane 4 tokens of one h (the transpose the V^T operand needs) from 8-byte
// pieces of 4 rows.
// p is split into a 16-bit high part and a 16-bit remainder, each multiplied
// by V on the matrix cores, so p.v keeps about 16 bits of p (within 2^-16
// relative, far inside the 2e-3 gate).
#include "kvc_device.h"
#include "kvc_dma.h"
#include "kvc_internal.h"
#include "kvc_mfma.h"

namespace kvc {

// LDS bytes of one staging slot (a K or V tile).
template <int H>
constexpr int mfma_tile_bytes() { return TILE * H * 2; }

// MASKED: a window or draft-tree mask is in use (the general per-key test);
// otherwise the causal test alone. nslots: staging slots per wave (2 or 3).
// One workgroup per CU (one wave per SIMD): the query rows stay in registers
// for a whole segment and the copies run on across unit boundaries. (A form
// with two workgroups per CU, the query rows in LDS and the copies stopping
// at each unit boundary, measured 1-4% slower on every verify shape.)
// Each unit a workgroup enters costs it a fold, a partial and a count, so the
// shares of the steps count a few virtual steps per unit (make_partition<true>):
// a workgroup whose range enters more units gets fewer steps.
template <bool BF, int H, int NB, bool PAGED, bool MASKED>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma_kernel(AttnArgs a, int nslots) {
  constexpr int RMAX = NB * 16;  // query rows per unit (row block)
  // Row stride (floats) of the waves' fold in LDS: H + 4 puts the 16 query
  // rows one fold write touches (one per lane of a 16-lane group) in
  // distinct banks (a stride of H sent all 16 to one bank).
  constexpr int OST = H + 4;
  constexpr int KS = H / 32;     // k-steps of S^T over h
  constexpr int MH = H / 16;     // 16-row h blocks of O^T
  constexpr int ROWB = H * 2;
  constexpr int NI = TILE * ROWB / 1024;  // copy instructions per tile
  constexpr int TILEB = mfma_tile_bytes<H>();

  // [2B + 1], then the slots
  extern __shared__ __attribute__((aligned(16))) int32_t s_pre[];
  __shared__ float s_m[RMAX], s_l[RMAX];
  __shared__ float s_o[RMAX * OST];  // the waves' fold
  __shared__ int32_t s_wave[WAVES], s_bad[WAVES], s_flag[2];

  build_tile_prefix(a, s_pre, s_wave);
  fill_invalid<H>(a, s_pre);
  // one workgroup per CU in launch order: equal shares, worker = workgroup
  const int worker = blockIdx.x;
  const Partition part = make_partition<true>(a, s_pre, worker);
  append_owned<H, THREADS, PAGED>(a, s_pre, part);
  if (part.lo >= part.hi) return;  // the whole workgroup: no barrier is skipped

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int c = lane & 15;   // column (query row) / A-row (token or h) within a 16 block
  const int g = lane >> 4;   // k-slot group
  char* ring_all = reinterpret_cast<char*>(s_pre) + prefix_bytes(a.B);
  char* ring = ring_all + wave * nslots * TILEB;
  const uint32_t ring_lds = lds_addr(ring);
  const lds_char* ring3 = (const lds_char*)ring;

  // Chunk swizzles (16-byte chunk j of row r sits at position j ^ swz(r)):
  // K: the 16 rows one A-operand read touches at one column fall in 16
  // distinct bank groups; V: the 8 rows x 2 chunks of one transposed read of
  // 32 lanes do.
  auto swz_k = [](int r) { return H == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto swz_v = [](int r) { return H == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };
  uint32_t lvk[NI], lvv[NI];
  tile_lane_offsets<H>(a, lane, swz_k, lvk);
  tile_lane_offsets<H>(a, lane, swz_v, lvv);
  // A operand of S^T: K row 16 mb + c, dims 32 ks + 8 g .. + 7 (chunk 4 ks + g);
  // swz_k(16 mb + c) == swz_k(c).
  uint32_t koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = c * ROWB + 16 * ((4 * ks + g) ^ swz_k(c));
  // A operand of O^T += V^T . P^T, k-slot (g, j) = token 4 g + j (j < 4) or
  // 16 + 4 g + j - 4: two transposed reads per 16-h block, lane 4 a + b of
  // group g addressing row 4 g + a (then + 16), dims 16 mh + 4 b .. + 3;
  // swz_v(r + 16) == swz_v(r).
  uint32_t voff[MH];
  {
    const int r = 4 * g + (c >> 2);
    const int b = c & 3;
#pragma unroll
    for (int mh = 0; mh < MH; ++mh)
      voff[mh] = r * ROWB + 16 * ((2 * mh + (b >> 1)) ^ swz_v(r)) + 8 * (b & 1);
  }

  // ---- copies: halves K(x), V(x) of steps x = lo, lo + 1, ... in slot order
  int nhalves = (int)(2 * (part.hi - part.lo));
  int hp = 0;         // halves issued
  int pslot = 0;      // slot of the next one
  bool pv = false;    // next one is a V half
  int bad_bits = 0;   // bad block entries, by segment ordinal mod 4
  StepCursor pc;
  pc.begin(a, s_pre, part, part.lo, wave);
  auto issue_next = [&]() __attribute__((always_inline)) {
    const uint32_t dst = ring_lds + pslot * TILEB;
    bool bad = false;
    if (!pv) {
      copy_tile<H, PAGED, MASKED>(a, pc.s, pc.kb, pc.tok0, dst, lane, swz_k, lvk, bad);
    } else {
      copy_tile<H, PAGED, MASKED>(a, pc.s, pc.vb, pc.tok0, dst, lane, swz_v, lvv, bad);
    }
    bad_bits |= (bad ? 1 : 0) << (pc.ord & 3);
    if (pv) pc.advance(a, s_pre, part);
    pv = !pv;
    ++hp;
    pslot = pslot + 1 == nslots ? 0 : pslot + 1;
  };
  auto prologue = [&]() __attribute__((always_inline)) {
    for (int i = 0; i < nslots && hp < nhalves; ++i) issue_next();
  };
  prologue();
  int hc = 0;      // halves consumed
  int cslot = 0;   // slot of the next one
  // Wait for half hc + ahead: the halves issued after it are in flight (at
  // most 2).
  auto wait_half = [&](int ahead) __attribute__((always_inline)) {
    const int later = hp - 1 - hc - ahead;
    if (later >= 2) wait_vm<2 * NI>(); else if (later == 1) wait_vm<NI>(); else wait_vm<0>();
  };
  auto release_half = [&]() __attribute__((always_inline)) {
    wait_lds();  // its reads have returned: the slot can be refilled
    if (hp < nhalves) issue_next();
    ++hc;
    cslot = cslot + 1 == nslots ? 0 : cslot + 1;
  };

  // A operand of S^T for the next tile, read from LDS a tile ahead (while
  // the previous tile's p.v products run)
  uint4 kf[2][KS];
  auto read_k = [&](int ahead) __attribute__((always_inline)) {  // K tile of half hc + ahead
    wait_half(ahead);
    const int slot = cslot + ahead >= nslots ? cslot + ahead - nslots : cslot + ahead;
    const char* kt = ring + slot * TILEB;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[mb][ks] = *reinterpret_cast<const uint4*>(kt + koff[ks] + mb * 16 * ROWB);
  };
  read_k(0);

  StepCursor cs;
  cs.begin(a, s_pre, part, part.lo, wave);
  SharedUnits shared;
  Segment early;             // a unit whose early part was counted last
  bool early_merge = false;  // (uniform)
  while (true) {
    const Segment s = cs.s;
    // Q^T fragments (B operand): query row rb*RMAX + 16 nb + c, h = 32 ks + 8 g + j.
    uint4 qf[NB][KS];
    int tq[NB];         // new-token index of this lane's query column
    // its tree-mask row: T <= RMAX <= 64 new tokens, so at most two words
    uint32_t tw[NB], tw1[NB];
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
      const uint32_t* trow = MASKED && a.tree ? a.tree + ((int64_t)s.b * a.T + tq[nb]) * a.tree_words : nullptr;
      tw[nb] = trow ? trow[0] : 0u;
      tw1[nb] = trow && a.tree_words > 1 ? trow[1] : 0u;
    }
    // Every outstanding load (these and the copies in flight) has landed,
    // so no wait for the query loads falls inside the tile loop.
    wait_stores();

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
    const int new0 = s.seq_len - a.T;

    for (;;) {
      // ---- S^T = K . Q^T (K was read a tile ahead)
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
      release_half();

      // ---- scale, mask, online softmax (one query row per lane column)
      const int tok0 = cs.tok0;
      // tiles wholly inside [new0 + 1 (new0 with a tree), seq_len - window)
      // are visible to every query
      const bool edge = tok0 + TILE > (MASKED && a.tree ? new0 : new0 + 1) ||
                        (MASKED && a.window > 0 && tok0 < s.seq_len - a.window);
      // All column blocks at once (independent chains side by side), one
      // wave-uniform decision whether any running max moves.
      float p[NB][2][4], mt[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = st[mb][nb][i] * a.scale_log2;
            const int tok = tok0 + mb * 16 + 4 * g + i;
            if (edge && !(MASKED ? key_visible(a, tok, new0, tq[nb], tok - new0 >= 32 ? tw1[nb] : tw[nb])
                                 : tok <= new0 + tq[nb]))
              v = -__builtin_inff();
            p[nb][mb][i] = v;
          }
        mt[nb] = fmaxf(fmaxf(fmaxf(p[nb][0][0], p[nb][0][1]), fmaxf(p[nb][0][2], p[nb][0][3])),
                       fmaxf(fmaxf(p[nb][1][0], p[nb][1][1]), fmaxf(p[nb][1][2], p[nb][1][3])));
      }
      bool grow = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        mt[nb] = max_cols4(mt[nb]);
        grow |= mt[nb] > m[nb] + RESCALE_MARGIN;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float mn = mt[nb] > m[nb] + RESCALE_MARGIN ? mt[nb] : m[nb];
          const float alpha = __builtin_amdgcn_exp2f(m[nb] - mn);  // 1 where unchanged
          l[nb] *= alpha;
#pragma unroll
          for (int mh = 0; mh < MH; ++mh) ot[mh][nb] *= alpha;
          m[nb] = mn;
        }
      }
      uint4 phi[NB], plo[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float e0 = __builtin_amdgcn_exp2f(p[nb][mb][i] - m[nb]);
            const float e1 = __builtin_amdgcn_exp2f(p[nb][mb][i + 1] - m[nb]);
            l[nb] += e0 + e1;
            split_pair<BF>(e0, e1, hw[mb * 2 + i / 2], lw[mb * 2 + i / 2]);
          }
        phi[nb] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        plo[nb] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
      // ---- V^T of this tile, and the next tile's K, possibly of the next
      // unit, read before the p.v products
      wait_half(0);
      const lds_char* vt_base = ring3 + cslot * TILEB;
      auto read_v = [&](int mh) __attribute__((always_inline)) {
        const uint2 lo4 = read_tr16(vt_base + voff[mh]);
        const uint2 hi4 = read_tr16(vt_base + voff[mh] + 16 * ROWB);
        return make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
      };
      uint4 vt[MH];
#pragma unroll
      for (int mh = 0; mh < MH; ++mh) vt[mh] = read_v(mh);
      if (cs.x + 1 < part.hi) read_k(1);

      // ---- O^T += V^T . P^T
#pragma unroll
      for (int mh = 0; mh < MH; ++mh) {
        const uint4 v = vt[mh];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          ot[mh][nb] = mfma16<BF>(v, phi[nb], ot[mh][nb]);
          ot[mh][nb] = mfma16<BF>(v, plo[nb], ot[mh][nb]);
        }
      }
      release_half();  // the V slot: the products have their operands
      if (cs.x + 1 == cs.end) break;  // segment done (also at the range's end)
      cs.advance(a, s_pre, part);
    }

    // ---- per-column totals of l (lanes of one column hold different tokens)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      l[nb] = sum_cols4(l[nb]);
    }
    {
      const bool bad = (bad_bits >> (cs.ord & 3)) & 1;
      bad_bits &= ~(1 << (cs.ord & 3));
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
              float* dst = &s_o[col * OST + mh * 16 + 4 * g + i];
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
    if (s.n_parts > 1 && cs.ord == 0 && cs.x + 1 < part.hi) {
      // The range's first segment, not its last: the later steps of a unit
      // shared with the worker before, done early. Its partial is counted
      // now, so that the worker holding the unit's first steps (done last)
      // merges it; if this count is the last (rare), the merge waits for the
      // range's end.
      store_partial<H, 1, OST>(a, s, worker, s_m, s_l, s_o, s_m, segbad);
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0) {
        const bool f = count_partial(a, s);
        if (f) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_flag[0] = f;
      }
      __syncthreads();
      if (s_flag[0]) {
        early_merge = true;
        early = s;
      }
    } else {
      finish_segment<H, 1, OST>(a, s, worker, s_m, s_l, s_o, s_m, segbad, shared);
    }
    if (cs.x + 1 >= part.hi) break;
    cs.advance(a, s_pre, part);
  }
  // every copy has landed and every slot has been read: the slots are free
  __syncthreads();
  count_and_merge<H, (RMAX * H + THREADS - 1) / THREADS>(a, shared, s_flag, reinterpret_cast<float*>(ring_all),
                     WAVES * nslots * TILEB / 4);
  if (early_merge)
    merge_partials<H, (RMAX * H + THREADS - 1) / THREADS>(a, early, reinterpret_cast<float*>(ring_all),
                                                          WAVES * nslots * TILEB / 4);
}

// ---------------------------------------------------------------- launch

template <bool BF, int H, int NB, bool PAGED, bool MASKED>
static hipError_t launch_mfma_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int LDS_PER_CU = 160 * 1024;
  const auto kern = attn_mfma_kernel<BF, H, NB, PAGED, MASKED>;
  static size_t static_lds = 0;
  static const hipError_t attr = [&] {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, (const void*)kern);
    if (e != hipSuccess) return e;
    static_lds = fa.sharedSizeBytes;
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)(LDS_PER_CU - static_lds));
  }();
  if (attr != hipSuccess) return attr;
  const size_t pre = prefix_bytes(a.B);
  // three slots per wave where the LDS allows (the prefix table grows with B)
  const size_t slots3 = (size_t)WAVES * 3 * mfma_tile_bytes<H>();
  const int nslots = static_lds + pre + slots3 <= (size_t)LDS_PER_CU ? 3 : 2;
  const size_t shmem = pre + (size_t)WAVES * nslots * mfma_tile_bytes<H>();
  if (static_lds + shmem > (size_t)LDS_PER_CU) return hipErrorInvalidConfiguration;
  // one worker per workgroup
  hipLaunchKernelGGL(kern, dim3(a.W), dim3(THREADS), shmem, stream, a, nslots);
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

int mfma_workgroups_per_cu(int B, int H, int RMAX) {
  (void)B;
  (void)H;
  (void)RMAX;
  return 1;
}

hipError_t launch_attn_mfma(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  const bool masked = a.window > 0 || a.tree != nullptr;
  return masked ? launch_mfma_m<true>(a, bf16, H, paged, stream)
                : launch_mfma_m<false>(a, bf16, H, paged, stream);
}

}  // namespace kvc
