// Split-KV attention on the matrix cores for long query blocks: a chunk of a
// prompt processed against the cache ("CS336, lectures 10 and 12", section
// on the two stages of inference: the prompt's tokens are processed in
// parallel, the compute-bound stage), where G * T query rows read each K/V
// row of a (b, k).
//
// A unit is (b, k, block of WIDE_ROWS = 4 x 32 query rows). The four waves of
// a workgroup hold 32 rows each and compute on the same K/V tiles: the
// workgroup copies each 32-token tile into LDS together (every wave a
// quarter of its copy instructions), and a barrier per tile makes all
// quarters visible and frees the slots of the tile before. One fetch of a
// K/V row thus serves 128 query rows, where the per-wave form (each wave its
// own tile for all of the unit's rows) serves at most 64; long blocks re-read
// the K/V rows once per row block, and with fewer rows per block those
// re-reads bound the per-wave form on prefill-sized chunks.
//
// Per tile and wave the arithmetic is that of the per-wave form
// (v_mfma_f32_16x16x32_{bf16,f16}, transposed score block, p split into a
// 16-bit high part and remainder, kvc_mfma.h): S^T = K . Q^T over the wave's
// two 16-row blocks, online softmax in fp32, O^T += V^T . P^T. The query
// rows live in LDS (each wave copies its own); the K/V tiles come through a
// ring of `nslots` halves (K and V tiles alternating), all but the tile in
// use in flight. Every wave computes every live tile of the unit; the key
// mask is evaluated only on tiles not wholly visible to its rows.
#include "kvc.h"
#include "kvc_device.h"
#include "kvc_dma.h"
#include "kvc_internal.h"
#include "kvc_mfma.h"

namespace kvc {

namespace {

constexpr int NB = 2;                // 16-row blocks per wave
constexpr int TREE_WORDS = KVC_MAX_TREE_T / 32;  // mask words per row

// The word of a tree-mask row holding the bit of new token u (u >= 0; an
// index past the row gives a word that is never consulted).
__device__ __forceinline__ uint32_t tree_word(const uint32_t (&row)[TREE_WORDS], int u) {
  const int w = u >> 5;
  uint32_t v = row[0];
#pragma unroll
  for (int i = 1; i < TREE_WORDS; ++i) v = w == i ? row[i] : v;
  return v;
}
constexpr int RW = NB * 16;          // query rows per wave
constexpr int MAX_SLOTS = 8;         // ring halves (waits are counted up to this)
constexpr int MIN_SLOTS = 4;         // a tile in use and the next one in flight
constexpr int SLOTS_TWO_PER_CU = 5;  // ring halves when two workgroups share a CU
constexpr int STATIC_LDS = 256;      // upper bound of the kernel's static LDS

template <int H>
constexpr size_t tile_bytes() { return (size_t)TILE * H * 2; }

__host__ __device__ constexpr size_t wide_dynamic_lds(int B, int H, int nslots) {
  return prefix_bytes(B) + (size_t)WIDE_ROWS * H * 2 + (size_t)nslots * TILE * H * 2;
}

// Wait until the copies of the half issued `later` halves before the newest
// one have landed (this wave's share: NIW instructions per half).
template <int NIW>
__device__ __forceinline__ void wait_halves(int later) {
  switch (later) {
    case 1: wait_vm<NIW>(); break;
    case 2: wait_vm<2 * NIW>(); break;
    case 3: wait_vm<3 * NIW>(); break;
    case 4: wait_vm<4 * NIW>(); break;
    case 5: wait_vm<5 * NIW>(); break;
    case 6: wait_vm<6 * NIW>(); break;
    case 7: wait_vm<7 * NIW>(); break;
    default: wait_vm<0>(); break;  // none later (or more than a ring holds): all
  }
}

// The workgroup's walk over the live tiles of its range, in order: every
// tile of every step except those holding no key any row of the unit can
// see (past the sequence's end; with a window, wholly before its first
// visible key). Live tiles of a step are consecutive and every step holds
// at least one (its unit's first step holds the first visible key, its last
// step the last key).
template <bool MASKED>
struct TileWalk {
  StepCursor st;  // as wave 0 sees it: st.tok0 is the step's first token
  int sub;        // tile within the step

  __device__ __forceinline__ bool live(const AttnArgs& a, int j) const {
    const int t0 = st.tok0 + j * TILE;
    return t0 < st.s.seq_len && (!MASKED || t0 + TILE > first_visible(a, st.s.seq_len));
  }
  __device__ __forceinline__ int tok0() const { return st.tok0 + sub * TILE; }
  __device__ __forceinline__ void first_live(const AttnArgs& a) {
    sub = 0;
    while (sub < WAVES - 1 && !live(a, sub)) ++sub;
  }
  __device__ __forceinline__ void begin(const AttnArgs& a, const int32_t* s_pre, const Partition& p) {
    st.begin(a, s_pre, p, p.lo, 0);
    first_live(a);
  }
  __device__ __forceinline__ bool step_last(const AttnArgs& a) const {
    return sub == WAVES - 1 || !live(a, sub + 1);
  }
  // the current tile is its segment's last / the range's last
  __device__ __forceinline__ bool seg_last(const AttnArgs& a) const { return st.x + 1 == st.end && step_last(a); }
  __device__ __forceinline__ bool range_last(const AttnArgs& a, const Partition& p) const {
    return st.x + 1 == p.hi && step_last(a);
  }
  // to the next live tile (the current one is not the range's last)
  __device__ __forceinline__ void next(const AttnArgs& a, const int32_t* s_pre, const Partition& p) {
    if (!step_last(a)) {
      ++sub;
      return;
    }
    st.advance(a, s_pre, p);
    first_live(a);
  }
};

}  // namespace

int wide_workgroups_per_cu(int B, int H) {
  return wide_dynamic_lds(B, H, SLOTS_TWO_PER_CU) + STATIC_LDS <= 80 * 1024 ? 2 : 1;
}

template <bool BF, int H, bool PAGED, bool MASKED>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_wide_kernel(AttnArgs a, int nslots) {
  constexpr int KS = H / 32;     // k-steps of S^T over h
  constexpr int MH = H / 16;     // 16-row h blocks of O^T
  constexpr int ROWB = H * 2;
  constexpr int NI = TILE * ROWB / 1024;  // copy instructions per tile
  constexpr int NIW = NI / WAVES;         // a wave's share of them
  static_assert(NI % WAVES == 0, "a tile's copies split evenly over the waves");
  constexpr int TILEB = TILE * ROWB;
  constexpr int QI = RW * ROWB / 1024;    // copy instructions of a wave's query rows

  // [2B + 1], the unit's query rows (RW per wave), then the ring
  extern __shared__ __attribute__((aligned(16))) int32_t s_pre[];
  __shared__ int32_t s_wave[WAVES], s_flag[2];
  __shared__ int32_t s_bad[16];  // per segment ordinal mod 16: a bad block entry was met

  if (threadIdx.x < 16) s_bad[threadIdx.x] = 0;  // ordered by the barriers below
  build_tile_prefix(a, s_pre, s_wave);
  fill_invalid<H>(a, s_pre);
  const int worker = worker_of(a, blockIdx.x);
  const Partition part = make_partition(a, s_pre, worker);
  append_owned<H, THREADS, PAGED>(a, s_pre, part);
  if (part.lo >= part.hi) return;  // the whole workgroup: no barrier is skipped

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int c = lane & 15;   // column (query row) / A-row (token or h) within a 16 block
  const int g = lane >> 4;   // k-slot group
  char* qarea = reinterpret_cast<char*>(s_pre) + prefix_bytes(a.B);
  char* qwave = qarea + wave * RW * ROWB;  // this wave's rows, swizzled as K
  char* ring = qarea + WIDE_ROWS * ROWB;
  const uint32_t ring_lds = lds_addr(ring);
  const lds_char* ring3 = (const lds_char*)ring;

  // chunk swizzles, as in the per-wave form: 16-byte chunk j of row r at
  // position j ^ swz(r), so that the A-operand reads are conflict-free
  auto swz_k = [](int r) { return H == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto swz_v = [](int r) { return H == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };
  uint32_t lvk[NIW], lvv[NIW];
  tile_lane_offsets<H, NIW>(a, lane, swz_k, lvk, wave * NIW);
  tile_lane_offsets<H, NIW>(a, lane, swz_v, lvv, wave * NIW);
  // A operand of S^T (K rows 16 mb + c) and B operand (query rows 16 nb + c):
  // chunk 4 ks + g; swz_k(16 m + c) == swz_k(c)
  uint32_t koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = c * ROWB + 16 * ((4 * ks + g) ^ swz_k(c));
  // A operand of O^T += V^T . P^T: two transposed reads per 16-h block
  uint32_t voff[MH];
  {
    const int r = 4 * g + (c >> 2);
    const int b = c & 3;
#pragma unroll
    for (int mh = 0; mh < MH; ++mh)
      voff[mh] = r * ROWB + 16 * ((2 * mh + (b >> 1)) ^ swz_v(r)) + 8 * (b & 1);
  }

  // ---- copies: halves K(t), V(t) of the live tiles t in walk order
  TileWalk<MASKED> pc;
  pc.begin(a, s_pre, part);
  bool pdone = false;  // every half of the range issued
  bool pv = false;     // next one is a V half
  int hp = 0;          // halves issued
  int pslot = 0;       // slot of the next one
  auto issue_next = [&]() __attribute__((always_inline)) {
    const uint32_t dst = ring_lds + pslot * TILEB;
    bool bad = false;
    if (!pv) {
      copy_tile_part<H, PAGED, MASKED, NIW>(a, pc.st.s, pc.st.kb, pc.tok0(), dst, lane, swz_k, lvk,
                                            wave * NIW, bad);
    } else {
      copy_tile_part<H, PAGED, MASKED, NIW>(a, pc.st.s, pc.st.vb, pc.tok0(), dst, lane, swz_v, lvv,
                                            wave * NIW, bad);
    }
    if (PAGED && __ballot(bad) != 0ull && lane == 0) atomicOr(&s_bad[pc.st.ord & 15], 1);
    if (pv) {
      if (pc.range_last(a, part)) pdone = true; else pc.next(a, s_pre, part);
    }
    pv = !pv;
    ++hp;
    pslot = pslot + 1 == nslots ? 0 : pslot + 1;
  };
  int hc = 0;     // halves consumed (the K half of the tile in use)
  int cslot = 0;  // its slot
  // keep the ring full: every slot but the tile in use (and, before the
  // barrier that frees them, the previous tile's) holds a half in flight
  auto fill = [&]() __attribute__((always_inline)) {
    while (!pdone && hp - hc < nslots) issue_next();
  };
  fill();

  TileWalk<MASKED> cs;
  cs.begin(a, s_pre, part);
  SharedUnits shared;
  while (true) {
    const Segment s = cs.st.s;
    const int ord = cs.st.ord;
    const int row0w = s.rb * a.RMAX + wave * RW;  // this wave's first row of the unit
    const int tq_lo = min(row0w, a.R - 1) / a.G;  // its first new token
    int tq[NB];         // new-token index of this lane's query column
    uint32_t tw[NB][TREE_WORDS];  // its tree-mask row (T <= KVC_MAX_TREE_T)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int rr = row0w + nb * 16 + c;
      tq[nb] = rr < a.R ? rr / a.G : a.T - 1;  // padding column: any valid row, discarded
      const uint32_t* trow = MASKED && a.tree ? a.tree + ((int64_t)s.b * a.T + tq[nb]) * a.tree_words : nullptr;
#pragma unroll
      for (int w = 0; w < TREE_WORDS; ++w) tw[nb][w] = trow && w < a.tree_words ? trow[w] : 0u;
    }
    // this wave's query rows into its LDS rows (rows past R repeat row R - 1;
    // their columns are discarded); only this wave reads them
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int q = i * 64 + lane;  // 16-byte chunk of the wave's rows
      const int r = q / (ROWB / 16);
      const int j = (q % (ROWB / 16)) ^ swz_k(r);
      const int rr = min(row0w + r, a.R - 1);
      dma16_addr(a.q + row_index(a, s.b, s.k, rr) * ROWB + j * 16, lds_addr(qwave) + i * 1024);
    }
    wait_vm<0>();  // the query rows (and every copy issued before them)

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
      // this wave's quarters of K(t) and V(t) have landed; after the barrier
      // every wave's have, and every wave is done with the previous tile
      wait_halves<NIW>(hp - hc - 2);
      __syncthreads();
      fill();
      const int kslot = cslot;
      const int vslot = cslot + 1 == nslots ? 0 : cslot + 1;

      // Every wave computes every tile, masked where needed: a branch around
      // the products (skipping tiles a wave's rows cannot see) makes the
      // compiler copy the accumulators in and out of it on every tile.
      const int tok0 = cs.tok0();
      {
        // ---- S^T = K . Q^T
        const char* kt = ring + kslot * TILEB;
        uint4 kf[2][KS];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kf[mb][ks] = *reinterpret_cast<const uint4*>(kt + koff[ks] + mb * 16 * ROWB);
        floatx4 st[2][NB];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const uint4 qv = *reinterpret_cast<const uint4*>(qwave + nb * 16 * ROWB + koff[ks]);
              acc = mfma16<BF>(kf[mb][ks], qv, acc);
            }
            st[mb][nb] = acc;
          }

        // ---- scale, mask, online softmax (one query row per lane column);
        // tiles wholly visible to every row of this wave skip the test
        const bool edge = tok0 + TILE > (MASKED && a.tree ? new0 : new0 + 1 + tq_lo) ||
                          (MASKED && a.window > 0 && tok0 < s.seq_len - a.window);
        float p[NB][2][4], mt[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[nb][mb][i] = st[mb][nb][i] * a.scale_log2;
        if (edge) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int tok = tok0 + mb * 16 + 4 * g + i;
                if (!(MASKED ? key_visible(a, tok, new0, tq[nb], tree_word(tw[nb], tok - new0))
                             : tok <= new0 + tq[nb]))
                  p[nb][mb][i] = -__builtin_inff();
              }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
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

        // ---- O^T += V^T . P^T
        const lds_char* vt_base = ring3 + vslot * TILEB;
#pragma unroll
        for (int mh = 0; mh < MH; ++mh) {
          const uint2 lo4 = read_tr16(vt_base + voff[mh]);
          const uint2 hi4 = read_tr16(vt_base + voff[mh] + 16 * ROWB);
          const uint4 v = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            ot[mh][nb] = mfma16<BF>(v, phi[nb], ot[mh][nb]);
            ot[mh][nb] = mfma16<BF>(v, plo[nb], ot[mh][nb]);
          }
        }
      }
      hc += 2;  // both halves are released at the next barrier
      cslot = vslot + 1 == nslots ? 0 : vslot + 1;
      if (cs.seg_last(a)) break;
      cs.next(a, s_pre, part);
    }

    // ---- per-column totals of l (lanes of one column hold different tokens)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) l[nb] = sum_cols4(l[nb]);
    // Every wave issued this segment's copies before the barrier of its last
    // tile, so the flag is final; the entry 8 ordinals ahead (never touched
    // by copies in flight, which run at most MAX_SLOTS / 2 tiles ahead) is
    // cleared for reuse.
    const bool bad = PAGED && s_bad[ord & 15] != 0;
    if (PAGED && wave == 0 && lane == 0) s_bad[(ord + 8) & 15] = 0;

    // ---- this wave's rows: the output, or a partial counted at the range's end
    const int rows = min(a.RMAX, a.R - s.rb * a.RMAX);  // valid rows of the unit
    const float qnan = __int_as_float(0x7fc00000);
    if (s.n_parts == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int lr = wave * RW + nb * 16 + c;
        if (lr < rows) {
#pragma unroll
          for (int mh = 0; mh < MH; ++mh)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              write_final(a, s.b, s.k, s.rb * a.RMAX + lr, H, mh * 16 + 4 * g + i,
                          bad ? qnan : ot[mh][nb][i], bad ? qnan : m[nb], bad ? qnan : l[nb]);
        }
      }
    } else {
      const int64_t slot = (int64_t)worker + s.unit;
      float* po = a.part_o + slot * a.RMAX * H;
      float* pml = a.part_ml + slot * a.RMAX * 2;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int lr = wave * RW + nb * 16 + c;
        if (lr < rows) {
#pragma unroll
          for (int mh = 0; mh < MH; ++mh)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              store_coherent(po + lr * H + mh * 16 + 4 * g + i, bad ? qnan : ot[mh][nb][i]);
          if (g == 0) {
            store_coherent(pml + lr * 2 + 0, bad ? qnan : m[nb]);
            store_coherent(pml + lr * 2 + 1, bad ? qnan : l[nb]);
          }
        }
      }
      shared.add(s);
    }
    if (cs.range_last(a, part)) break;
    cs.next(a, s_pre, part);
  }
  // every copy has landed and been read: the query rows and the ring are free
  __syncthreads();
  count_and_merge<H, WIDE_ROWS * H / THREADS>(a, shared, s_flag, reinterpret_cast<float*>(qarea),
                                              (int)((WIDE_ROWS * ROWB + nslots * TILEB) / 4));
}

// ---------------------------------------------------------------- launch

template <bool BF, int H, bool PAGED, bool MASKED>
static hipError_t launch_wide_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int LDS_PER_CU = 160 * 1024;
  const auto kern = attn_wide_kernel<BF, H, PAGED, MASKED>;
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
  if (a.RMAX != WIDE_ROWS || static_lds > (size_t)STATIC_LDS) return hipErrorInvalidConfiguration;
  // two workgroups per CU with SLOTS_TWO_PER_CU halves where they fit, else
  // one with as many halves as its LDS holds
  int nslots = SLOTS_TWO_PER_CU;
  if (wide_workgroups_per_cu(a.B, H) == 1) {
    const size_t fixed = wide_dynamic_lds(a.B, H, 0) + static_lds;
    nslots = fixed < (size_t)LDS_PER_CU ? (int)((LDS_PER_CU - fixed) / tile_bytes<H>()) : 0;
    if (nslots > MAX_SLOTS) nslots = MAX_SLOTS;
    if (nslots < MIN_SLOTS) return hipErrorInvalidConfiguration;
  }
  const size_t shmem = wide_dynamic_lds(a.B, H, nslots);
  hipLaunchKernelGGL(kern, dim3(a.W), dim3(THREADS), shmem, stream, a, nslots);
  return hipGetLastError();
}

template <bool MASKED>
static hipError_t launch_wide_m(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  if (bf16) {
    if (H == 64)
      return paged ? launch_wide_t<true, 64, true, MASKED>(a, stream)
                   : launch_wide_t<true, 64, false, MASKED>(a, stream);
    return paged ? launch_wide_t<true, 128, true, MASKED>(a, stream)
                 : launch_wide_t<true, 128, false, MASKED>(a, stream);
  }
  if (H == 64)
    return paged ? launch_wide_t<false, 64, true, MASKED>(a, stream)
                 : launch_wide_t<false, 64, false, MASKED>(a, stream);
  return paged ? launch_wide_t<false, 128, true, MASKED>(a, stream)
               : launch_wide_t<false, 128, false, MASKED>(a, stream);
}

hipError_t launch_attn_wide(const AttnArgs& a, bool bf16, int H, bool paged, hipStream_t stream) {
  const bool masked = a.window > 0 || a.tree != nullptr;
  return masked ? launch_wide_m<true>(a, bf16, H, paged, stream)
                : launch_wide_m<false>(a, bf16, H, paged, stream);
}

}  // namespace kvc
