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
// quarters visible and frees the slot of the tile before. One fetch of a K/V
// row thus serves 128 query rows.
//
// Per tile and wave (v_mfma_f32_16x16x32_{bf16,f16}, transposed score block):
// S^T = K . Q^T over the wave's two 16-row blocks, the query operand held in
// registers for the whole segment; online softmax in fp32 with the scale
// folded into the exponent's argument (exp2(s * c - m), c = |scale| log2 e;
// a negative scale flips the sign bits of the query operand instead, which
// is exact), the reference m raised only when the weights show it is needed
// (no per-tile maximum otherwise); p split into a 16-bit high part and the
// remainder (split_pair_fast); O^T += V^T . P^T. The K/V tiles come through
// a 64 KB ring of NR slots (a K tile and a V tile each), up to NR - 1 tiles in
// flight ahead of the one in use; the ring is refilled within a segment
// only, so each segment (one unit's share of this workgroup's range) starts
// with its own prologue of copies. The key mask is evaluated only on tiles
// not wholly visible to a wave's rows.
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
// A lane's sum of its 8 weights of a row in one tile that leaves every
// weight within the accumulators' range without a new reference.
constexpr float WEIGHT_BOUND = 256.0f;
constexpr int STATIC_LDS = 256;      // upper bound of the kernel's static LDS
constexpr int LDS_PER_CU = 160 * 1024;
constexpr int RING_BYTES = 64 * 1024;  // the K/V ring: 4 slots at H = 128, 8 at H = 64

// Ring slots: a K tile and a V tile each.
__host__ __device__ constexpr int ring_slots(int H) { return RING_BYTES / (2 * TILE * H * 2); }

__host__ __device__ constexpr size_t wide_dynamic_lds(int B) {
  return prefix_bytes(B) + (size_t)RING_BYTES;
}

// Wait until this wave's copies of the tile that `later` tiles were issued
// after have landed (NT instructions per tile; later < 8).
template <int NT>
__device__ __forceinline__ void wait_tiles(int later) {
  switch (later) {
    case 1: wait_vm<NT>(); break;
    case 2: wait_vm<2 * NT>(); break;
    case 3: wait_vm<3 * NT>(); break;
    case 4: wait_vm<4 * NT>(); break;
    case 5: wait_vm<5 * NT>(); break;
    case 6: wait_vm<6 * NT>(); break;
    default: wait_vm<0>(); break;  // none later: all
  }
}

// Two probability weights e0, e1 (finite, >= 0) as a packed 16-bit high part
// and a packed 16-bit remainder, hi + lo = e to about 2^-16 relative: the
// high part is one packed conversion; each remainder e - hi is one dot
// product of the packed high part with (-1, 0) or (0, -1) accumulated onto
// e, exact in fp32 (hi is e rounded to 16 bits, so e - hi is representable);
// the remainders are packed by one more conversion. The (-1, 0) and (0, -1)
// pairs come in registers (split_constants): as inline constants of the dot
// product their 16-bit encoding would be the assembler's to choose.
struct SplitConsts {
  uint32_t nx, ny;
};
template <bool BF>
__device__ __forceinline__ SplitConsts split_constants() {
  // -1 in the low / high half: bf16 0xBF80, f16 0xBC00
  SplitConsts k{BF ? 0x0000BF80u : 0x0000BC00u, BF ? 0xBF800000u : 0xBC000000u};
  asm volatile("" : "+v"(k.nx), "+v"(k.ny));
  return k;
}
template <bool BF>
__device__ __forceinline__ void split_pair_fast(float e0, float e1, const SplitConsts& k, uint32_t& hi,
                                                uint32_t& lo) {
  typedef __attribute__((ext_vector_type(2))) float float2_t;
  if constexpr (BF) {
    const bf162_t h = __builtin_convertvector((float2_t){e0, e1}, bf162_t);
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf162_t, k.nx), e0, false);
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf162_t, k.ny), e1, false);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){r0, r1}, bf162_t));
  } else {
    const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(e0, e1));
    const float r0 = __builtin_amdgcn_fdot2(h, __builtin_bit_cast(half2_t, k.nx), e0, false);
    const float r1 = __builtin_amdgcn_fdot2(h, __builtin_bit_cast(half2_t, k.ny), e1, false);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
  }
}

}  // namespace

int wide_workgroups_per_cu(int B, int H) {
  (void)H;
  return wide_dynamic_lds(B) + STATIC_LDS <= LDS_PER_CU / 2 ? 2 : 1;
}

template <bool BF, int H, bool PAGED, bool MASKED>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_wide_kernel(AttnArgs a) {
  constexpr int KS = H / 32;     // k-steps of S^T over h
  constexpr int MH = H / 16;     // 16-row h blocks of O^T
  constexpr int ROWB = H * 2;
  constexpr int HALFB = TILE * ROWB;      // one K or V tile
  constexpr int NI = HALFB / 1024;        // copy instructions per K or V tile
  constexpr int NIW = NI / WAVES;         // a wave's share of them
  static_assert(NI % WAVES == 0, "a tile's copies split evenly over the waves");
  constexpr int SLOTB = 2 * HALFB;        // ring slot: the K tile, then the V tile
  constexpr int NR = ring_slots(H);
  constexpr int DEPTH = NR - 1;           // tiles in flight ahead of the one in use
  static_assert(DEPTH >= 2 && DEPTH <= 7, "waits are counted for these depths");

  // [2B + 1], then the ring
  extern __shared__ __attribute__((aligned(16))) int32_t s_pre[];
  __shared__ int32_t s_wave[WAVES], s_flag[2];
  __shared__ int32_t s_bad[4];  // per segment ordinal mod 4: a bad block entry was met
  __shared__ int32_t s_count, s_early;  // a split unit's count; an early part was the last

  if (threadIdx.x < 4) s_bad[threadIdx.x] = 0;  // ordered by the barriers below
  build_tile_prefix(a, s_pre, s_wave);
  fill_invalid<H>(a, s_pre);
  const int worker = worker_of(a, blockIdx.x);
  const Partition part = make_partition<false>(a, s_pre, worker);
  append_owned<H, THREADS, PAGED>(a, s_pre, part);
  if (part.lo >= part.hi) return;  // the whole workgroup: no barrier is skipped

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int c = lane & 15;   // column (query row) / A-row (token or h) within a 16 block
  const int g = lane >> 4;   // k-slot group
  char* ring = reinterpret_cast<char*>(s_pre) + prefix_bytes(a.B);
  const uint32_t ring_lds = lds_addr(ring);
  const lds_char* ring3 = (const lds_char*)ring;

  // chunk swizzles: 16-byte chunk j of row r at position j ^ swz(r), so that
  // the A-operand reads are conflict-free
  auto swz_k = [](int r) { return H == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto swz_v = [](int r) { return H == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };
  uint32_t lvk[NIW], lvv[NIW];
  tile_lane_offsets<H, NIW>(a, lane, swz_k, lvk, wave * NIW);
  tile_lane_offsets<H, NIW>(a, lane, swz_v, lvv, wave * NIW);
  // A operand of S^T (K rows 16 mb + c): chunk 4 ks + g; swz_k(16 m + c) == swz_k(c)
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
  // the exponent's scale c > 0; a negative scale negates the query operand.
  // A scale below the smallest normal float (zero included) is taken as that
  // value: every s * c then rounds away in exp2(s * c - m) just as s * 0
  // would, while masked scores (-inf) keep -inf * c = -inf.
  const float sc = fmaxf(fabsf(a.scale_log2), __FLT_MIN__);
  const SplitConsts skc = split_constants<BF>();
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  SharedUnits shared;
  Segment early;             // a unit whose early part was counted last
  bool early_merge = false;  // (uniform)
  // Ring slots run on across segments: a segment's prologue fills the slots
  // after the previous segment's last tile, which a slower wave may still be
  // reading (a prologue holds at most NR - 1 tiles, so it never reaches
  // that slot; the first barrier of the segment frees it).
  int islot = 0;  // slot of the next tile issued
  int cslot = 0;  // slot of the next tile computed
  int64_t x = part.lo;
  for (int ord = 0; x < part.hi; ++ord) {
    const Segment s = find_segment(a, s_pre, part, x);
    x += s.t_end - s.t_begin;
    // live tiles: the segment's tokens up to the sequence's end (and, with a
    // window, from the tile holding the first visible key); never empty
    int t_lo = s.t_begin * STEP;
    if (MASKED) t_lo = max(t_lo, first_visible(a, s.seq_len) & ~(TILE - 1));
    const int t_hi = min(s.t_end * STEP, s.seq_len);
    const int nt = __builtin_amdgcn_readfirstlane((t_hi - t_lo + TILE - 1) / TILE);
    const int64_t hoff = (int64_t)s.k * a.stride_head + (PAGED ? 0 : (int64_t)s.b * a.stride_seq);
    const char* kb = a.k + hoff;
    const char* vb = a.v + hoff;
    int* bad_flag = &s_bad[ord & 3];

    const int row0w = s.rb * a.RMAX + wave * RW;  // this wave's first row of the unit
    const int tq_lo = min(row0w, a.R - 1) / a.G;  // its first new token
    const int new0 = s.seq_len - a.T;
    // this wave's query rows as the B operand of S^T: rows 16 nb + c, chunk
    // 4 ks + g (rows past R repeat row R - 1; their columns are discarded)
    uint4 qv[NB][KS];
    int tq[NB];                   // new-token index of this lane's query column
    uint32_t tw[NB][TREE_WORDS];  // its tree-mask row
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int rr = min(row0w + nb * 16 + c, a.R - 1);
      tq[nb] = rr / a.G;
      const char* qrow = a.q + row_index(a, s.b, s.k, rr) * ROWB;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = *reinterpret_cast<const uint4*>(qrow + 16 * (4 * ks + g));
        v.x ^= qsign;
        v.y ^= qsign;
        v.z ^= qsign;
        v.w ^= qsign;
        qv[nb][ks] = v;
      }
      const uint32_t* trow = MASKED && a.tree ? a.tree + ((int64_t)s.b * a.T + tq[nb]) * a.tree_words : nullptr;
#pragma unroll
      for (int w = 0; w < TREE_WORDS; ++w) tw[nb][w] = trow && w < a.tree_words ? trow[w] : 0u;
    }

    // tile j of the segment into ring slot `slot`
    auto issue = [&](int j, int slot) __attribute__((always_inline)) {
      const int tok = t_lo + j * TILE;
      const uint32_t dst = ring_lds + slot * SLOTB;
      bool bad = false;
      copy_tile_part<H, PAGED, MASKED, NIW>(a, s, kb, tok, dst, lane, swz_k, lvk, wave * NIW, bad);
      copy_tile_part<H, PAGED, MASKED, NIW>(a, s, vb, tok, dst + HALFB, lane, swz_v, lvv, wave * NIW, bad);
      if (PAGED && __ballot(bad) != 0ull && lane == 0) atomicOr(bad_flag, 1);
    };
    const int pro = min(DEPTH, nt);
    for (int j = 0; j < pro; ++j) {
      issue(j, islot);
      islot = islot + 1 == NR ? 0 : islot + 1;
    }
    // the query rows and tree words have landed (the compiler's own wait,
    // which also covers the copies just issued); later uses wait no more
    asm volatile("" ::"v"(qv[0][0].x), "v"(qv[NB - 1][KS - 1].w), "v"(tw[0][0]), "v"(tw[NB - 1][TREE_WORDS - 1]));

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

    for (int i = 0; i < nt; ++i) {
      // this wave's copies of tile i have landed; after the barrier every
      // wave's have, and every wave is done with tile i - 1, whose slot the
      // next issue refills
      if (i + DEPTH <= nt)
        wait_vm<(DEPTH - 1) * 2 * NIW>();
      else
        wait_tiles<2 * NIW>(nt - i - 1);
      __syncthreads();
      if (i + DEPTH < nt) {
        issue(i + DEPTH, islot);
        islot = islot + 1 == NR ? 0 : islot + 1;
      }
      const int tok0 = t_lo + i * TILE;

      // ---- the tile's operands from LDS, K for S^T and V^T for O^T, all
      // read up front so that their latency overlaps the first products
      // (the scheduling barrier keeps the compiler from moving the reads
      // down to their uses)
      const char* kt = ring + cslot * SLOTB;
      const lds_char* vt_base = ring3 + cslot * SLOTB + HALFB;
      uint4 kf[2][KS];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[mb][ks] = *reinterpret_cast<const uint4*>(kt + koff[ks] + mb * 16 * ROWB);
      uint4 vf[MH];
#pragma unroll
      for (int mh = 0; mh < MH; ++mh) {
        const uint2 lo4 = read_tr16(vt_base + voff[mh]);
        const uint2 hi4 = read_tr16(vt_base + voff[mh] + 16 * ROWB);
        vf[mh] = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- S^T = K . Q^T, row block 0 first
      floatx4 st[2][NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16<BF>(kf[mb][ks], qv[nb][ks], acc);
          st[mb][nb] = acc;
        }

      // ---- mask (tiles not wholly visible to every row of this wave)
      const bool edge = tok0 + TILE > (MASKED && a.tree ? new0 : new0 + 1 + tq_lo) ||
                        (MASKED && a.window > 0 && tok0 < s.seq_len - a.window);
      if (edge) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int tok = tok0 + mb * 16 + 4 * g + i4;
              if (!(MASKED ? key_visible(a, tok, new0, tq[nb], tree_word(tw[nb], tok - new0))
                           : tok <= new0 + tq[nb]))
                st[mb][nb][i4] = -__builtin_inff();
            }
      }

      // ---- online softmax (one query row per lane column). The weights
      // 2^(s c - m) are taken against the current reference m first; a
      // lane's sum of its 8 weights of a row bounds each of them, so while
      // every such sum is at most 2^8 no weight exceeds 2^8 (the
      // accumulators' range, as with a lazily raised maximum) and no
      // maximum is needed. Otherwise (a row's first visible keys, or a key
      // far above the reference) the reference is raised to the tile's
      // maximum where that is larger, and the weights are taken again.
      uint4 phi[NB], plo[NB];
      float tsum[NB];
      auto weights = [&](int nb) __attribute__((always_inline)) {
        uint32_t hw[4], lw[4];
        float ps[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; i4 += 2) {
            // a masked score (-inf) gives exp2(-inf) = 0 (c > 0)
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[mb][nb][i4], sc, -m[nb]));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[mb][nb][i4 + 1], sc, -m[nb]));
            ps[mb * 2 + i4 / 2] = e0 + e1;
            split_pair_fast<BF>(e0, e1, skc, hw[mb * 2 + i4 / 2], lw[mb * 2 + i4 / 2]);
          }
        tsum[nb] = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        phi[nb] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        plo[nb] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      };
      auto settle = [&](int nb) __attribute__((always_inline)) {
        // (NaN: over the bound)
        if (__builtin_amdgcn_ballot_w64(!(tsum[nb] <= WEIGHT_BOUND)) != 0ull) {
          float p8[8];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) p8[mb * 4 + i4] = st[mb][nb][i4] * sc;
          const float mr = fmaxf(fmaxf(fmaxf(p8[0], p8[1]), fmaxf(p8[2], p8[3])),
                                 fmaxf(fmaxf(p8[4], p8[5]), fmaxf(p8[6], p8[7])));
          // (-inf for a row with no visible key in the tile: unchanged)
          const float mn = fmaxf(m[nb], max_cols4(mr));
          const float alpha = __builtin_amdgcn_exp2f(m[nb] - mn);  // 1 where unchanged
          l[nb] *= alpha;
#pragma unroll
          for (int mh = 0; mh < MH; ++mh) ot[mh][nb] *= alpha;
          m[nb] = mn;
          weights(nb);
        }
        l[nb] += tsum[nb];
      };
      // ---- O^T += V^T . P^T
      auto pv = [&](int nb) __attribute__((always_inline)) {
#pragma unroll
        for (int mh = 0; mh < MH; ++mh) {
          ot[mh][nb] = mfma16<BF>(vf[mh], phi[nb], ot[mh][nb]);
          ot[mh][nb] = mfma16<BF>(vf[mh], plo[nb], ot[mh][nb]);
        }
      };
      // block by block: one block's products overlap the other's weights
      weights(0);
      settle(0);
      pv(0);
      weights(1);
      settle(1);
      pv(1);
      cslot = cslot + 1 == NR ? 0 : cslot + 1;
    }

    // ---- per-column totals of l (lanes of one column hold different tokens)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) l[nb] = sum_cols4(l[nb]);
    // Every wave issued this segment's copies before the barrier of its last
    // tile, so the flag is final. The flag two segments ahead is cleared
    // here: its last readers (two segments back) passed this segment's first
    // barrier before it, and its first writers come after the next
    // segment's first barrier, which wave 0 reaches only after clearing it.
    const bool bad = PAGED && *bad_flag != 0;
    if (PAGED && wave == 0 && lane == 0) s_bad[(ord + 2) & 3] = 0;

    // ---- this wave's rows: the output, or a partial. Of a unit split over
    // several workers, the part in the first segment of a range holds the
    // unit's later steps and is done early: its partial is counted at once.
    // The part in the last segment of a range holds the unit's first steps
    // and is done last: of a unit split in two, when the other part has
    // been counted, it is merged with it in registers (no partial stored
    // for it). Any other partial is counted at the range's end
    // (count_and_merge).
    const int rows = min(a.RMAX, a.R - s.rb * a.RMAX);  // valid rows of the unit
    const float qnan = __int_as_float(0x7fc00000);
    const bool first_seg = ord == 0, last_seg = x >= part.hi;
    bool own_merge = false;
    if (s.n_parts == 2 && last_seg && !first_seg) {
      if (threadIdx.x == 0)
        s_count = __hip_atomic_load(&a.counters[s.unit], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      own_merge = s_count == 1;  // (uniform) the other part was counted
      // its stores were acknowledged before its count
      if (own_merge) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    if (own_merge) {
      // the other part (the next worker's) into registers: all loads in
      // flight together, then merged into this part's state in place
      const int64_t so = (int64_t)s.first_wg + (worker == s.first_wg ? 1 : 0) + s.unit;
      float2_t mlo[NB], ov[NB][MH][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int lrc = min(wave * RW + nb * 16 + c, rows - 1);  // (rows past the unit: never stored)
        const float* po = a.part_o + (so * a.RMAX + lrc) * H + 4 * g;
        mlo[nb] = load_coherent2(a.part_ml + (so * a.RMAX + lrc) * 2);
#pragma unroll
        for (int mh = 0; mh < MH; ++mh) {
          ov[nb][mh][0] = load_coherent2(po + mh * 16);
          ov[nb][mh][1] = load_coherent2(po + mh * 16 + 2);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float M0 = bad ? qnan : m[nb];
        const float Mn = fmaxf(M0, mlo[nb].x);
        const float w0 = __builtin_amdgcn_exp2f(M0 - Mn), w1 = __builtin_amdgcn_exp2f(mlo[nb].x - Mn);
        l[nb] = (bad ? qnan : l[nb]) * w0 + mlo[nb].y * w1;
        m[nb] = Mn;
#pragma unroll
        for (int mh = 0; mh < MH; ++mh) {
          ot[mh][nb][0] = ot[mh][nb][0] * w0 + ov[nb][mh][0].x * w1;
          ot[mh][nb][1] = ot[mh][nb][1] * w0 + ov[nb][mh][0].y * w1;
          ot[mh][nb][2] = ot[mh][nb][2] * w0 + ov[nb][mh][1].x * w1;
          ot[mh][nb][3] = ot[mh][nb][3] * w0 + ov[nb][mh][1].y * w1;
        }
      }
      if (threadIdx.x == 0)
        __hip_atomic_store(&a.counters[s.unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (s.n_parts == 1 || own_merge) {
      // (a bad part: NaN through its l; a row with no visible key: 0 / 0)
      const bool nan_out = bad && !own_merge;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int lr = wave * RW + nb * 16 + c;
        if (lr < rows) {
          const int64_t ri = row_index(a, s.b, s.k, s.rb * a.RMAX + lr);
          const float inv = nan_out ? qnan : 1.0f / l[nb];
#pragma unroll
          for (int mh = 0; mh < MH; ++mh)
            store_out4(a.out, ri * H + mh * 16 + 4 * g, a.out_dtype, ot[mh][nb][0] * inv, ot[mh][nb][1] * inv,
                       ot[mh][nb][2] * inv, ot[mh][nb][3] * inv);
          if (g == 0 && a.lse) a.lse[ri] = nan_out ? qnan : (m[nb] + __log2f(l[nb])) * LN2;
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
          for (int mh = 0; mh < MH; ++mh) {
            const floatx4 o = ot[mh][nb];
            store_coherent2(po + lr * H + mh * 16 + 4 * g, bad ? qnan : o[0], bad ? qnan : o[1]);
            store_coherent2(po + lr * H + mh * 16 + 4 * g + 2, bad ? qnan : o[2], bad ? qnan : o[3]);
          }
          if (g == 0) store_coherent2(pml + lr * 2, bad ? qnan : m[nb], bad ? qnan : l[nb]);
        }
      }
      if (first_seg && !last_seg) {
        // count now; the rare last count merges at the range's end
        wait_stores();
        __syncthreads();
        if (threadIdx.x == 0) {
          const bool f = count_partial(a, s);
          if (f) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          s_early = f;
        }
        __syncthreads();
        if (s_early) {
          early_merge = true;
          early = s;
        }
      } else {
        shared.add(s);
      }
    }
  }
  // every copy has landed and been read: the ring is free
  __syncthreads();
  count_and_merge<H, WIDE_ROWS * H / THREADS>(a, shared, s_flag, reinterpret_cast<float*>(ring),
                                              RING_BYTES / 4);
  if (early_merge) merge_partials<H, WIDE_ROWS * H / THREADS>(a, early, reinterpret_cast<float*>(ring), RING_BYTES / 4);
}

// ---------------------------------------------------------------- launch

template <bool BF, int H, bool PAGED, bool MASKED>
static hipError_t launch_wide_t(const AttnArgs& a, hipStream_t stream) {
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
  const size_t shmem = wide_dynamic_lds(a.B);
  if (shmem + static_lds > (size_t)LDS_PER_CU) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kern, dim3(a.W), dim3(THREADS), shmem, stream, a);
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
