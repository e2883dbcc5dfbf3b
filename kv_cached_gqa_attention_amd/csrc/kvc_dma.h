// Streaming K/V tiles from HBM straight into LDS (gfx950 global_load_lds_dwordx4).
//
// One wave instruction copies 64 x 16 bytes: lane L's 16 bytes, read at
// sbase + voff(L), land at LDS byte m0 + 16 L (layout and the 18-bit LDS
// address range checked on the GPU). The data never occupies registers, so
// how much a wave keeps in flight is set by an LDS ring, not by its register
// budget.
//
// The copies are issued through inline assembly: the compiler neither counts
// nor waits for them (its own LDS-DMA tracking waits for all of them before
// any LDS read). Each kernel waits itself with wait_vm<N>, N being the number
// of copies it issued after the one it needs: vector memory loads complete in
// order, so once at most N are outstanding that one has landed. Compiler-
// visible vector loads or stores issued in between only make such a wait
// stricter. Uniform lookups inside a streaming loop (block-table entries,
// tree words) use scalar loads, which count on another counter.
#pragma once

#include "kvc_device.h"

namespace kvc {

// Bytes of the per-workgroup prefix table (2B + 1 ints, see
// build_tile_prefix) at the start of dynamic LDS, rounded up so the staging
// slots after it stay 16-byte aligned.
__host__ __device__ constexpr size_t prefix_bytes(int B) {
  return ((size_t)(2 * B + 1) * 4 + 15) & ~(size_t)15;
}

// LDS byte address of shared storage (the low half of its generic address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Copy 64 x 16 bytes: from sbase (wave-uniform) + voff (per lane, 32-bit
// unsigned) to LDS lds + 16 * lane. The copy takes its LDS address from m0,
// which no other instruction of these kernels uses (the compiler is told it
// is clobbered; the kernels' assembly is checked to hold no other m0 use).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = uniform_u32((uint32_t)u), hi = uniform_u32((uint32_t)(u >> 32));
  return reinterpret_cast<const char*>(lo | (hi << 32));
}

// m0 is named as clobbered; clang warns that it is a reserved register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// (The scalar operands are wave-uniform by construction; readfirstlane
// states it to the compiler, which otherwise may hold them in vector
// registers.)
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(uniform_u32(lds)), "v"(voff), "s"(uniform_ptr(sbase))
      : "memory", "m0");
}

// Same with a full 64-bit address per lane.
__device__ __forceinline__ void dma16_addr(const char* addr, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(uniform_u32(lds)), "v"(addr)
      : "memory", "m0");
}

#pragma clang diagnostic pop

// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until this wave's LDS reads have returned (before a slot they read is
// refilled).
__device__ __forceinline__ void wait_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Scalar load of a wave-uniform element of read-only memory.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int64_t i) {
  return ((const_i32_ptr)p)[i];
}
__device__ __forceinline__ uint32_t load_uniform(const uint32_t* p, int64_t i) {
  return (uint32_t)((const_i32_ptr)p)[i];
}

// A wave's walk over the steps of its workgroup's range, one tile per step,
// for issuing copies ahead of the compute: the current segment, the first
// token of this wave's tile at the current step, and the unit's K and V
// bases (the sequence's rows, or the pool with a block table).
struct StepCursor {
  int64_t x;      // flat step
  int64_t end;    // one past the segment's last
  int ord;        // segments entered before this one
  int tok0;       // first token of this wave's tile
  int wave;
  const char* kb;
  const char* vb;
  Segment s;

  __device__ __forceinline__ void begin(const AttnArgs& a, const int32_t* s_pre, const Partition& p, int64_t x0,
                        int w) {
    x = x0;
    ord = 0;
    wave = w;
    enter(a, s_pre, p);
  }
  __device__ __forceinline__ void advance(const AttnArgs& a, const int32_t* s_pre, const Partition& p) {
    ++x;
    tok0 += STEP;
    if (x == end && x < p.hi) {
      ++ord;
      enter(a, s_pre, p);
    }
  }

 private:
  __device__ __forceinline__ void enter(const AttnArgs& a, const int32_t* s_pre, const Partition& p) {
    s = find_segment(a, s_pre, p, x);
    end = x + (s.t_end - s.t_begin);
    tok0 = (s.t_begin * WAVES + wave) * TILE;
    const int64_t off = (int64_t)s.k * a.stride_head + (a.table ? 0 : (int64_t)s.b * a.stride_seq);
    kb = a.k + off;
    vb = a.v + off;
  }
};

// Copy the tile of TILE token rows starting at token `first` of one unit's K
// or V (base: the unit's rows, or the pool) to LDS at `lds`:
// row r (ROWB = 2H bytes) at lds + r * ROWB, its 16-byte chunk j at position
// j ^ swz(r) (swz: the kernel's bank-conflict swizzle, an involution on
// chunk positions). One instruction covers RPI = 64 / (ROWB / 16)
// consecutive rows; lane L reads row i * RPI + L / CPR of instruction i,
// whose in-tile byte offset lvoff[i] (row * stride_tok + 16 * chunk) the
// kernel computes once (tile_lane_offsets). copy_tile_part issues only the
// NIW instructions i0 .. i0 + NIW - 1 (a wave's share when the waves of a
// workgroup copy one tile together), lvoff holding their offsets.
//
// Tiles wholly inside the visible rows take a uniform base per block: with a
// block table, a block of at least TILE rows holds the whole tile (one
// scalar load of its entry), smaller blocks of at least RPI rows hold whole
// instructions (one entry per block). Other tiles (a unit's edges) clamp
// rows past the sequence's end, or before its first visible key, to the
// nearest valid row (their keys are masked); blocks smaller than RPI rows
// take per-lane entries (vector loads, which the compiler waits for,
// together with every copy issued before them). An entry outside the pool
// reads block 0 and sets `bad`.
template <int H, int NIW = TILE * H * 2 / 1024, typename Swz>
__device__ __forceinline__ void tile_lane_offsets(const AttnArgs& a, int lane, Swz swz, uint32_t (&lvoff)[NIW],
                                                  int i0 = 0) {
  constexpr int CPR = H * 2 / 16;
  constexpr int RPI = 64 / CPR;
  const int rl = lane / CPR;
  const int p = lane % CPR;
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int r = (i0 + i) * RPI + rl;
    lvoff[i] = (uint32_t)r * (uint32_t)a.stride_tok + (uint32_t)(p ^ swz(r)) * 16u;
  }
}

template <int H, bool PAGED, bool MASKED, int NIW, typename Swz>
__device__ __forceinline__ void copy_tile_part(const AttnArgs& a, const Segment& g, const char* base,
                                               int first, uint32_t lds, int lane, Swz swz,
                                               const uint32_t (&lvoff)[NIW], int i0, bool& bad) {
  constexpr int ROWB = H * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int RPI = 64 / CPR;
  const int last = g.seq_len - 1;
  const int vis0 = MASKED ? first_visible(a, g.seq_len) : 0;
  const int64_t trow = PAGED ? (int64_t)g.b * a.max_blocks : 0;
  const int bmask = (1 << a.block_shift) - 1;
  if (first >= vis0 && first + TILE - 1 <= last && (!PAGED || a.block_shift >= 5)) {
    const char* sb;
    if constexpr (PAGED) {
      int blk = load_uniform(a.table, trow + (first >> a.block_shift));
      if ((unsigned)blk >= (unsigned)a.num_blocks) {
        bad = true;
        blk = 0;
      }
      sb = base + (int64_t)blk * a.stride_seq + (int64_t)(first & bmask) * a.stride_tok;
    } else {
      sb = base + (int64_t)first * a.stride_tok;
    }
#pragma unroll
    for (int i = 0; i < NIW; ++i) dma16(sb, lvoff[i], lds + (i0 + i) * 1024);
    return;
  }
  if (PAGED && first >= vis0 && first + TILE - 1 <= last && (1 << a.block_shift) >= RPI) {
    // blocks of RPI..TILE-1 rows: a new entry where a block starts (tiles
    // start on a block boundary here), and for the first instruction
    const char* sb = base;
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int r0 = (i0 + i) * RPI;  // the instruction's first row in the tile
      if (i == 0 || (r0 & bmask) == 0) {
        int blk = load_uniform(a.table, trow + ((first + r0) >> a.block_shift));
        if ((unsigned)blk >= (unsigned)a.num_blocks) {
          bad = true;
          blk = 0;
        }
        // lvoff[i] counts rows from the tile's start
        sb = reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(base) + (int64_t)blk * a.stride_seq +
                                           (int64_t)((r0 & bmask) - r0) * a.stride_tok);
      }
      dma16(sb, lvoff[i], lds + (i0 + i) * 1024);
    }
    return;
  }
  // edges of a unit, and blocks smaller than one instruction's rows
  const int rl = lane / CPR;
  const int p = lane % CPR;
  const uint32_t stok = (uint32_t)a.stride_tok;
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int r = (i0 + i) * RPI + rl;
    const uint32_t jb = (uint32_t)(p ^ swz(r)) * 16u;
    const int t0 = first + (i0 + i) * RPI;
    int tb = min(t0, last);
    if constexpr (MASKED) tb = max(tb, vis0);
    int tok = min(t0 + rl, last);
    if constexpr (MASKED) tok = max(tok, vis0);
    if constexpr (PAGED) {
      if ((1 << a.block_shift) < RPI) {
        int blk = a.table[trow + (tok >> a.block_shift)];
        if ((unsigned)blk >= (unsigned)a.num_blocks) {
          bad = true;
          blk = 0;
        }
        dma16_addr(base + (int64_t)blk * a.stride_seq + (int64_t)(tok & bmask) * a.stride_tok + jb,
                   lds + (i0 + i) * 1024);
      } else {
        // tb and every clamped row of this instruction share one block
        int blk = load_uniform(a.table, trow + (tb >> a.block_shift));
        if ((unsigned)blk >= (unsigned)a.num_blocks) {
          bad = true;
          blk = 0;
        }
        const char* sb = base + (int64_t)blk * a.stride_seq + (int64_t)(tb & bmask) * a.stride_tok;
        dma16(sb, (uint32_t)(tok - tb) * stok + jb, lds + (i0 + i) * 1024);
      }
    } else {
      dma16(base + (int64_t)tb * a.stride_tok, (uint32_t)(tok - tb) * stok + jb, lds + (i0 + i) * 1024);
    }
  }
}

// The whole tile (every instruction), as one wave copies it.
template <int H, bool PAGED, bool MASKED, typename Swz>
__device__ __forceinline__ void copy_tile(const AttnArgs& a, const Segment& g, const char* base,
                                          int first, uint32_t lds, int lane, Swz swz,
                                          const uint32_t (&lvoff)[TILE * H * 2 / 1024], bool& bad) {
  copy_tile_part<H, PAGED, MASKED, TILE * H * 2 / 1024>(a, g, base, first, lds, lane, swz, lvoff, 0, bad);
}

}  // namespace kvc
