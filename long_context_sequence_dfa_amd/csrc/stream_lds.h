// stream_lds.h -- streaming of 64-row bf16 operand tiles from HBM into LDS for
// the gfx950 attention kernels: the LDS tile layout, direct (register-free)
// loads issued so that several tiles are in flight at once, and the explicit
// wait that tells a wave when its part of a tile has landed.
#pragma once

#include "device_util.h"

namespace dfa {

// Row order of a 32-row operand block inside the S (or S^T) MFMA: swaps bits
// 2 and 3 of the row index, so that the accumulator of a lane holds 8
// consecutive rows per 16-row step -- the operand layout of the next product.
__device__ __forceinline__ int kperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// 64-row tile in LDS: pitch HD*2 + 32 bytes, logical 16-byte chunk c of row r
// stored at chunk c ^ bit3(r).  Both the b128 reads of 16 rows (MFMA operands
// in kperm row order) and the transposing reads of 4 rows x 32 bytes then hit
// distinct banks, and every operand address stays affine in the loop indices.
template <int HD>
struct Tile64 {
  static constexpr int ROWS = 64;
  static constexpr int RB = HD * 2 + 32;             // row pitch in bytes
  static constexpr int TB = ROWS * RB;               // tile bytes
  static constexpr int LPR = HD * 2 / 16;            // 16-byte data chunks per row

  // b128 operand read: row kperm(c32) of a 32-row block, chunk pair 2 ks + g
  // (add 32 ks bytes and 32 RB per block)
  __device__ static int a_off(int lane) {
    const int g = lane >> 5, c32 = lane & 31;
    return kperm(c32) * RB + 16 * (g ^ ((c32 >> 2) & 1));
  }
  // transposing read of a 16-row group: rows 8g + (lane&15)/4 (+4 for the
  // upper half), 4 bf16 columns at 16((lane>>4)&1) + 4(lane&3) (add 16 RB per
  // row group and 64 bytes per block of 32 columns)
  __device__ static int t_off(int lane) {
    const int g = lane >> 5;
    return (8 * g + (lane & 15) / 4) * RB + 16 * ((2 * ((lane >> 4) & 1) + (lane & 3) / 2) ^ g) +
           8 * (lane & 1);
  }
};

// 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return static_cast<unsigned>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)(p)));
#else
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>(p));  // host pass only
#endif
}

// Direct loads from base + off (off per lane, base uniform) into LDS at
// lds + BYTES * lane (lds uniform).  They are written as inline assembly so
// that the compiler, which cannot tell which tile a later LDS read touches,
// does not make every LDS read wait for them: callers wait explicitly
// (vm_wait, then a barrier) before reading a tile.  The compiler inserts no
// hazard padding inside an asm block, so the block carries its own: a vector
// memory instruction may read an SGPR only 5 wait states after a VALU wrote
// it (the base often comes from v_readfirstlane), and the LDS DMA needs one
// wait state after the M0 write; s_nop 4 covers both.
__device__ __forceinline__ void dma16(const void *base, unsigned off, unsigned lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(uniform_u64(reinterpret_cast<uint64_t>(base))),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds)));
}
__device__ __forceinline__ void dma4(const void *base, unsigned off, unsigned lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(off), "s"(uniform_u64(reinterpret_cast<uint64_t>(base))),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds)));
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order); other counters are not waited.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Runtime (wave-uniform) count; counts above 24 wait for everything.
__device__ __forceinline__ void vm_wait(int n) {
  switch (n) {
#define DFA_VM_CASE(N) \
  case N:              \
    vm_wait<N>();      \
    break;
    DFA_VM_CASE(1) DFA_VM_CASE(2) DFA_VM_CASE(3) DFA_VM_CASE(4) DFA_VM_CASE(5) DFA_VM_CASE(6)
    DFA_VM_CASE(7) DFA_VM_CASE(8) DFA_VM_CASE(9) DFA_VM_CASE(10) DFA_VM_CASE(11) DFA_VM_CASE(12)
    DFA_VM_CASE(13) DFA_VM_CASE(14) DFA_VM_CASE(15) DFA_VM_CASE(16) DFA_VM_CASE(17) DFA_VM_CASE(18)
    DFA_VM_CASE(19) DFA_VM_CASE(20) DFA_VM_CASE(21) DFA_VM_CASE(22) DFA_VM_CASE(23) DFA_VM_CASE(24)
#undef DFA_VM_CASE
    default:
      vm_wait<0>();
  }
}

// Direct loads of two 64-row tiles (separate row strides, e.g. K and V) into
// the Tile64 layout by NW waves.  One instruction writes 64 lanes x 16
// contiguous bytes of LDS, so instruction i fills the tile's padded 16-byte
// chunks 64 i .. 64 i + 63 in row-major order: every lane of every
// instruction is used (ROWS * RB / 1024 instructions per tile, exact), rows
// simply continue across instruction boundaries, and a lane that lands on a
// pad chunk re-reads its row's first data chunk.  Wave w issues instructions
// w, w + NW, ...; a lane's source offsets are fixed, so they are computed
// once (32-bit: the host guarantees that 64 rows span less than 2^31 bytes).
// Rows past the piece re-read its last row; the caller's mask drops them.
template <int HD, int NW>
struct TileStream {
  using T = Tile64<HD>;
  static constexpr int CPR = T::RB / 16;            // 16-byte chunks per padded row
  static constexpr int NI = T::ROWS * CPR / 64;     // instructions per tile
  static_assert(T::ROWS * CPR % 64 == 0, "a tile is a whole number of instructions");
  static constexpr int MW = (NI + NW - 1) / NW;     // instructions per wave and tensor (max)
  int wv, lane;
  unsigned rsa, rsb;
  unsigned oa[MW], ob[MW];

  // instructions this wave issues per tensor and tile (wave-uniform)
  __device__ int count() const { return wv < NI ? (NI - wv + NW - 1) / NW : 0; }
  // tile row and source chunk of this lane in instruction i
  __device__ int row_of(int i) const { return (64 * i + lane) / CPR; }
  __device__ int chunk_of(int i) const {
    const int c = (64 * i + lane) % CPR;
    return c < T::LPR ? c ^ ((row_of(i) >> 3) & 1) : 0;
  }

  __device__ TileStream(int wave, int lane_, int64_t rs_a, int64_t rs_b)
      : wv(wave), lane(lane_), rsa(static_cast<unsigned>(rs_a)), rsb(static_cast<unsigned>(rs_b)) {
#pragma unroll
    for (int m = 0; m < MW; ++m) {
      const int i = wv + NW * m, r = row_of(i), c = chunk_of(i);
      oa[m] = r * rsa + 16 * c;
      ob[m] = r * rsb + 16 * c;
    }
  }

  // ga/gb: first row of the tile; la/lb: LDS tile addresses; rows: rows left
  // in the piece from the first row on (>= 1)
  __device__ void load(const char *ga, const char *gb, unsigned la, unsigned lb, int64_t rows) const {
    if (rows >= T::ROWS) {
#pragma unroll
      for (int m = 0; m < MW; ++m) {
        const int i = wv + NW * m;
        if (i < NI) {
          dma16(ga, oa[m], la + 1024 * i);
          dma16(gb, ob[m], lb + 1024 * i);
        }
      }
    } else {
      const int last = static_cast<int>(rows - 1);
#pragma unroll
      for (int m = 0; m < MW; ++m) {
        const int i = wv + NW * m;
        if (i < NI) {
          const int r = row_of(i), rr = r < last ? r : last, c = chunk_of(i);
          dma16(ga, rr * rsa + 16 * c, la + 1024 * i);
          dma16(gb, rr * rsb + 16 * c, lb + 1024 * i);
        }
      }
    }
  }
};

}  // namespace dfa
