// device_util.h -- small device helpers for the gfx950 kernels: vector types,
// MFMA wrappers, the transposing LDS read and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A(32x16) * B(16x32) + C on the matrix cores.  Lane l supplies
// A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32]; lane l receives
// C[8*(i/4) + 4*(l/32) + i%4][l%32] in element i.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j names 4 consecutive 16-bit elements; lane i receives element i%4 of
// the elements named by lanes 4e + i/4, e = 0..3.  Used so that lane i of a
// group gets column i of a row-major 4x16 tile.
__device__ __forceinline__ bf16x4 lds_read_tr(const char *p) {
  typedef __attribute__((address_space(3))) short4v lds_s4;
  short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(x));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(x >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Lane `l` (wave-uniform) of a 64-bit value.
__device__ __forceinline__ int64_t readlane64(int64_t x, int l) {
  const unsigned lo = __builtin_amdgcn_readlane(static_cast<unsigned>(x), l);
  const unsigned hi = __builtin_amdgcn_readlane(static_cast<unsigned>(static_cast<uint64_t>(x) >> 32), l);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Read of a work-table entry (wave-uniform address, constant for the whole
// launch) with scalar loads (early-clobber outputs: the second load of a
// pair still reads the base).  Written as inline assembly so that it stays a
// scalar load even where the compiler cannot prove the memory unmodified: a
// vector load here would share the vector-memory counter with the tile
// streams, and waiting for it would also wait for every tile in flight.
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void sload_words(uint64_t b, uint32_t (&w)[2]) {
  u32x2 x;
  asm("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(x) : "s"(b));
  w[0] = x[0], w[1] = x[1];
}
__device__ __forceinline__ void sload_words(uint64_t b, uint32_t (&w)[6]) {
  u32x4 x;
  u32x2 y;
  asm("s_load_dwordx4 %0, %2, 0x0\n\ts_load_dwordx2 %1, %2, 0x10\n\ts_waitcnt lgkmcnt(0)"
      : "=&s"(x), "=&s"(y)
      : "s"(b));
  for (int i = 0; i < 4; ++i) w[i] = x[i];
  w[4] = y[0], w[5] = y[1];
}
__device__ __forceinline__ void sload_words(uint64_t b, uint32_t (&w)[8]) {
  u32x8_t x;
  asm("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(x) : "s"(b));
  for (int i = 0; i < 8; ++i) w[i] = x[i];
}
__device__ __forceinline__ void sload_words(uint64_t b, uint32_t (&w)[10]) {
  u32x8_t x;
  u32x2 y;
  asm("s_load_dwordx8 %0, %2, 0x0\n\ts_load_dwordx2 %1, %2, 0x20\n\ts_waitcnt lgkmcnt(0)"
      : "=&s"(x), "=&s"(y)
      : "s"(b));
  for (int i = 0; i < 8; ++i) w[i] = x[i];
  w[8] = y[0], w[9] = y[1];
}
__device__ __forceinline__ void sload_words(uint64_t b, uint32_t (&w)[12]) {
  u32x8_t x;
  u32x4 y;
  asm("s_load_dwordx8 %0, %2, 0x0\n\ts_load_dwordx4 %1, %2, 0x20\n\ts_waitcnt lgkmcnt(0)"
      : "=&s"(x), "=&s"(y)
      : "s"(b));
  for (int i = 0; i < 8; ++i) w[i] = x[i];
  for (int i = 0; i < 4; ++i) w[8 + i] = y[i];
}
template <class T>
__device__ __forceinline__ T ld_table(const T *p) {
  static_assert(sizeof(T) % 4 == 0, "table entries are whole dwords");
  uint32_t w[sizeof(T) / 4];
  sload_words(uniform_u64(reinterpret_cast<uint64_t>(p)), w);
  T r;
  __builtin_memcpy(&r, w, sizeof(T));
  return r;
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds + 16 l (the LDS address must be uniform across the wave).
__device__ __forceinline__ void load_lds16(const void *g, void *lds) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds(g, (lds_void *)(lds), 16, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work item (batch-head, work tile) of workgroup `bid` when n = n_tiles * BH
// items run on a grid of xcd_grid(n) workgroups; work tiles come sorted by
// decreasing cost.  Workgroup i is dispatched to XCD i mod 8, and each XCD
// has its own L2.  With BH a multiple of 8, XCD x takes the BH / 8 whole
// batch-heads x BH / 8 .. (x + 1) BH / 8 - 1, one after the other, each tile
// by tile: the workgroups an XCD runs side by side then share one head and
// read its K/V (or Q/dO) tiles from that L2, and every XCD gets the same mix
// of costs.  Otherwise items go out with the batch-head fastest (an XCD
// split by heads would leave some XCDs only the costly tiles).  False for
// padding workgroups.
__device__ __forceinline__ bool xcd_item(int64_t bid, int64_t n_tiles, int BH, int &bh, int64_t &tile) {
  const int64_t n = n_tiles * BH;
  if (BH % 8 == 0) {
    const int64_t i = (bid & 7) * (n / 8) + (bid >> 3);
    bh = static_cast<int>(i / n_tiles);
    tile = i - static_cast<int64_t>(bh) * n_tiles;
    return true;  // the grid is exactly n workgroups
  }
  if (bid >= n) return false;
  bh = static_cast<int>(bid % BH);
  tile = bid / BH;
  return true;
}
// Grid size for n items mapped by xcd_item: 8 ceil(n / 8).
inline int64_t xcd_grid(int64_t n) { return (n + 7) / 8 * 8; }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max / sum over the lane pair (l, l ^ 32), returned in both lanes: one
// v_permlane32_swap (lanes 32..63 of the first operand trade places with
// lanes 0..31 of the second) instead of a round trip through LDS
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scheduling hint for a run of N MFMAs, each fed by R LDS operand reads:
// keep the reads of D products in flight ahead of the products that consume
// them.
template <int N, int D, int R = 1>
__device__ __forceinline__ void sched_lds_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, D * R, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < N - D; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, D, 0);
}

// Weights of the log-sum-exp merge of two normalised partials of one row
// (Striped Attention Guide, "Algorithmic Mechanics" 1, steps 4-6, with each
// partial already divided by its own row sum): LSE = M + ln(e^{la-M} + e^{lp-M}),
// O = wa O_acc + wp O_part.  Two empty rows (-inf) give weights 0 and -inf.
__device__ __forceinline__ void merge_weights(float la, float lp, float &wa, float &wp,
                                              float &lse) {
  const float M = fmaxf(la, lp);
  if (M == -INFINITY) {
    wa = 0.f;
    wp = 0.f;
    lse = -INFINITY;
    return;
  }
  const float ea = expf(la - M), ep = expf(lp - M);
  lse = M + logf(ea + ep);
  wa = expf(la - lse);
  wp = expf(lp - lse);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

}  // namespace dfa

