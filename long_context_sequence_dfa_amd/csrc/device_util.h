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

// Read of a schedule table entry that stays constant for the whole launch:
// through the constant address space the compiler may use scalar loads and
// keep everything derived from the entry in scalar registers.
template <class T>
__device__ __forceinline__ T ld_table(const T *p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(const __attribute__((address_space(4))) T *)(p);
#else
  return *p;  // host pass only; never executed
#endif
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
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_swap32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

}  // namespace dfa

