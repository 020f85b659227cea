// rope.hip -- rotary position embedding at absolute positions (Striped
// Attention Guide, "Preserving Rotary Position Embeddings (RoPE)": every
// token vector turns by its absolute sequence index before the ring
// exchange, so striping the storage changes no angle).  Pair c =
// (x[2c], x[2c+1]) of the token at position p turns by p * base^(-2c/d)
// (RoFormer's interleaved form); the inverse turns back (the transpose, for
// gradients).
//
// The tensors hold global token order, so a token's absolute position is
// its index plus pos_offset: the pages' "m * P + p" for local row m of rank
// p is exactly the global index of that row.
//
// Bound by HBM (one read and one write per element).  One thread per
// (token, 16 bytes of pairs) -- one pair when rows are not 16-byte aligned:
// consecutive threads cover consecutive pairs of a row, so a wave reads
// whole rows; the angles, their cosines and sines are computed once in fp64
// and reused for every batch entry and head; each output is rounded once
// from the fp64 result.
#include "dfa_internal.h"

namespace dfa {
namespace {

constexpr int kRopeThreads = 256;

// PPT consecutive pairs per thread: 16-byte accesses when rows allow them.
template <typename T, int PPT>
struct Vec {
  typedef T v __attribute__((ext_vector_type(2 * PPT)));
};

template <typename T, int PPT>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeArgs a) {
  using V = typename Vec<T, PPT>::v;
  const int lanes = a.head_dim / (2 * PPT);  // threads per row
  const int tok_per_block = kRopeThreads / lanes;
  const int tid = threadIdx.x;
  const int tl = tid / lanes, c0 = (tid % lanes) * PPT;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * tok_per_block + tl;
  if (tl >= tok_per_block || t >= a.seqlen) return;
  double sn[PPT], cs[PPT];
#pragma unroll
  for (int u = 0; u < PPT; ++u) {
    const double theta = static_cast<double>(a.pos_offset + t) *
                         pow(a.base, -2.0 * static_cast<double>(c0 + u) / a.head_dim);
    sincos(theta, &sn[u], &cs[u]);
    if (a.inverse) sn[u] = -sn[u];
  }
  const T *x = static_cast<const T *>(a.x);
  T *y = static_cast<T *>(a.y);
  for (int b = 0; b < a.batch; ++b) {
    const T *xr = x + b * a.xs[0] + t * a.xs[1] + 2 * c0;
    T *yr = y + b * a.ys[0] + t * a.ys[1] + 2 * c0;
#pragma unroll 4
    for (int h = 0; h < a.heads; ++h) {
      const V v = *reinterpret_cast<const V *>(xr + h * a.xs[2]);
      V o;
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const double x0 = static_cast<double>(static_cast<float>(v[2 * u]));
        const double x1 = static_cast<double>(static_cast<float>(v[2 * u + 1]));
        o[2 * u] = static_cast<T>(static_cast<float>(x0 * cs[u] - x1 * sn[u]));
        o[2 * u + 1] = static_cast<T>(static_cast<float>(x0 * sn[u] + x1 * cs[u]));
      }
      *reinterpret_cast<V *>(yr + h * a.ys[2]) = o;
    }
  }
}

template <typename T, int PPT>
hipError_t launch_rope_t(const RopeArgs &a, hipStream_t s) {
  const int tok_per_block = kRopeThreads / (a.head_dim / (2 * PPT));
  const int64_t grid = (a.seqlen + tok_per_block - 1) / tok_per_block;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((rope_kernel<T, PPT>), dim3(static_cast<unsigned>(grid)), dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, int dtype_bf16, hipStream_t s) {
  if (a.seqlen <= 0) return hipSuccess;
  // 16-byte accesses need every row start 16-byte aligned and whole vectors per row
  const int64_t el = dtype_bf16 ? 8 : 4;  // elements per 16 bytes
  bool vec = a.head_dim % el == 0 && reinterpret_cast<uintptr_t>(a.x) % 16 == 0 &&
             reinterpret_cast<uintptr_t>(a.y) % 16 == 0;
  for (int i = 0; i < 3; ++i) vec = vec && a.xs[i] % el == 0 && a.ys[i] % el == 0;
  if (dtype_bf16) return vec ? launch_rope_t<__bf16, 4>(a, s) : launch_rope_t<__bf16, 1>(a, s);
  return vec ? launch_rope_t<float, 2>(a, s) : launch_rope_t<float, 1>(a, s);
}

}  // namespace dfa
