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
// (token, pair): consecutive threads cover consecutive pairs of a row, so a
// wave reads whole rows; the angle, its cosine and sine are computed once in
// fp64 and reused for every batch entry and head; each output is rounded
// once from the fp64 result.
#include "dfa_internal.h"

namespace dfa {
namespace {

constexpr int kRopeThreads = 256;

template <typename T>
struct Pair;
template <>
struct Pair<__bf16> {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
};
template <>
struct Pair<float> {
  typedef float v2 __attribute__((ext_vector_type(2)));
};

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeArgs a) {
  using V2 = typename Pair<T>::v2;
  const int pairs = a.head_dim / 2;
  const int tok_per_block = kRopeThreads / pairs;
  const int tid = threadIdx.x;
  const int tl = tid / pairs, c = tid % pairs;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * tok_per_block + tl;
  if (tl >= tok_per_block || t >= a.seqlen) return;
  const double theta =
      static_cast<double>(a.pos_offset + t) * pow(a.base, -2.0 * static_cast<double>(c) / a.head_dim);
  double sn, cs;
  sincos(theta, &sn, &cs);
  if (a.inverse) sn = -sn;
  const T *x = static_cast<const T *>(a.x);
  T *y = static_cast<T *>(a.y);
  for (int b = 0; b < a.batch; ++b) {
    const T *xr = x + b * a.xs[0] + t * a.xs[1] + 2 * c;
    T *yr = y + b * a.ys[0] + t * a.ys[1] + 2 * c;
#pragma unroll 4
    for (int h = 0; h < a.heads; ++h) {
      const V2 v = *reinterpret_cast<const V2 *>(xr + h * a.xs[2]);
      const double x0 = static_cast<double>(static_cast<float>(v[0]));
      const double x1 = static_cast<double>(static_cast<float>(v[1]));
      V2 o;
      o[0] = static_cast<T>(static_cast<float>(x0 * cs - x1 * sn));
      o[1] = static_cast<T>(static_cast<float>(x0 * sn + x1 * cs));
      *reinterpret_cast<V2 *>(yr + h * a.ys[2]) = o;
    }
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, int dtype_bf16, hipStream_t s) {
  if (a.seqlen <= 0) return hipSuccess;
  const int tok_per_block = kRopeThreads / (a.head_dim / 2);
  const int64_t grid = (a.seqlen + tok_per_block - 1) / tok_per_block;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (dtype_bf16)
    hipLaunchKernelGGL(rope_kernel<__bf16>, dim3(static_cast<unsigned>(grid)), dim3(kRopeThreads), 0, s, a);
  else
    hipLaunchKernelGGL(rope_kernel<float>, dim3(static_cast<unsigned>(grid)), dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dfa
