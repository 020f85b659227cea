// rowwise.hip -- HBM-bound row kernels: accumulator init, log-sum-exp merge,
// finalisation, zero fill and the backward's D = rowsum(dO * O) (stored as -D).
//
// Merge rule (Striped Attention Guide, "Algorithmic Mechanics" 1, steps 4-7,
// written for partials that are already normalised): with
// M = max(LSE_a, LSE_b), LSE = M + ln(e^{LSE_a-M} + e^{LSE_b-M}) and
// O = e^{LSE_a-LSE} O_a + e^{LSE_b-LSE} O_b.  Two empty rows (LSE = -inf)
// merge to O = 0, LSE = -inf: the max is tested before any subtraction, so
// -inf - -inf never occurs.
#include "device_util.h"
#include "dfa_internal.h"

namespace dfa {
namespace {

constexpr int NT = 256;

// one thread per (row, 4 floats); HD/4 threads of a row sit in one wave
template <int HD>
__global__ __launch_bounds__(NT) void merge_rows_kernel(float *o_acc, float *lse_acc,
                                                        const float *o_part,
                                                        const float *lse_part, int64_t n_rows) {
  constexpr int C4 = HD / 4;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
  if (tid >= n_rows * C4) return;
  const int64_t r = tid / C4;
  const int c = static_cast<int>(tid % C4);
  float wa, wp, lse;
  merge_weights(lse_acc[r], lse_part[r], wa, wp, lse);
  f32x4 *oa = reinterpret_cast<f32x4 *>(o_acc + r * HD) + c;
  const f32x4 op = reinterpret_cast<const f32x4 *>(o_part + r * HD)[c];
  const f32x4 av = *oa;
  f32x4 res;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    res[e] = (wa == 0.f ? 0.f : wa * av[e]) + (wp == 0.f ? 0.f : wp * op[e]);
  *oa = res;
  if (c == 0) lse_acc[r] = lse;
}

__global__ __launch_bounds__(NT) void acc_init_kernel(float *o_acc, float *lse_acc, int64_t rows,
                                                      int hd) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
  const int64_t c4 = hd / 4;
  if (tid < rows * c4) reinterpret_cast<f32x4 *>(o_acc)[tid] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (tid < rows) lse_acc[tid] = -INFINITY;
}

// acc [B][Hq][N][HD] -> O[b][pos][h][:] (dtype) and lse [B][Hq][N]
template <int HD, bool BF16>
__global__ __launch_bounds__(NT) void finalize_kernel(const float *o_acc, const float *lse_acc,
                                                      void *o, int64_t os0, int64_t os1,
                                                      int64_t os2, float *lse, int hq,
                                                      int64_t n, int64_t rows) {
  constexpr int C4 = HD / 4;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
  if (tid >= rows * C4) return;
  const int64_t r = tid / C4;
  const int c = static_cast<int>(tid % C4);
  const int64_t bh = r / n, pos = r % n;
  const int64_t b = bh / hq, h = bh % hq;
  const f32x4 v = reinterpret_cast<const f32x4 *>(o_acc + r * HD)[c];
  const int64_t off = b * os0 + pos * os1 + h * os2 + 4 * c;
  if (BF16) {
    bf16x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = static_cast<__bf16>(v[e]);
    *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(o) + off) = w;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + off) = v;
  }
  if (c == 0) lse[r] = lse_acc[r];
}

// x[b][t][h][:] = 0 for every row (16 bytes per thread); lse = -inf
__global__ __launch_bounds__(NT) void zero_rows_kernel(char *x, int64_t s0, int64_t s1, int64_t s2,
                                                       int esize, int heads, int64_t n,
                                                       int row_bytes, float *lse, int64_t rows) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
  const int c16 = row_bytes / 16;
  if (tid < rows * c16) {
    const int64_t r = tid / c16;
    const int c = static_cast<int>(tid % c16);
    const int64_t b = r / (n * heads), rem = r % (n * heads);
    const int64_t t = rem / heads, h = rem % heads;
    st16(x + esize * (b * s0 + t * s1 + h * s2) + 16 * c, u32x4{0, 0, 0, 0});
  }
  if (lse && tid < rows) lse[tid] = -INFINITY;  // [B][H][N] has the same row count
}

// -D[b][h][pos] = -sum_c dO[b][pos][h][c] * O[b][pos][h][c] (stored negated: the
// gradient kernels start their dP accumulators from it) and LSE*log2(e).
// A row is read by LPR lanes, 16 contiguous bytes each, so every load of a
// wave covers RPW whole rows; each lane keeps U rows' loads in flight, then
// the row's partial sums meet in a butterfly over its LPR lanes.
template <int HD, bool BF16>
__global__ __launch_bounds__(NT) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPL = BF16 ? 8 : 4;  // elements per 16-byte load
  constexpr int LPR = HD / EPL;      // lanes per row
  constexpr int RPW = 64 / LPR;      // rows per wave and load
  constexpr int U = 4;               // rows per lane
  static_assert(HD % EPL == 0 && 64 % LPR == 0, "a row is a whole number of lanes");
  const Geom &G = a.g;
  const int lane = threadIdx.x & 63, sub = lane % LPR, grp = lane / LPR;
  const int64_t rows = static_cast<int64_t>(G.batch) * G.hq * G.seqlen;
  const int64_t r0 = ((static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x) >> 6) * (RPW * U);
  if (r0 >= rows) return;  // wave-uniform
  const int esz = BF16 ? 2 : 4;
  const char *ob = static_cast<const char *>(a.o), *db = static_cast<const char *>(a.dout);
  u32x4 ov[U], dv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = r0 + u * RPW + grp;
    if (r < rows) {
      const int64_t bh = r / G.seqlen, pos = r % G.seqlen;
      const int64_t off = esz * ((bh / G.hq) * G.os[0] + pos * G.os[1] + (bh % G.hq) * G.os[2]) + 16 * sub;
      ov[u] = ld16(ob + off);
      dv[u] = ld16(db + off);
    } else {
      ov[u] = dv[u] = u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (BF16) {
        s = fmaf(__uint_as_float(ov[u][e] << 16), __uint_as_float(dv[u][e] << 16), s);
        s = fmaf(__uint_as_float(ov[u][e] & 0xffff0000u), __uint_as_float(dv[u][e] & 0xffff0000u), s);
      } else {
        s = fmaf(__uint_as_float(ov[u][e]), __uint_as_float(dv[u][e]), s);
      }
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m);
    const int64_t r = r0 + u * RPW + grp;
    if (sub == 0 && r < rows) {
      a.dd[r] = -s;
      a.lse2[r] = a.lse[r] * kLog2e;
    }
  }
}

inline unsigned blocks_for(int64_t threads) { return static_cast<unsigned>((threads + NT - 1) / NT); }

}  // namespace

hipError_t launch_acc_init(float *o_acc, float *lse_acc, int64_t rows, int hd, hipStream_t s) {
  const int64_t th = rows * (hd / 4) > rows ? rows * (hd / 4) : rows;
  if (th == 0) return hipSuccess;
  hipLaunchKernelGGL(acc_init_kernel, dim3(blocks_for(th)), dim3(NT), 0, s, o_acc, lse_acc, rows, hd);
  return hipGetLastError();
}

hipError_t launch_merge_rows(float *o_acc, float *lse_acc, const float *o_part,
                             const float *lse_part, int64_t n_rows, int hd, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const int64_t th = n_rows * (hd / 4);
  if (hd == 128)
    hipLaunchKernelGGL(merge_rows_kernel<128>, dim3(blocks_for(th)), dim3(NT), 0, s, o_acc,
                       lse_acc, o_part, lse_part, n_rows);
  else
    hipLaunchKernelGGL(merge_rows_kernel<64>, dim3(blocks_for(th)), dim3(NT), 0, s, o_acc,
                       lse_acc, o_part, lse_part, n_rows);
  return hipGetLastError();
}

hipError_t launch_finalize(const float *o_acc, const float *lse_acc, void *o, const int64_t os[3],
                           int dtype, float *lse, int batch, int hq, int64_t n, int hd,
                           hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(batch) * hq * n;
  if (rows == 0) return hipSuccess;
  const int64_t th = rows * (hd / 4);
  dim3 gr(blocks_for(th)), bl(NT);
  const bool bf = dtype == 1;
  if (hd == 128 && bf)
    hipLaunchKernelGGL((finalize_kernel<128, true>), gr, bl, 0, s, o_acc, lse_acc, o, os[0], os[1], os[2], lse, hq, n, rows);
  else if (hd == 128)
    hipLaunchKernelGGL((finalize_kernel<128, false>), gr, bl, 0, s, o_acc, lse_acc, o, os[0], os[1], os[2], lse, hq, n, rows);
  else if (bf)
    hipLaunchKernelGGL((finalize_kernel<64, true>), gr, bl, 0, s, o_acc, lse_acc, o, os[0], os[1], os[2], lse, hq, n, rows);
  else
    hipLaunchKernelGGL((finalize_kernel<64, false>), gr, bl, 0, s, o_acc, lse_acc, o, os[0], os[1], os[2], lse, hq, n, rows);
  return hipGetLastError();
}

hipError_t launch_zero_rows(void *x, const int64_t strides[3], int dtype, int batch, int64_t n,
                            int heads, int hd, float *lse, hipStream_t s) {
  const int esize = dtype == 1 ? 2 : 4;
  const int row_bytes = hd * esize;
  const int64_t rows = static_cast<int64_t>(batch) * n * heads;
  if (rows == 0) return hipSuccess;
  const int64_t th = rows * (row_bytes / 16);
  hipLaunchKernelGGL(zero_rows_kernel, dim3(blocks_for(th)), dim3(NT), 0, s,
                     static_cast<char *>(x), strides[0], strides[1], strides[2], esize, heads, n,
                     row_bytes, lse, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdArgs &a, int dtype, int hd, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.g.batch) * a.g.hq * a.g.seqlen;
  if (rows == 0) return hipSuccess;
  // 64 threads per wave, each wave 4 * 64 / (hd / 8 or hd / 4) rows
  const int64_t rows_per_wave = 4 * 64 / (dtype == 1 ? hd / 8 : hd / 4);
  dim3 gr(blocks_for((rows + rows_per_wave - 1) / rows_per_wave * 64)), bl(NT);
  const bool bf = dtype == 1;
  if (hd == 128 && bf)
    hipLaunchKernelGGL((bwd_pre_kernel<128, true>), gr, bl, 0, s, a);
  else if (hd == 128)
    hipLaunchKernelGGL((bwd_pre_kernel<128, false>), gr, bl, 0, s, a);
  else if (bf)
    hipLaunchKernelGGL((bwd_pre_kernel<64, true>), gr, bl, 0, s, a);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<64, false>), gr, bl, 0, s, a);
  return hipGetLastError();
}

}  // namespace dfa
