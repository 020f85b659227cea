// attn_bwd_f32.hip -- fp32 backward of blockwise causal attention (vector ALU).
//
// Probabilities are recomputed from the saved log-sum-exp instead of being
// stored (FlashAttention glossary page, first two paragraphs):
//   P_ij = e^{scale q_i.k_j - LSE_i},  dP_ij = dO_i.v_j,
//   dS_ij = P_ij (dP_ij - D_i) with D_i = rowsum(dO_i * O_i),
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//   dV_j = sum_i P_ij dO_i.
// Packed documents restrict every pair to one document (Striped Attention
// Guide, "Production Deployment and Best Practices", item 3).
// Two kernels, neither with atomics: a query-major one owns dQ rows and walks
// each query piece's blocks; a key-major one owns dK/dV rows, walks the blocks
// that read its key piece and sums over the query heads of its group.
#include "device_util.h"
#include "dfa_internal.h"

#include <stdint.h>

namespace dfa {
namespace {

constexpr int TQ = kF32TileQ;
constexpr int TK = kF32TileKV;
constexpr int TS = 32;  // streamed rows per LDS tile

template <int HD>
__global__ __launch_bounds__(TQ) void dq_f32_kernel(BwdArgs a) {
  __shared__ float ks[TS][HD + 1];
  __shared__ float vs[TS][HD + 1];
  const int tid = threadIdx.x;
  const Geom &G = a.g;
  const int BH = G.batch * G.hq;
  const int64_t bid = blockIdx.x;
  const int bh = static_cast<int>(bid % BH);
  const Tile tl = a.qtiles[bid / BH];
  const QSeg seg = a.qsegs[tl.seg];
  const int b = bh / G.hq, h = bh % G.hq, hk = h / G.group;
  const int64_t row = static_cast<int64_t>(tl.tile) * TQ + tid;
  const bool valid = row < seg.len_q;
  const int64_t rlast = ((tl.tile + 1LL) * TQ < seg.len_q ? (tl.tile + 1LL) * TQ : seg.len_q) - 1;
  const float *qp = static_cast<const float *>(a.q) + b * G.qs[0] + h * G.qs[2];
  const float *dop = static_cast<const float *>(a.dout) + b * G.os[0] + h * G.os[2];
  const float *kp = static_cast<const float *>(a.k) + b * G.ks[0] + hk * G.ks[2];
  const float *vp = static_cast<const float *>(a.v) + b * G.vs[0] + hk * G.vs[2];
  float qv[HD], dov[HD], acc[HD];
  float lse = 0.f, dd = 0.f;
  int64_t pos = 0;
  // packed documents: keys before qlo are invisible to this row, before wlo
  // to every row of the workgroup
  int64_t qlo = 0, wlo = 0, dhi;
  if (G.n_docs) {
    doc_range(G.docs, G.n_docs, piece_pos(seg.q_start, seg.stride, seg.run, valid ? row : rlast), qlo, dhi);
    doc_range(G.docs, G.n_docs, piece_pos(seg.q_start, seg.stride, seg.run, tl.tile * static_cast<int64_t>(TQ)),
              wlo, dhi);
  }
  if (valid) {
    pos = piece_pos(seg.q_start, seg.stride, seg.run, row);
#pragma unroll
    for (int c = 0; c < HD; ++c) {
      qv[c] = qp[pos * G.qs[1] + c];
      dov[c] = dop[pos * G.os[1] + c];
    }
    lse = a.lse[(static_cast<int64_t>(b) * G.hq + h) * G.seqlen + pos];
    dd = a.dd[(static_cast<int64_t>(b) * G.hq + h) * G.seqlen + pos];
  } else {
#pragma unroll
    for (int c = 0; c < HD; ++c) qv[c] = dov[c] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < HD; ++c) acc[c] = 0.f;
  for (int k = 0; k < seg.blk_count; ++k) {
    const KvRef r = a.qkv[seg.blk_begin + k];
    // keys at or before the tile's last query row
    const int64_t hi = piece_count_le(r.kv_start, seg.stride, seg.run, r.len_kv,
                                      piece_pos(seg.q_start, seg.stride, seg.run, rlast));
    const int64_t jlo = piece_count_le(r.kv_start, seg.stride, seg.run, r.len_kv, wlo - 1);
    for (int64_t j0 = jlo / TS * TS; j0 < hi; j0 += TS) {
      __syncthreads();
      for (int e = tid; e < TS * HD; e += TQ) {
        const int jj = e / HD, c = e % HD;
        const int64_t j = j0 + jj;
        float x = 0.f, y = 0.f;
        if (j < r.len_kv) {
          const int64_t kpos = piece_pos(r.kv_start, seg.stride, seg.run, j);
          x = kp[kpos * G.ks[1] + c];
          y = vp[kpos * G.vs[1] + c];
        }
        ks[jj][c] = x;
        vs[jj][c] = y;
      }
      __syncthreads();
      if (!valid) continue;
      for (int jj = 0; jj < TS; ++jj) {
        const int64_t j = j0 + jj;
        if (j >= r.len_kv) continue;
        const int64_t kpos = piece_pos(r.kv_start, seg.stride, seg.run, j);
        if (kpos > pos || kpos < qlo) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < HD; ++c) {
          s = fmaf(qv[c], ks[jj][c], s);
          dp = fmaf(dov[c], vs[jj][c], dp);
        }
        const float p = expf(s * G.scale - lse);
        const float ds = p * (dp + dd) * G.scale;  // dd holds -D
#pragma unroll
        for (int c = 0; c < HD; ++c) acc[c] = fmaf(ds, ks[jj][c], acc[c]);
      }
    }
  }
  if (!valid) return;
  float *out = static_cast<float *>(a.dq) + b * G.qs[0] + pos * G.qs[1] + h * G.qs[2];
#pragma unroll
  for (int c = 0; c < HD; ++c) out[c] = acc[c];
}

template <int HD>
__global__ __launch_bounds__(TK) void dkdv_f32_kernel(BwdArgs a) {
  __shared__ float qs_[TS][HD + 1];
  __shared__ float ds_[TS][HD + 1];
  __shared__ float ls_[TS], dd_[TS];
  const int tid = threadIdx.x;
  const Geom &G = a.g;
  const int BH = G.batch * G.hkv;
  const int64_t bid = blockIdx.x;
  const int bh = static_cast<int>(bid % BH);
  const Tile tl = a.kvtiles[bid / BH];
  const KvSeg seg = a.kvsegs[tl.seg];
  const int b = bh / G.hkv, hk = bh % G.hkv;
  const int64_t j = static_cast<int64_t>(tl.tile) * TK + tid;
  const int64_t j0 = static_cast<int64_t>(tl.tile) * TK;
  const bool valid = j < seg.len_kv;
  const float *kp = static_cast<const float *>(a.k) + b * G.ks[0] + hk * G.ks[2];
  const float *vp = static_cast<const float *>(a.v) + b * G.vs[0] + hk * G.vs[2];
  float kv_[HD], vv[HD], dk[HD], dv[HD];
  int64_t pos = 0;
  // packed documents: queries at or after khi cannot see this key, at or
  // after whi no key of the workgroup (the largest bound: positions rise)
  int64_t khi = INT64_MAX, whi = INT64_MAX, dlo;
  if (G.n_docs) {
    const int64_t jl = (j0 + TK < seg.len_kv ? j0 + TK : seg.len_kv) - 1;
    doc_range(G.docs, G.n_docs, piece_pos(seg.kv_start, seg.stride, seg.run, valid ? j : jl), dlo, khi);
    doc_range(G.docs, G.n_docs, piece_pos(seg.kv_start, seg.stride, seg.run, jl), dlo, whi);
  }
  if (valid) {
    pos = piece_pos(seg.kv_start, seg.stride, seg.run, j);
#pragma unroll
    for (int c = 0; c < HD; ++c) {
      kv_[c] = kp[pos * G.ks[1] + c];
      vv[c] = vp[pos * G.vs[1] + c];
    }
  } else {
#pragma unroll
    for (int c = 0; c < HD; ++c) kv_[c] = vv[c] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < HD; ++c) dk[c] = dv[c] = 0.f;
  for (int gi = 0; gi < G.group; ++gi) {
    const int h = hk * G.group + gi;
    const float *qp = static_cast<const float *>(a.q) + b * G.qs[0] + h * G.qs[2];
    const float *dop = static_cast<const float *>(a.dout) + b * G.os[0] + h * G.os[2];
    const float *lsep = a.lse + (static_cast<int64_t>(b) * G.hq + h) * G.seqlen;
    const float *ddp = a.dd + (static_cast<int64_t>(b) * G.hq + h) * G.seqlen;
    for (int k = 0; k < seg.blk_count; ++k) {
      const QRef r = a.kvq[seg.blk_begin + k];
      // the first query row at or after the tile's first key
      const int64_t lo = piece_count_le(r.q_start, seg.stride, seg.run, r.len_q,
                                        piece_pos(seg.kv_start, seg.stride, seg.run, j0) - 1);
      const int64_t iend = G.n_docs ? piece_count_le(r.q_start, seg.stride, seg.run, r.len_q, whi - 1) : r.len_q;
      for (int64_t i0 = lo; i0 < iend; i0 += TS) {
        __syncthreads();
        for (int e = tid; e < TS * HD; e += TK) {
          const int ii = e / HD, c = e % HD;
          const int64_t i = i0 + ii;
          float x = 0.f, y = 0.f;
          if (i < r.len_q) {
            const int64_t qpos = piece_pos(r.q_start, seg.stride, seg.run, i);
            x = qp[qpos * G.qs[1] + c];
            y = dop[qpos * G.os[1] + c];
          }
          qs_[ii][c] = x;
          ds_[ii][c] = y;
        }
        if (tid < TS) {
          const int64_t i = i0 + tid;
          const int64_t qpos = piece_pos(r.q_start, seg.stride, seg.run, i < r.len_q ? i : 0);
          ls_[tid] = i < r.len_q ? lsep[qpos] : 0.f;
          dd_[tid] = i < r.len_q ? ddp[qpos] : 0.f;
        }
        __syncthreads();
        if (!valid) continue;
        for (int ii = 0; ii < TS; ++ii) {
          const int64_t i = i0 + ii;
          if (i >= r.len_q) continue;
          const int64_t qpos = piece_pos(r.q_start, seg.stride, seg.run, i);
          if (pos > qpos || qpos >= khi) continue;
          float s = 0.f, dp = 0.f;
#pragma unroll
          for (int c = 0; c < HD; ++c) {
            s = fmaf(qs_[ii][c], kv_[c], s);
            dp = fmaf(ds_[ii][c], vv[c], dp);
          }
          const float p = expf(s * G.scale - ls_[ii]);
          const float dsv = p * (dp + dd_[ii]) * G.scale;  // dd_ holds -D
#pragma unroll
          for (int c = 0; c < HD; ++c) {
            dk[c] = fmaf(dsv, qs_[ii][c], dk[c]);
            dv[c] = fmaf(p, ds_[ii][c], dv[c]);
          }
        }
      }
    }
  }
  if (!valid) return;
  float *ok = static_cast<float *>(a.dk) + b * G.ks[0] + pos * G.ks[1] + hk * G.ks[2];
  float *ov = static_cast<float *>(a.dv) + b * G.vs[0] + pos * G.vs[1] + hk * G.vs[2];
#pragma unroll
  for (int c = 0; c < HD; ++c) {
    ok[c] = dk[c];
    ov[c] = dv[c];
  }
}

}  // namespace

hipError_t launch_bwd_dq_f32(const BwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (hd == 128)
    hipLaunchKernelGGL(dq_f32_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(TQ), 0, s, a);
  else
    hipLaunchKernelGGL(dq_f32_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(TQ), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const BwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (hd == 128)
    hipLaunchKernelGGL(dkdv_f32_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(TK), 0, s, a);
  else
    hipLaunchKernelGGL(dkdv_f32_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(TK), 0, s, a);
  return hipGetLastError();
}

}  // namespace dfa
