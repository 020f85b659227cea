// attn_fwd_f32.hip -- fp32 forward of blockwise causal attention (vector ALU).
//
// The fp32 path serves small problems (e.g. one head, N = 1024, d = 64) where
// exactness to 1e-4 matters more than speed.  One workgroup of 64 threads
// owns 64 query rows of a query piece; each thread owns one row and keeps its
// running max, sum and output in registers while the workgroup streams
// 64-key K/V tiles of the piece's blocks, in the host table's order, through LDS.
// The update is the online-softmax rescaling of the Striped Attention Guide,
// "Algorithmic Mechanics" 1, steps 1-7.  With packed documents a key is also
// invisible when it lies before the first position of the query's document
// (same page, "Production Deployment and Best Practices", item 3).
#include "device_util.h"
#include "dfa_internal.h"

namespace dfa {
namespace {

constexpr int TQ = kF32TileQ;
constexpr int TK = 32;

template <int HD, int OUT>
__global__ __launch_bounds__(TQ) void fwd_f32_kernel(FwdArgs a) {
  __shared__ float ks[TK][HD + 1];
  __shared__ float vs[TK][HD + 1];
  const int tid = threadIdx.x;
  const Geom &G = a.g;
  const int BH = G.batch * G.hq;
  const int64_t bid = blockIdx.x;
  const int bh = static_cast<int>(bid % BH);
  const int64_t ti = bid / BH;
  const int b = bh / G.hq, h = bh % G.hq, hk = h / G.group;
  QSeg seg;
  int64_t qt;
  if (a.segs) {
    const Tile t = a.tiles[ti];
    seg = a.segs[t.seg];
    qt = t.tile;
  } else {
    seg = a.seg0;
    qt = ti;
  }
  const int64_t row = qt * TQ + tid;
  const bool valid = row < seg.len_q;
  const int64_t rlast = ((qt + 1) * TQ < seg.len_q ? (qt + 1) * TQ : seg.len_q) - 1;
  const int64_t qpos = piece_pos(seg.q_start, seg.stride, seg.run, valid ? row : rlast);
  // packed documents: this row sees keys at positions >= qlo only; wlo is
  // the bound of the workgroup's first row (the smallest: positions rise)
  int64_t qlo = 0, wlo = 0, dhi;
  if (G.n_docs) {
    doc_range(G.docs, G.n_docs, qpos, qlo, dhi);
    doc_range(G.docs, G.n_docs, piece_pos(seg.q_start, seg.stride, seg.run, qt * TQ), wlo, dhi);
  }

  const float *qp = static_cast<const float *>(a.q) + b * G.qs[0] + h * G.qs[2];
  const float *kp = static_cast<const float *>(a.k) + b * G.ks[0] + hk * G.ks[2];
  const float *vp = static_cast<const float *>(a.v) + b * G.vs[0] + hk * G.vs[2];

  float qv[HD], acc[HD];
  if (valid) {
    const float *src = qp + piece_pos(seg.q_start, seg.stride, seg.run, row) * G.qs[1];
#pragma unroll
    for (int c = 0; c < HD; ++c) qv[c] = src[c];
  } else {
#pragma unroll
    for (int c = 0; c < HD; ++c) qv[c] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < HD; ++c) acc[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nblk = a.segs ? seg.blk_count : 1;
  for (int k = 0; k < nblk; ++k) {
    const KvRef r = a.segs ? a.kv[seg.blk_begin + k] : a.kv0;
    // keys at or before the tile's last query row
    const int64_t hi = piece_count_le(r.kv_start, seg.stride, seg.run, r.len_kv,
                                      piece_pos(seg.q_start, seg.stride, seg.run, rlast));
    // keys before wlo are invisible to every row of the workgroup
    const int64_t jlo = piece_count_le(r.kv_start, seg.stride, seg.run, r.len_kv, wlo - 1);
    for (int64_t j0 = jlo / TK * TK; j0 < hi; j0 += TK) {
      __syncthreads();
      for (int e = tid; e < TK * HD; e += TQ) {
        const int jj = e / HD, c = e % HD;
        const int64_t j = j0 + jj;
        float kvk = 0.f, kvv = 0.f;
        if (j < r.len_kv) {
          const int64_t pos = piece_pos(r.kv_start, seg.stride, seg.run, j);
          kvk = kp[pos * G.ks[1] + c];
          kvv = vp[pos * G.vs[1] + c];
        }
        ks[jj][c] = kvk;
        vs[jj][c] = kvv;
      }
      __syncthreads();
      float x[TK];
      float mx = -INFINITY;
      for (int jj = 0; jj < TK; ++jj) {
        const int64_t j = j0 + jj;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < HD; ++c) s = fmaf(qv[c], ks[jj][c], s);
        s *= G.scale;
        const int64_t kpos = piece_pos(r.kv_start, seg.stride, seg.run, j);
        const bool vis = j < r.len_kv && kpos <= qpos && kpos >= qlo;
        x[jj] = vis ? s : -INFINITY;
        mx = fmaxf(mx, x[jj]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = expf(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < HD; ++c) acc[c] *= alpha;
      for (int jj = 0; jj < TK; ++jj) {
        const float p = expf(x[jj] - m_use);
        l_run += p;
#pragma unroll
        for (int c = 0; c < HD; ++c) acc[c] = fmaf(p, vs[jj][c], acc[c]);
      }
      m_run = m_new;
    }
  }
  if (!valid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
  if (OUT == 0) {
    const int64_t pos = piece_pos(seg.q_start, seg.stride, seg.run, row);
    float *op = static_cast<float *>(a.o) + b * G.os[0] + pos * G.os[1] + h * G.os[2];
#pragma unroll
    for (int c = 0; c < HD; ++c) op[c] = acc[c] * inv;
    a.lse[(static_cast<int64_t>(b) * G.hq + h) * G.seqlen + pos] = lse;
  } else if (OUT == 2) {
    // merge into the accumulator row (one ring step's rows are distinct)
    const int64_t arow = (static_cast<int64_t>(b) * G.hq + h) * G.seqlen +
                         piece_pos(seg.q_start, seg.stride, seg.run, row);
    float *ao = static_cast<float *>(a.o) + arow * HD;
    float wa, wp, lnew;
    merge_weights(a.lse[arow], lse, wa, wp, lnew);
    wp *= inv;
#pragma unroll
    for (int c = 0; c < HD; ++c) ao[c] = (wa == 0.f ? 0.f : wa * ao[c]) + (wp == 0.f ? 0.f : wp * acc[c]);
    a.lse[arow] = lnew;
  } else {
    const int64_t prow = seg.part_off + (static_cast<int64_t>(b) * G.hq + h) * seg.len_q + row;
    float *op = static_cast<float *>(a.o) + prow * HD;
#pragma unroll
    for (int c = 0; c < HD; ++c) op[c] = acc[c] * inv;
    a.lse[prow] = lse;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 gr(static_cast<unsigned>(grid)), bl(TQ);
  if (hd == 128) {
    if (a.out_mode == 0)
      hipLaunchKernelGGL((fwd_f32_kernel<128, 0>), gr, bl, 0, s, a);
    else if (a.out_mode == 2)
      hipLaunchKernelGGL((fwd_f32_kernel<128, 2>), gr, bl, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_f32_kernel<128, 1>), gr, bl, 0, s, a);
  } else if (hd == 64) {
    if (a.out_mode == 0)
      hipLaunchKernelGGL((fwd_f32_kernel<64, 0>), gr, bl, 0, s, a);
    else if (a.out_mode == 2)
      hipLaunchKernelGGL((fwd_f32_kernel<64, 2>), gr, bl, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_f32_kernel<64, 1>), gr, bl, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfa
