// attn_fwd_bf16.hip -- bf16 forward of blockwise causal attention on gfx950.
//
// One workgroup (4 waves) owns 128 query rows of one query piece, one batch
// entry and one query head.  It walks the piece's blocks in ring-step order
// (the key/value shard a virtual rank holds at each step, read in place) and,
// inside each block, the 64-key tiles that hold at least one visible key.
// Per tile it keeps the running row max m, the running row sum l and the
// running output O, rescaling by alpha = e^{m_old - m_new} (Striped Attention
// Guide, "Algorithmic Mechanics" 1, steps 1-6), then normalises once at the
// end (step 7) and emits LSE = m + ln l.  Tiles past the causal limit are
// never visited and only tiles that straddle the diagonal evaluate the mask
// ("Algorithmic Mechanics" 2, intra- vs inter-block masking).
//
// gfx950 mapping:
//  * each wave computes S^T = K Q^T for 32 queries x 64 keys with
//    v_mfma_f32_32x32x16_bf16, so every lane owns one query column: the row
//    max and sum need only the lane's own 32 values plus one exchange with
//    lane l^32;
//  * key rows enter the MFMA in a bit-swapped order (kperm) so that the S^T
//    accumulator of a lane holds 8 consecutive keys per 16-key step -- exactly
//    the B operand of O^T = V^T P^T, so P goes from accumulator to MFMA
//    operand without touching LDS;
//  * V^T operands come straight from the row-major V tile in LDS through
//    ds_read_b64_tr_b16; the K and V tiles get different row pitches so that
//    both the b128 reads of K and the transposing reads of V are free of
//    bank conflicts;
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are
//    issued before the current tile's MFMAs;
//  * the vector ALU is the scarce unit next to the MFMAs, so the softmax is
//    kept lean: one FMA folds scale, log2(e) and the max into the exponent,
//    and the running output is rescaled only when a row's max grows by more
//    than 2^8 (exact: every probability is taken against the same reference
//    max as its row sum, and stays below 2^8).
// Score arithmetic runs in the log2 domain: x = s * scale * log2(e).
#include "device_util.h"
#include "dfa_internal.h"

namespace dfa {
namespace {

constexpr int BQ = kFwdTileQ;  // 128 query rows per workgroup
constexpr int BK = 64;         // keys per tile
constexpr int NT = 256;        // threads per workgroup

// Row order of key tiles inside the S^T MFMA: swaps bits 2 and 3 of the
// row index (see the header comment).
__device__ __forceinline__ int kperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

struct BlockWalk {
  int64_t kv_start, len_kv, diag, ntiles;
};

__device__ __forceinline__ BlockWalk block_walk(const FwdArgs &a, const QSeg &seg, int k,
                                                int64_t iend) {
  KvRef r = a.segs ? a.kv[seg.blk_begin + k] : a.kv0;
  BlockWalk w;
  w.kv_start = r.kv_start;
  w.len_kv = r.len_kv;
  w.diag = r.diag_offset;
  // the last row iend-1 sees keys j <= iend-1+diag
  int64_t hi = iend + r.diag_offset;
  if (hi > r.len_kv) hi = r.len_kv;
  w.ntiles = hi > 0 ? (hi + BK - 1) / BK : 0;
  return w;
}

template <int HD, int OUT>
__global__ __launch_bounds__(NT, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int KP = HD * 2 + 16;   // K tile pitch: b128 reads of 16 rows are conflict-free
  constexpr int VP = HD * 2 + 32;   // V tile pitch: transposing reads of 4 rows are conflict-free
  constexpr int KB = BK * KP;
  constexpr int BUF = KB + BK * VP;
  constexpr int KS = HD / 16;       // MFMA k-steps over head_dim
  constexpr int DT = HD / 32;       // 32-row output tiles over head_dim
  constexpr int CH = HD / 8;        // 16-byte chunks per row
  constexpr int RPP = NT / CH;      // rows per load pass
  constexpr int NP = BK / RPP;      // load passes per tile
  constexpr float TAU = 8.f;        // lazy rescale threshold (log2 units)
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c32 = lane & 31;
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
  const int64_t i0 = qt * BQ;
  const int64_t i0w = i0 + wave * 32;
  const int64_t iend = (i0 + BQ < seg.len_q) ? i0 + BQ : seg.len_q;
  const float c = G.scale_log2;

  const char *qb = static_cast<const char *>(a.q) + 2 * (b * G.qs[0] + h * G.qs[2]);
  const char *kb = static_cast<const char *>(a.k) + 2 * (b * G.ks[0] + hk * G.ks[2]);
  const char *vb = static_cast<const char *>(a.v) + 2 * (b * G.vs[0] + hk * G.vs[2]);
  const int64_t krs = 2 * G.ks[1] * seg.stride, vrs = 2 * G.vs[1] * seg.stride;  // bytes per row

  // Q^T operand (B of S^T = K Q^T): lane holds Q[row][16ks + 8g .. +8].
  // Rows past the piece read its last row (their outputs are never stored).
  bf16x8 qf[KS];
  {
    int64_t row = i0w + c32;
    row = row < seg.len_q ? row : seg.len_q - 1;
    const char *src = qb + 2 * (seg.q_start + row * seg.stride) * G.qs[1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(src + (2 * ks + g) * 16));
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- tile walk state ----
  int k = 0;
  BlockWalk cw{0, 0, 0, 0};
  const int nblk = a.segs ? seg.blk_count : 1;
  while (k < nblk) {
    cw = block_walk(a, seg, k, iend);
    if (cw.ntiles > 0) break;
    ++k;
  }

  const int lrow = tid / CH, lch = tid % CH;
  u32x4 kr[NP], vr[NP];
  // rows past the block's key piece re-read its last row; the mask zeroes them
  auto gload = [&](const BlockWalk &w, int64_t t) {
    const char *kp = kb + 2 * w.kv_start * G.ks[1] + lch * 16;
    const char *vp = vb + 2 * w.kv_start * G.vs[1] + lch * 16;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      int64_t j = t * BK + lrow + p * RPP;
      j = j < w.len_kv ? j : w.len_kv - 1;
      kr[p] = ld16(kp + j * krs);
      vr[p] = ld16(vp + j * vrs);
    }
  };
  auto lstore = [&](int buf) {
    char *kt = smem + buf * BUF;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      st16(kt + (lrow + p * RPP) * KP + lch * 16, kr[p]);
      st16(kt + KB + (lrow + p * RPP) * VP + lch * 16, vr[p]);
    }
  };

  int64_t t = 0;
  int cur = 0;
  if (k < nblk) {
    gload(cw, 0);
    lstore(0);
  }
  __syncthreads();

  const int kr0 = kperm(c32) * KP + g * 16;
  const int vrow = 8 * g + (lane & 15) / 4;
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int voff = vrow * VP + vcol * 2;
  while (k < nblk) {
    // next (block, tile)
    int kn = k;
    int64_t tn = t + 1;
    BlockWalk nw = cw;
    if (tn >= cw.ntiles) {
      tn = 0;
      ++kn;
      while (kn < nblk) {
        nw = block_walk(a, seg, kn, iend);
        if (nw.ntiles > 0) break;
        ++kn;
      }
    }
    const bool have_next = kn < nblk;
    if (have_next) gload(nw, tn);

    // ---- compute the current tile ----
    const int64_t j0 = t * BK;
    if (j0 <= i0w + 31 + cw.diag) {  // some row of this wave sees a key of the tile
      const char *kt = smem + cur * BUF;
      const char *vt = kt + KB;
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s0 = mfma32(__builtin_bit_cast(bf16x8, ld16(kt + kr0 + ks * 32)), qf[ks], s0);
        s1 = mfma32(__builtin_bit_cast(bf16x8, ld16(kt + kr0 + 32 * KP + ks * 32)), qf[ks], s1);
      }
      // element i of s0 / s1 is key j0 + 32*(i/16) + 16*((i%16)/8) + 8g + i%8
      if ((j0 + BK - 1 > i0w + cw.diag) || (j0 + BK > cw.len_kv)) {
        // 32-bit local offsets: key j0 + jj is visible iff jj <= lim
        const int64_t lim64 = i0w + c32 + cw.diag - j0;
        const int64_t len64 = cw.len_kv - 1 - j0;
        const int lim = static_cast<int>(lim64 < len64 ? (lim64 < -1 ? -1 : lim64) : (len64 < -1 ? -1 : len64));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int jj = 16 * (i / 8) + 8 * g + (i % 8);
          if (jj > lim) s0[i] = -INFINITY;
          if (jj + 32 > lim) s1[i] = -INFINITY;
        }
      }
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      mx = fmaxf(mx, wave_swap32(mx)) * c;
      // raise the reference max only when it grows by more than TAU: P <= 2^TAU
      if (__any(mx > m_run + TAU)) {
        const float m_new = fmaxf(m_run, mx);
        // 1 for rows whose max did not rise (also all-masked rows: no -inf - -inf);
        // 0 when a row sees its first key
        const float alpha = m_new > m_run ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float psum = 0.f;
      bf16x8 pb[4];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p0 = fast_exp2(__builtin_fmaf(s0[i], c, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(s1[i], c, -m_use));
        psum += p0 + p1;
        pb[i / 8][i % 8] = static_cast<__bf16>(p0);
        pb[2 + i / 8][i % 8] = static_cast<__bf16>(p1);
      }
      l_run += psum;
      // O^T += V^T P^T: A = V^T rows (d) x 16 keys, read transposed from LDS
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const char *vp = vt + 16 * kk * VP + voff;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x4 lo = lds_read_tr(vp + dt * 64);
          const bf16x4 hi = lds_read_tr(vp + 4 * VP + dt * 64);
          acc[dt] = mfma32(cat8(lo, hi), pb[kk], acc[dt]);
        }
      }
    }

    if (have_next) lstore(cur ^ 1);
    __syncthreads();
    cur ^= 1;
    k = kn;
    t = tn;
    cw = nw;
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
  const float l_tot = l_run + wave_swap32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  const int64_t row = i0w + c32;
  if (row < seg.len_q) {
    if (OUT == 0) {
      const int64_t pos = seg.q_start + row * seg.stride;
      char *ob = static_cast<char *>(a.o) + 2 * (b * G.os[0] + pos * G.os[1] + h * G.os[2]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[dt][4 * q4 + e] * inv);
          const int d0 = 32 * dt + 8 * q4 + 4 * g;
          *reinterpret_cast<bf16x4 *>(ob + 2 * d0) = v;
        }
      if (g == 0) a.lse[(static_cast<int64_t>(b) * G.hq + h) * G.seqlen + pos] = lse;
    } else {
      const int64_t prow = seg.part_off + (static_cast<int64_t>(b) * G.hq + h) * seg.len_q + row;
      float *op = static_cast<float *>(a.o) + prow * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[dt][4 * q4 + e] * inv;
          *reinterpret_cast<f32x4 *>(op + 32 * dt + 8 * q4 + 4 * g) = v;
        }
      if (g == 0) a.lse[prow] = lse;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 gr(static_cast<unsigned>(grid)), bl(NT);
  if (hd == 128) {
    if (a.out_mode == 0)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, 0>), gr, bl, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<128, 1>), gr, bl, 0, s, a);
  } else if (hd == 64) {
    if (a.out_mode == 0)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 0>), gr, bl, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 1>), gr, bl, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfa
