// attn_bwd_bf16.hip -- bf16 backward of blockwise causal attention on gfx950.
//
// The backward keeps no attention matrix: P is recomputed from the saved
// log-sum-exp (FlashAttention glossary page, first two paragraphs;
// "rematerialisation-aware gradient checkpointing" on the DistFlashAttn
// paper record).  With D_i = rowsum(dO_i * O_i):
//   P_ij = e^{scale q_i.k_j - LSE_i},  dP_ij = dO_i.v_j,  dS_ij = P_ij (dP_ij - D_i)
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
//
// Two kernels, no atomics, deterministic:
//  * dq: query-major, shaped like the forward -- a workgroup owns 128 query
//    rows, walks its query piece's blocks in ring-step order and computes
//    S^T = K Q^T, dP^T = V dO^T and dQ^T += K^T dS^T on the matrix cores.
//    Each lane owns one query column, so LSE_i and D_i are per-lane scalars.
//  * dkdv: key-major -- a workgroup owns 128 key rows (K and V live in
//    registers as MFMA operands), walks every block that reads its key piece
//    and every query head of its group, and computes S = Q K^T, dP = dO V^T,
//    dV^T += dO^T P and dK^T += Q^T dS.  Each lane owns one key column.
// Q/dO (or K/V) tiles are double-buffered in LDS; transposed operands come
// from ds_read_b64_tr_b16 on the row-major tiles.
#include "device_util.h"
#include "dfa_internal.h"

namespace dfa {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ int kperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// ============================ dQ (query-major) ============================
constexpr int DQ_BQ = kFwdTileQ;  // 128
constexpr int DQ_BK = 64;

template <int HD>
__global__ __launch_bounds__(NT, 2) void dq_bf16_kernel(BwdArgs a) {
  constexpr int PITCH = HD * 2 + 32;  // K tile: transposing reads of 4 rows conflict-free
  constexpr int VPITCH = HD * 2 + 16; // V tile: b128 reads of 16 rows conflict-free
  constexpr int TILEB = DQ_BK * PITCH;
  constexpr int BUFB = TILEB + DQ_BK * VPITCH;
  constexpr int KS = HD / 16, DT = HD / 32, CH = HD / 8, RPP = NT / CH, NP = DQ_BK / RPP;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUFB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c32 = lane & 31;
  const Geom &G = a.g;
  const float c = G.scale_log2;
  const int BH = G.batch * G.hq;
  const int64_t bid = blockIdx.x;
  const int bh = static_cast<int>(bid % BH);
  const Tile tl = ld_table(a.qtiles + bid / BH);
  const QSeg seg = ld_table(a.qsegs + tl.seg);
  const int b = bh / G.hq, h = bh % G.hq, hk = h / G.group;
  const int64_t i0 = static_cast<int64_t>(tl.tile) * DQ_BQ;
  const int64_t i0w = i0 + wave * 32;
  const int64_t iend = (i0 + DQ_BQ < seg.len_q) ? i0 + DQ_BQ : seg.len_q;

  const char *kb = static_cast<const char *>(a.k) + 2 * (b * G.ks[0] + hk * G.ks[2]);
  const char *vb = static_cast<const char *>(a.v) + 2 * (b * G.vs[0] + hk * G.vs[2]);
  const int64_t krs = 2 * G.ks[1] * seg.stride, vrs = 2 * G.vs[1] * seg.stride;

  // rows past the piece read its last row; they are never stored
  bf16x8 qf[KS], df[KS];
  const int64_t row = i0w + c32;
  const bool valid = row < seg.len_q;
  const int64_t pos = seg.q_start + (valid ? row : seg.len_q - 1) * seg.stride;
  {
    const char *qsrc = static_cast<const char *>(a.q) + 2 * (b * G.qs[0] + pos * G.qs[1] + h * G.qs[2]);
    const char *dsrc = static_cast<const char *>(a.dout) + 2 * (b * G.os[0] + pos * G.os[1] + h * G.os[2]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, ld16(qsrc + (2 * ks + g) * 16));
      df[ks] = __builtin_bit_cast(bf16x8, ld16(dsrc + (2 * ks + g) * 16));
    }
  }
  const int64_t lr = (static_cast<int64_t>(b) * G.hq + h) * G.seqlen + pos;
  const float lse2 = a.lse[lr] * kLog2e;
  const float dd = a.dd[lr];

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  struct Walk {
    int64_t kv_start, len_kv, diag, ntiles;
  };
  auto walk = [&](int k) {
    const KvRef r = ld_table(a.qkv + seg.blk_begin + k);
    Walk w{r.kv_start, r.len_kv, r.diag_offset, 0};
    int64_t hi = iend + r.diag_offset;
    if (hi > r.len_kv) hi = r.len_kv;
    w.ntiles = hi > 0 ? (hi + DQ_BK - 1) / DQ_BK : 0;
    return w;
  };
  const int nblk = seg.blk_count;
  int k = 0;
  Walk cw{0, 0, 0, 0};
  while (k < nblk) {
    cw = walk(k);
    if (cw.ntiles > 0) break;
    ++k;
  }
  const int lrow = tid / CH, lch = tid % CH;
  u32x4 kr[NP], vr[NP];
  // rows past the key piece re-read its last row; the mask zeroes them
  auto gload = [&](const Walk &w, int64_t t) {
    const char *kp = kb + 2 * w.kv_start * G.ks[1] + lch * 16;
    const char *vp = vb + 2 * w.kv_start * G.vs[1] + lch * 16;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      int64_t j = t * DQ_BK + lrow + p * RPP;
      j = j < w.len_kv ? j : w.len_kv - 1;
      kr[p] = ld16(kp + j * krs);
      vr[p] = ld16(vp + j * vrs);
    }
  };
  auto lstore = [&](int buf) {
    char *kt = smem + buf * BUFB;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      st16(kt + (lrow + p * RPP) * PITCH + lch * 16, kr[p]);
      st16(kt + TILEB + (lrow + p * RPP) * VPITCH + lch * 16, vr[p]);
    }
  };
  int64_t t = 0;
  int cur = 0;
  if (k < nblk) {
    gload(cw, 0);
    lstore(0);
  }
  __syncthreads();
  while (k < nblk) {
    int kn = k;
    int64_t tn = t + 1;
    Walk nw = cw;
    if (tn >= cw.ntiles) {
      tn = 0;
      ++kn;
      while (kn < nblk) {
        nw = walk(kn);
        if (nw.ntiles > 0) break;
        ++kn;
      }
    }
    const bool have_next = kn < nblk;
    if (have_next) gload(nw, tn);

    const int64_t j0 = t * DQ_BK;
    if (j0 <= i0w + 31 + cw.diag) {
      const char *kt = smem + cur * BUFB;
      const char *vt = kt + TILEB;
      f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = f32x16{}, p1 = f32x16{};
      const int ro = kperm(c32) * PITCH + g * 16;
      const int vo = kperm(c32) * VPITCH + g * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 k0 = __builtin_bit_cast(bf16x8, ld16(kt + ro + ks * 32));
        const bf16x8 k1 = __builtin_bit_cast(bf16x8, ld16(kt + ro + 32 * PITCH + ks * 32));
        const bf16x8 v0 = __builtin_bit_cast(bf16x8, ld16(vt + vo + ks * 32));
        const bf16x8 v1 = __builtin_bit_cast(bf16x8, ld16(vt + vo + 32 * VPITCH + ks * 32));
        s0 = mfma32(k0, qf[ks], s0);
        s1 = mfma32(k1, qf[ks], s1);
        p0 = mfma32(v0, df[ks], p0);
        p1 = mfma32(v1, df[ks], p1);
      }
      if ((j0 + DQ_BK - 1 > i0w + cw.diag) || (j0 + DQ_BK > cw.len_kv)) {
        // local key j0 + jj is visible iff jj <= lim (32-bit)
        const int64_t lim64 = row + cw.diag - j0, len64 = cw.len_kv - 1 - j0;
        const int64_t m64 = lim64 < len64 ? lim64 : len64;
        const int lim = static_cast<int>(m64 < -1 ? -1 : m64);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int jj = 16 * (i / 8) + 8 * g + (i % 8);
          if (jj > lim) s0[i] = -INFINITY;
          if (jj + 32 > lim) s1[i] = -INFINITY;
        }
      }
      bf16x8 dsb[4];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pa = fast_exp2(__builtin_fmaf(s0[i], c, -lse2));
        const float pc = fast_exp2(__builtin_fmaf(s1[i], c, -lse2));
        dsb[i / 8][i % 8] = static_cast<__bf16>(pa * (p0[i] - dd));
        dsb[2 + i / 8][i % 8] = static_cast<__bf16>(pc * (p1[i] - dd));
      }
      // dQ^T += K^T dS^T: A = K^T (d x 16 keys) read transposed from the K tile
      const int krow = 8 * g + (lane & 15) / 4;
      const int kcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const char *kp = kt + (16 * kk + krow) * PITCH + kcol * 2;  // kt: current K tile
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x4 lo = lds_read_tr(kp + dt * 64);
          const bf16x4 hi = lds_read_tr(kp + 4 * PITCH + dt * 64);
          acc[dt] = mfma32(cat8(lo, hi), dsb[kk], acc[dt]);
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
  if (!valid) return;
  char *ob = static_cast<char *>(a.dq) + 2 * (b * G.qs[0] + pos * G.qs[1] + h * G.qs[2]);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[dt][4 * q4 + e] * G.scale);
      *reinterpret_cast<bf16x4 *>(ob + 2 * (32 * dt + 8 * q4 + 4 * g)) = v;
    }
}

// ========================= dK, dV (key-major) =========================
constexpr int KV_BK = kBwdTileKV;  // 128 key rows per workgroup
constexpr int KV_BQ = 64;          // query rows per streamed tile

// Key-major gradient kernels.  MODE 1 accumulates dV^T += dO^T P (needs S
// only), MODE 2 accumulates dK^T += Q^T dS (needs S and dP).  Splitting the
// two keeps one 64-register accumulator set per wave, so two waves share each
// SIMD and hide each other's LDS and exponent latency; S is recomputed in both.
constexpr int KV_DV = 1, KV_DK = 2;

template <int HD, int MODE>
__global__ __launch_bounds__(NT, 2) void dkdv_bf16_kernel(BwdArgs a) {
  // Streamed Q/dO tiles: pitch HD*2 + 32 and logical 16-byte chunk c of row r
  // stored at chunk c ^ bit3(r).  Both the b128 row reads of 16 rows and the
  // transposing reads of 4 rows x 32 bytes then hit distinct banks, and every
  // operand address stays affine in the loop indices.
  constexpr int RB = HD * 2 + 32;
  constexpr int TB = KV_BQ * RB;
  constexpr int BUFB = 2 * TB + 2 * KV_BQ * 4;  // Q, dO, LSE*log2(e), D
  constexpr int KS = HD / 16, DT = HD / 32;
  constexpr int LPR = HD * 2 / 16;           // data lanes per row in a direct load
  constexpr int LPRP = RB / 16;              // lanes per row including the pad
  constexpr int RPI = 64 / LPRP;             // rows per direct load instruction
  constexpr int NI = (KV_BQ + RPI - 1) / RPI;   // direct loads per tile and tensor
  constexpr bool DK = MODE == KV_DK;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUFB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const Geom &G = a.g;
  const float c = G.scale_log2;
  const int BH = G.batch * G.hkv;
  const int64_t bid = blockIdx.x;
  const int bh = static_cast<int>(bid % BH);
  const Tile tl = ld_table(a.kvtiles + bid / BH);
  const KvSeg seg = ld_table(a.kvsegs + tl.seg);
  const int b = bh / G.hkv, hk = bh % G.hkv;
  const int64_t j0 = static_cast<int64_t>(tl.tile) * KV_BK;
  const int64_t j0w = j0 + wave * 32;
  const int64_t col = j0w + c32;  // this lane's key row
  const bool valid = col < seg.len_kv;
  const int64_t pos = seg.kv_start + (valid ? col : seg.len_kv - 1) * seg.stride;

  // K (and for dK also V) as B operands of S = Q K^T and dP = dO V^T; rows
  // past the key piece read its last row and are never stored
  bf16x8 kf[KS], vf[DK ? KS : 1];
  {
    const char *ksrc = static_cast<const char *>(a.k) + 2 * (b * G.ks[0] + pos * G.ks[1] + hk * G.ks[2]);
    const char *vsrc = static_cast<const char *>(a.v) + 2 * (b * G.vs[0] + pos * G.vs[1] + hk * G.vs[2]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, ld16(ksrc + (2 * ks + g) * 16));
      if (DK) vf[ks] = __builtin_bit_cast(bf16x8, ld16(vsrc + (2 * ks + g) * 16));
    }
  }
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  // walk over (group head, block, query tile)
  struct Walk {
    int64_t q_start, len_q, diag, t0, t1;  // query tiles [t0, t1)
    int h;
  };
  auto walk = [&](int gi, int k) {
    const QRef r = ld_table(a.kvq + seg.blk_begin + k);
    Walk w{r.q_start, r.len_q, r.diag_offset, 0, 0, hk * G.group + gi};
    int64_t lo = j0 - r.diag_offset;  // first query row that sees key row j0
    if (lo < 0) lo = 0;
    if (lo < r.len_q) {
      w.t0 = lo / KV_BQ;
      w.t1 = (r.len_q + KV_BQ - 1) / KV_BQ;
    }
    return w;
  };
  const int nblk = seg.blk_count, ngrp = G.group;
  int gi = 0, k = 0;
  Walk cw{};
  auto advance_to_nonempty = [&](int &gi_, int &k_, Walk &w_) {
    while (gi_ < ngrp) {
      while (k_ < nblk) {
        w_ = walk(gi_, k_);
        if (w_.t1 > w_.t0) return;
        ++k_;
      }
      ++gi_;
      k_ = 0;
    }
  };
  advance_to_nonempty(gi, k, cw);
  int64_t t = cw.t0;

  // bytes between consecutive rows of the piece (the host guarantees that 64
  // rows span less than 2^31 bytes, so per-lane row offsets fit 32 bits)
  const int64_t qrs = 2 * G.qs[1] * seg.stride, ors = 2 * G.os[1] * seg.stride;
  float lsr = 0.f, ddr = 0.f;
  // Q and dO rows go straight from HBM into the LDS tile (no registers): a
  // direct load writes 64 lanes x 16 contiguous bytes, so LPRP lanes cover one
  // padded row (the pad lanes re-write the row's first chunk into the pad).
  // Wave w issues loads w, w + 4, ...; each lane's row and chunk are fixed,
  // so its byte offsets are computed once.  Rows past the query piece re-read
  // its last row (ragged tiles only) and the mask drops them.  LSE and D of
  // the 64 rows travel through two registers.
  constexpr int MW = (NI + 3) / 4;  // loads per wave and tensor
  const int wv = wave;
  const int l_row = lane / LPRP, l_p = lane % LPRP;
  auto lrow = [&](int m) { return (wv + 4 * m) * RPI + l_row; };
  auto lchunk = [&](int r) { return l_p < LPR ? (l_p ^ ((r >> 3) & 1)) : 0; };
  auto lon = [&](int m) { return wv + 4 * m < NI && l_row < RPI && lrow(m) < KV_BQ; };
  unsigned qo_m[MW], oo_m[MW];
#pragma unroll
  for (int m = 0; m < MW; ++m) {
    const int r = lrow(m);
    qo_m[m] = static_cast<unsigned>(r * qrs) + 16 * lchunk(r);
    oo_m[m] = static_cast<unsigned>(r * ors) + 16 * lchunk(r);
  }
  auto dload = [&](const Walk &w, int64_t tt, int buf) {
    char *base = smem + buf * BUFB;
    const int64_t i0 = tt * KV_BQ;
    const char *qb = static_cast<const char *>(a.q) +
                     2 * (b * G.qs[0] + (w.q_start + i0 * seg.stride) * G.qs[1] + w.h * G.qs[2]);
    const char *db = static_cast<const char *>(a.dout) +
                     2 * (b * G.os[0] + (w.q_start + i0 * seg.stride) * G.os[1] + w.h * G.os[2]);
    if (i0 + KV_BQ <= w.len_q) {
#pragma unroll
      for (int m = 0; m < MW; ++m) {
        if (wv + 4 * m < NI && lon(m)) {
          const int r0 = (wv + 4 * m) * RPI;
          load_lds16(qb + qo_m[m], base + r0 * RB);
          load_lds16(db + oo_m[m], base + TB + r0 * RB);
        }
      }
    } else {  // ragged last tile: rows past the piece re-read its last row
      const int last = static_cast<int>(w.len_q - 1 - i0);
#pragma unroll
      for (int m = 0; m < MW; ++m) {
        if (wv + 4 * m < NI && lon(m)) {
          const int r0 = (wv + 4 * m) * RPI;
          const int r = lrow(m), rr = r < last ? r : last;
          load_lds16(qb + rr * qrs + 16 * lchunk(r), base + r0 * RB);
          load_lds16(db + rr * ors + 16 * lchunk(r), base + TB + r0 * RB);
        }
      }
    }
    if (tid < KV_BQ) {
      int64_t i = i0 + tid;
      i = i < w.len_q ? i : w.len_q - 1;
      const int64_t r = (static_cast<int64_t>(b) * G.hq + w.h) * G.seqlen + w.q_start + i * seg.stride;
      lsr = a.lse[r] * kLog2e;
      if (DK) ddr = a.dd[r];
    }
  };
  auto stats_store = [&](int buf) {
    if (tid < KV_BQ) {
      float *st = reinterpret_cast<float *>(smem + buf * BUFB + 2 * TB);
      st[tid] = lsr;
      if (DK) st[KV_BQ + tid] = ddr;
    }
  };

  int cur = 0;
  if (gi < ngrp) {
    dload(cw, t, 0);
    stats_store(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // per-lane operand offsets (independent of the tile); loop indices only
  // add compile-time constants to them
  const int a_off = kperm(c32) * RB + 16 * (g ^ ((c32 >> 2) & 1));
  const int t_off = (8 * g + (lane & 15) / 4) * RB +
                    16 * ((2 * ((lane >> 4) & 1) + (lane & 3) / 2) ^ g) + 8 * (lane & 1);
  while (gi < ngrp) {
    int gn = gi, kn = k;
    int64_t tn = t + 1;
    Walk nw = cw;
    if (tn >= cw.t1) {
      ++kn;
      advance_to_nonempty(gn, kn, nw);
      tn = nw.t0;
    }
    const bool have_next = gn < ngrp;
    if (have_next) dload(nw, tn, cur ^ 1);

    const int64_t qi0 = t * KV_BQ;
    // some pair of this wave visible: largest query row sees smallest key row
    if (qi0 + KV_BQ - 1 + cw.diag >= j0w) {
      const char *qt = smem + cur * BUFB;
      const char *dt_ = qt + TB;
      const float *lt = reinterpret_cast<const float *>(qt + 2 * TB);
      const float *ddt = lt + KV_BQ;
      // local query qq (0..63) of the tile is kept iff lo <= qq < hi
      const bool need_mask = (qi0 + cw.diag < j0w + 31) || (qi0 + KV_BQ > cw.len_q);
      int lo = 0, hi = KV_BQ;
      if (need_mask) {
        const int64_t lo64 = col - cw.diag - qi0, hi64 = cw.len_q - qi0;
        lo = static_cast<int>(lo64 < 0 ? 0 : (lo64 > KV_BQ ? KV_BQ : lo64));
        hi = static_cast<int>(hi64 > KV_BQ ? KV_BQ : hi64);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {  // two halves of 32 query rows
        f32x16 s = f32x16{}, dpm = f32x16{};
        const char *qa = qt + a_off + 32 * mt * RB, *da = dt_ + a_off + 32 * mt * RB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = mfma32(__builtin_bit_cast(bf16x8, ld16(qa + ks * 32)), kf[ks], s);
          if (DK) dpm = mfma32(__builtin_bit_cast(bf16x8, ld16(da + ks * 32)), vf[ks], dpm);
        }
        // element i is query row qi0 + 32mt + 16(i/8) + 8g + i%8; masked
        // scores become -inf (probability 0)
        if (need_mask) {
          const int x = 8 * g - lo;  // qq - lo without the element's constant part
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const unsigned rel = static_cast<unsigned>(x + 32 * mt + 16 * (i / 8) + (i % 8));
            if (rel >= static_cast<unsigned>(hi - lo)) s[i] = -INFINITY;
          }
        }
        bf16x8 ob[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int qoff = 32 * mt + 16 * u + 8 * g;
          const f32x4 la = *reinterpret_cast<const f32x4 *>(lt + qoff);
          const f32x4 lb = *reinterpret_cast<const f32x4 *>(lt + qoff + 4);
          f32x4 da4 = f32x4{}, db4 = f32x4{};
          if (DK) {
            da4 = *reinterpret_cast<const f32x4 *>(ddt + qoff);
            db4 = *reinterpret_cast<const f32x4 *>(ddt + qoff + 4);
          }
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int i = 8 * u + w;
            const float p = fast_exp2(__builtin_fmaf(s[i], c, -(w < 4 ? la[w] : lb[w - 4])));
            ob[u][w] = static_cast<__bf16>(DK ? p * (dpm[i] - (w < 4 ? da4[w] : db4[w - 4])) : p);
          }
        }
        // dV^T += dO^T P or dK^T += Q^T dS: A operand read transposed from LDS
        const char *src = DK ? qt : dt_;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int o = t_off + 16 * (2 * mt + u) * RB;
#pragma unroll
          for (int e = 0; e < DT; ++e)
            acc[e] = mfma32(cat8(lds_read_tr(src + o + 64 * e), lds_read_tr(src + o + 4 * RB + 64 * e)),
                            ob[u], acc[e]);
        }
      }
    }
    if (have_next) stats_store(cur ^ 1);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
    __syncthreads();
    cur ^= 1;
    gi = gn;
    k = kn;
    t = tn;
    cw = nw;
  }
  if (!valid) return;
  char *out = DK ? static_cast<char *>(a.dk) + 2 * (b * G.ks[0] + pos * G.ks[1] + hk * G.ks[2])
                 : static_cast<char *>(a.dv) + 2 * (b * G.vs[0] + pos * G.vs[1] + hk * G.vs[2]);
  const float osc = DK ? G.scale : 1.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = static_cast<__bf16>(acc[dt][4 * q4 + e] * osc);
      *reinterpret_cast<bf16x4 *>(out + 2 * (32 * dt + 8 * q4 + 4 * g)) = x;
    }
}

}  // namespace

hipError_t launch_bwd_dq_bf16(const BwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (hd == 128)
    hipLaunchKernelGGL(dq_bf16_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s, a);
  else if (hd == 64)
    hipLaunchKernelGGL(dq_bf16_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 gr(static_cast<unsigned>(grid)), bl(NT);
  if (hd == 128) {
    hipLaunchKernelGGL((dkdv_bf16_kernel<128, KV_DK>), gr, bl, 0, s, a);
    hipLaunchKernelGGL((dkdv_bf16_kernel<128, KV_DV>), gr, bl, 0, s, a);
  } else if (hd == 64) {
    hipLaunchKernelGGL((dkdv_bf16_kernel<64, KV_DK>), gr, bl, 0, s, a);
    hipLaunchKernelGGL((dkdv_bf16_kernel<64, KV_DV>), gr, bl, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfa
