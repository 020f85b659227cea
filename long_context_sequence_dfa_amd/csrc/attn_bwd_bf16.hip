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

// Streamed operand tiles of 64 rows: pitch HD*2 + 32 bytes, logical 16-byte
// chunk c of row r stored at chunk c ^ bit3(r).  Both the b128 reads of 16
// rows (MFMA operands in kperm row order) and the transposing reads of 4 rows
// x 32 bytes then hit distinct banks, and every operand address stays affine
// in the loop indices.
template <int HD>
struct Tile64 {
  static constexpr int ROWS = 64;
  static constexpr int RB = HD * 2 + 32;       // row pitch in bytes
  static constexpr int TB = ROWS * RB;         // tile bytes
  static constexpr int LPR = HD * 2 / 16;      // data lanes per row in a direct load
  static constexpr int LPRP = RB / 16;         // lanes per row including the pad
  static constexpr int RPI = 64 / LPRP;        // rows per direct-load instruction
  static constexpr int NI = (ROWS + RPI - 1) / RPI;  // instructions per tile
  static constexpr int MW = (NI + 3) / 4;      // instructions per wave (4 waves)

  // b128 operand read of row kperm(c32), chunk pair (2ks + g): offset + 32 ks
  __device__ static int a_off(int lane) {
    const int g = lane >> 5, c32 = lane & 31;
    return kperm(c32) * RB + 16 * (g ^ ((c32 >> 2) & 1));
  }
  // transposing read: rows 16u + 8g + (lane&15)/4 (+4 for the upper half),
  // 4 bf16 columns at 16((lane>>4)&1) + 4(lane&3) (+32 per column block)
  __device__ static int t_off(int lane) {
    const int g = lane >> 5;
    return (8 * g + (lane & 15) / 4) * RB + 16 * ((2 * ((lane >> 4) & 1) + (lane & 3) / 2) ^ g) +
           8 * (lane & 1);
  }
};

// Direct HBM -> LDS loads of two 64-row tiles (same row count, separate row
// strides) into the swizzled layout of Tile64.  A direct load writes 64 lanes
// x 16 contiguous bytes, so LPRP lanes cover one padded row (pad lanes re-write
// the row's first chunk into the pad).  Wave w issues instructions w, w + 4,
// ...; each lane's row and chunk are fixed, so its byte offsets are computed
// once (32-bit: the host guarantees 64 rows span less than 2^31 bytes).  Rows
// past the piece re-read its last row; the caller's mask drops them.
template <int HD>
struct PairLoader {
  using T = Tile64<HD>;
  int wv, l_row, l_p;
  int64_t rsa, rsb;
  unsigned oa[T::MW], ob[T::MW];

  __device__ int lrow(int m) const { return (wv + 4 * m) * T::RPI + l_row; }
  __device__ int lchunk(int r) const { return l_p < T::LPR ? (l_p ^ ((r >> 3) & 1)) : 0; }
  __device__ bool lon(int m) const { return wv + 4 * m < T::NI && l_row < T::RPI && lrow(m) < T::ROWS; }

  __device__ PairLoader(int wave, int lane, int64_t rs_a, int64_t rs_b)
      : wv(wave), l_row(lane / T::LPRP), l_p(lane % T::LPRP), rsa(rs_a), rsb(rs_b) {
#pragma unroll
    for (int m = 0; m < T::MW; ++m) {
      const int r = lrow(m);
      oa[m] = static_cast<unsigned>(r * rsa) + 16 * lchunk(r);
      ob[m] = static_cast<unsigned>(r * rsb) + 16 * lchunk(r);
    }
  }

  // ga/gb: first row of the tile; rows: rows left in the piece from there
  __device__ void load(const char *ga, const char *gb, char *la, char *lb, int64_t rows) const {
    if (rows >= T::ROWS) {
#pragma unroll
      for (int m = 0; m < T::MW; ++m)
        if (wv + 4 * m < T::NI && lon(m)) {
          const int r0 = (wv + 4 * m) * T::RPI;
          load_lds16(ga + oa[m], la + r0 * T::RB);
          load_lds16(gb + ob[m], lb + r0 * T::RB);
        }
    } else {
      const int last = static_cast<int>(rows - 1);
#pragma unroll
      for (int m = 0; m < T::MW; ++m)
        if (wv + 4 * m < T::NI && lon(m)) {
          const int r0 = (wv + 4 * m) * T::RPI;
          const int r = lrow(m), rr = r < last ? r : last;
          load_lds16(ga + rr * rsa + 16 * lchunk(r), la + r0 * T::RB);
          load_lds16(gb + rr * rsb + 16 * lchunk(r), lb + r0 * T::RB);
        }
    }
  }
};

// ============================ dQ (query-major) ============================
constexpr int DQ_BQ = kDqTileQ;  // 128
constexpr int DQ_BK = 64;

template <int HD>
__global__ __launch_bounds__(NT, 2) void dq_bf16_kernel(BwdArgs a) {
  using TL = Tile64<HD>;
  static_assert(TL::ROWS == DQ_BK, "key tiles are 64 rows");
  constexpr int RB = TL::RB, TB = TL::TB, BUFB = 2 * TB;  // K, V
  constexpr int KS = HD / 16, DT = HD / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUFB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // K and V rows go straight into LDS
  const PairLoader<HD> ld(wave, lane, 2 * G.ks[1] * seg.stride, 2 * G.vs[1] * seg.stride);
  auto gload = [&](const Walk &w, int64_t t, int buf) {
    char *base = smem + buf * BUFB;
    const int64_t jt = t * DQ_BK;
    const int64_t p0 = w.kv_start + jt * seg.stride;
    ld.load(kb + 2 * p0 * G.ks[1], vb + 2 * p0 * G.vs[1], base, base + TB, w.len_kv - jt);
  };
  int64_t t = 0;
  int cur = 0;
  if (k < nblk) gload(cw, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int a_off = TL::a_off(lane);
  const int t_off = TL::t_off(lane);
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
    if (kn < nblk) gload(nw, tn, cur ^ 1);

    const int64_t j0 = t * DQ_BK;
    if (j0 <= i0w + 31 + cw.diag) {
      const char *kt = smem + cur * BUFB;
      const char *vt = kt + TB;
      const bool need_mask = (j0 + DQ_BK - 1 > i0w + cw.diag) || (j0 + DQ_BK > cw.len_kv);
      int x = 0;
      if (need_mask) {
        // element i of half kh is local key jj = 32kh + 16(i/8) + 8g + i%8,
        // visible iff jj <= lim; x = 8g - lim
        const int64_t lim64 = row + cw.diag - j0, len64 = cw.len_kv - 1 - j0;
        const int64_t m64 = lim64 < len64 ? lim64 : len64;
        x = 8 * g - static_cast<int>(m64 < -1 ? -1 : (m64 > DQ_BK ? DQ_BK : m64));
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {  // two halves of 32 keys
        f32x16 sv = f32x16{}, pv = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int o = a_off + 32 * kh * RB + ks * 32;
          sv = mfma32(__builtin_bit_cast(bf16x8, ld16(kt + o)), qf[ks], sv);
          pv = mfma32(__builtin_bit_cast(bf16x8, ld16(vt + o)), df[ks], pv);
        }
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (x + 32 * kh + 16 * (i / 8) + (i % 8) > 0) sv[i] = -INFINITY;
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pa = fast_exp2(__builtin_fmaf(sv[i], c, -lse2));
          dsb[i / 8][i % 8] = static_cast<__bf16>(pa * (pv[i] - dd));
        }
        // dQ^T += K^T dS^T: A = K^T (d x 16 keys) read transposed from the K tile
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int o = t_off + 16 * (2 * kh + u) * RB;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            acc[dt] = mfma32(cat8(lds_read_tr(kt + o + 64 * dt), lds_read_tr(kt + o + 4 * RB + 64 * dt)),
                             dsb[u], acc[dt]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
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
  using TL = Tile64<HD>;
  static_assert(TL::ROWS == KV_BQ, "query tiles are 64 rows");
  constexpr int RB = TL::RB;
  constexpr int TB = TL::TB;
  constexpr int BUFB = 2 * TB + 2 * KV_BQ * 4;  // Q, dO, LSE*log2(e), D
  constexpr int KS = HD / 16, DT = HD / 32;
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

  float lsr = 0.f, ddr = 0.f;
  // Q and dO rows go straight into LDS; LSE and D of the 64 rows travel
  // through two registers.
  const PairLoader<HD> ld(wave, lane, 2 * G.qs[1] * seg.stride, 2 * G.os[1] * seg.stride);
  auto dload = [&](const Walk &w, int64_t tt, int buf) {
    char *base = smem + buf * BUFB;
    const int64_t i0 = tt * KV_BQ;
    const char *qb = static_cast<const char *>(a.q) +
                     2 * (b * G.qs[0] + (w.q_start + i0 * seg.stride) * G.qs[1] + w.h * G.qs[2]);
    const char *db = static_cast<const char *>(a.dout) +
                     2 * (b * G.os[0] + (w.q_start + i0 * seg.stride) * G.os[1] + w.h * G.os[2]);
    ld.load(qb, db, base, base + TB, w.len_q - i0);
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
  const int a_off = TL::a_off(lane);
  const int t_off = TL::t_off(lane);
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
