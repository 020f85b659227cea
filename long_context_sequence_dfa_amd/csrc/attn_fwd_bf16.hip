// attn_fwd_bf16.hip -- bf16 forward of blockwise causal attention on gfx950.
//
// One workgroup (8 waves) owns 256 query rows of one query piece, one batch
// entry and one query head.  It walks the piece's blocks (the key/value
// shards a virtual rank holds over the ring steps, read in place) in the
// order of the host's table and, inside each block, the 64-key tiles that
// hold at least one visible key.
// Per tile it keeps the running row max m, the running row sum l and the
// running output O, rescaling by alpha = e^{m_old - m_new} (Striped Attention
// Guide, "Algorithmic Mechanics" 1, steps 1-6), then normalises once at the
// end (step 7) and emits LSE = m + ln l.  Tiles past the causal limit are
// never visited and only tiles that straddle the diagonal evaluate the mask
// ("Algorithmic Mechanics" 2, intra- vs inter-block masking).  With packed
// documents a key before the first position of the row's document is masked
// too, and tiles before the first row's document are skipped (same page,
// "Production Deployment and Best Practices", item 3).
//
// gfx950 mapping:
//  * each wave computes S^T = K Q^T for 32 queries x 64 keys with
//    v_mfma_f32_32x32x16_bf16, so every lane owns one query column: the row
//    max and sum need only the lane's own 32 values plus one exchange with
//    lane l^32 (v_permlane32_swap);
//  * key rows enter the MFMA in a bit-swapped order (kperm) so that the S^T
//    accumulator of a lane holds 8 consecutive keys per 16-key step -- exactly
//    the B operand of O^T = V^T P^T, so P goes from accumulator to MFMA
//    operand without touching LDS;
//  * V^T operands come straight from the row-major V tile in LDS through
//    ds_read_b64_tr_b16; the swizzled tile layout keeps both the b128 reads
//    of K and the transposing reads of V free of bank conflicts;
//  * K/V tiles stream through NS LDS stages by direct HBM->LDS loads issued
//    NS - 1 tiles ahead (stream_lds.h); one barrier per tile;
//  * the vector ALU is the scarce unit next to the MFMAs, so the softmax is
//    kept lean: one FMA folds scale, log2(e) and the max into the exponent,
//    and the running output is rescaled only when a row's max grows by more
//    than 2^8 (exact: every probability is taken against the same reference
//    max as its row sum, and stays below 2^8).
// Score arithmetic runs in the log2 domain: x = s * scale * log2(e).
#include "dfa_internal.h"
#include "stream_lds.h"

namespace dfa {
namespace {

constexpr int NW = kFwdWaves;  // waves per workgroup
constexpr int NT = 64 * NW;    // threads per workgroup
constexpr int BQ = kFwdTileQ;  // query rows per workgroup (32 per wave)
constexpr int BK = 64;         // keys per streamed tile
constexpr int NS = kFwdStages; // K/V tiles resident in LDS (NS - 1 in flight)
static_assert(BQ == 32 * NW, "one 32-query column block per wave");

struct BlockWalk {
  int64_t kv_start, len_kv, diag, ntiles;
  int64_t t0;  // first tile with a key visible to some row (packed documents)
  int64_t te;  // interleaved walk: end of the current group's tiles of this block
};

// The key piece of block k; ntiles covers every key at or before the
// workgroup's last query row (local row iend-1, global position q_last), t0
// skips the tiles before wlo, the first position of the first row's document
// (0 without packed documents).  RUNS: pieces made of runs (stripe blocks),
// visibility from global positions; otherwise rows start + i*stride and the
// block's diagonal.
template <bool RUNS>
__device__ __forceinline__ BlockWalk walk_of(const KvRef &r, const QSeg &seg, int64_t iend,
                                             int64_t q_last, int64_t wlo) {
  BlockWalk w;
  w.kv_start = r.kv_start;
  w.len_kv = r.len_kv;
  w.diag = r.diag_offset;
  int64_t hi;
  if constexpr (RUNS) {
    hi = piece_count_le(r.kv_start, seg.stride, seg.run, r.len_kv, q_last);
  } else {
    hi = iend + r.diag_offset;  // the last row iend-1 sees keys j <= iend-1+diag
    if (hi > r.len_kv) hi = r.len_kv;
  }
  w.ntiles = hi > 0 ? (hi + BK - 1) / BK : 0;
  w.t0 = wlo > 0 ? piece_count_le(r.kv_start, seg.stride, seg.run, r.len_kv, wlo - 1) / BK : 0;
  w.te = w.ntiles;
  return w;
}

template <bool TABLE, bool RUNS>
__device__ __forceinline__ BlockWalk block_walk(const FwdArgs &a, const QSeg &seg, int k,
                                                int64_t iend, int64_t q_last, int64_t wlo) {
  KvRef r;
  if constexpr (TABLE)
    r = ld_table(a.kv + seg.blk_begin + k);
  else
    r = a.kv0;
  return walk_of<RUNS>(r, seg, iend, q_last, wlo);
}

// TABLE: the query piece and its blocks come from the work tables (fused and
// stepwise walks); otherwise from seg0/kv0 (one block).
// ILV: the interleaved walk (fused mode only).
template <int HD, int OUT, bool TABLE, bool RUNS, bool DOCS, bool ILV = false>
__global__ __launch_bounds__(NT, 8 / NW) void fwd_bf16_kernel(FwdArgs a) {
  using TL = Tile64<HD>;
  static_assert(TL::ROWS == BK, "key tiles are 64 rows");
  constexpr int RB = TL::RB, TB = TL::TB;
  constexpr int STAGE = 2 * TB;     // K tile, V tile
  constexpr int KS = HD / 16;       // MFMA k-steps over head_dim
  constexpr int DT = HD / 32;       // 32-row output tiles over head_dim
  constexpr float TAU = 8.f;        // lazy rescale threshold (log2 units)
  constexpr float PSUM_MAX = 32768.f;  // unmasked tiles: largest accepted row-half sum of P
  __shared__ __attribute__((aligned(16))) char smem[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const Geom &G = a.g;
  const int BH = G.batch * G.hq;
  int bh;
  int64_t ti;
  if constexpr (OUT == 0) {
    if (!xcd_item(blockIdx.x, a.n_tiles, BH, bh, ti)) return;
  } else {
    // per-step partials: batch-head fastest measured faster (in one ring
    // step every virtual rank reads another shard, so an XCD's workgroups
    // share no K/V whichever way they are grouped)
    const int64_t bid = blockIdx.x;
    if (bid >= (TABLE ? a.n_tiles : (a.seg0.len_q + BQ - 1) / BQ) * static_cast<int64_t>(BH)) return;
    bh = static_cast<int>(bid % BH);
    ti = bid / BH;
  }
  const int b = bh / G.hq, h = bh % G.hq, hk = h / G.group;

  QSeg seg;
  int64_t qt;
  if constexpr (TABLE) {
    const Tile t = ld_table(a.tiles + ti);
    seg = ld_table(a.segs + t.seg);
    qt = t.tile;
  } else {
    seg = a.seg0;
    qt = ti;
  }
  const int64_t i0 = qt * BQ;
  const int64_t i0w = i0 + wave * 32;
  const int64_t iend = (i0 + BQ < seg.len_q) ? i0 + BQ : seg.len_q;
  // global position of local row i of a piece of this workgroup
  auto pos_of = [&](int64_t start, int64_t i) {
    return RUNS ? piece_pos(start, seg.stride, seg.run, i) : start + i * seg.stride;
  };
  const int64_t rs = RUNS ? piece_row_step(seg.stride, seg.run) : seg.stride;  // row step in a tile
  // global position of the first row of 64-row tile t of a piece (a run is
  // 64 * 2^tsh rows, so the tile's run and offset are a shift and a mask)
  const int tsh = RUNS && seg.run > 1 ? __builtin_ctzll(static_cast<uint64_t>(seg.run)) - 6 : 0;
  auto tile_pos = [&](int64_t start, int64_t t_) {
    if constexpr (RUNS) {
      if (seg.run > 1) return start + (t_ >> tsh) * seg.stride + ((t_ & ((int64_t{1} << tsh) - 1)) << 6);
    }
    return start + t_ * (BK * seg.stride);
  };
  const int64_t q_last = RUNS ? pos_of(seg.q_start, iend - 1) : 0;
  // global position of this wave's first row (extrapolated past a ragged end:
  // only the mask's row comparisons use it)
  const int64_t gq_w = RUNS ? pos_of(seg.q_start, i0w) : 0;
  const float c = G.scale_log2;
  // packed documents: this lane's row sees keys at positions >= qlo only;
  // qlo_w is the largest bound of the wave (its last row), wlo the smallest
  // of the workgroup (its first row) -- positions rise with the row index
  int32_t qlo = 0, qlo_w = 0;
  int64_t wlo = 0;
  if constexpr (DOCS) {
    int64_t lo, hi_;
    const int64_t r = i0w + c32;
    doc_range(G.docs, G.n_docs, pos_of(seg.q_start, r < seg.len_q ? r : seg.len_q - 1), lo, hi_);
    qlo = static_cast<int32_t>(lo);
    qlo_w = __builtin_amdgcn_readlane(qlo, 31);
    doc_range(G.docs, G.n_docs, pos_of(seg.q_start, i0), lo, hi_);
    wlo = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(lo));
  }

  const char *qb = static_cast<const char *>(a.q) + 2 * (b * G.qs[0] + h * G.qs[2]);
  const char *kb = static_cast<const char *>(a.k) + 2 * (b * G.ks[0] + hk * G.ks[2]);
  const char *vb = static_cast<const char *>(a.v) + 2 * (b * G.vs[0] + hk * G.vs[2]);

  // Q^T operand (B of S^T = K Q^T): lane holds Q[row][16ks + 8g .. +8].
  // Rows past the piece read its last row (their outputs are never stored).
  bf16x8 qf[KS];
  {
    int64_t row = i0w + c32;
    row = row < seg.len_q ? row : seg.len_q - 1;
    const char *src = qb + 2 * pos_of(seg.q_start, row) * G.qs[1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(src + (2 * ks + g) * 16));
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  bool ref_ok = false;  // every row of the wave has a finite reference max

  // ---- tile sequence: (block k, tile t) over the blocks with visible keys ----
  const int nblk = TABLE ? seg.blk_count : 1;
  // Interleaved (the host's choice when every block is a near-triangle, as
  // under striping): tiles [g, g + G) of every block, then [g + G, g + 2G),
  // G = kIlvTiles.  The query tiles of one head that run side by side on an
  // XCD then read key tiles of one narrow window (from L2, a few MB) whatever
  // their row ranges, where walking block after block spread them over
  // every block and sent each read to HBM; G > 1 keeps the cursor's block
  // switch off most tiles.  Lane l holds block l's walk (at most 64 blocks).
  static_assert((kIlvTiles & (kIlvTiles - 1)) == 0, "group size: a power of two");
  int64_t iw_kv = 0;
  int32_t iw_len = 0, iw_diag = 0, iw_nt = 0, iw_t0 = 0, ilv_tend = 0;
  int64_t ilv_tbeg = 0;
  if constexpr (ILV) {
    if (lane < nblk) {
      const auto w = walk_of<RUNS>(a.kv[seg.blk_begin + lane], seg, iend, q_last, wlo);
      iw_kv = w.kv_start;
      iw_len = static_cast<int32_t>(w.len_kv);
      iw_diag = static_cast<int32_t>(w.diag);
      iw_nt = static_cast<int32_t>(w.ntiles);
      iw_t0 = static_cast<int32_t>(w.t0);
    }
    int32_t tb = 0x7fffffff;
    for (int l = 0; l < nblk; ++l) {
      const int32_t nt = __builtin_amdgcn_readlane(iw_nt, l), t0 = __builtin_amdgcn_readlane(iw_t0, l);
      if (nt > t0) {
        ilv_tend = nt > ilv_tend ? nt : ilv_tend;
        tb = t0 < tb ? t0 : tb;
      }
    }
    ilv_tbeg = tb & ~static_cast<int64_t>(kIlvTiles - 1);
  }
  auto first = [&](int &k_, BlockWalk &w_) {
    while (k_ < nblk) {
      w_ = block_walk<TABLE, RUNS>(a, seg, k_, iend, q_last, wlo);
      if (w_.ntiles > w_.t0) return;
      ++k_;
    }
  };
  auto next = [&](int &k_, int64_t &t_, BlockWalk &w_) {
    if constexpr (ILV) {
      if (++t_ < w_.te) return;
      // next block of the group, or the first block of the next group; the
      // group start moves once per pass over the blocks, ending at ilv_tend
      int64_t g = (t_ - 1) & ~static_cast<int64_t>(kIlvTiles - 1);
      for (;;) {
        if (++k_ >= nblk) {
          k_ = 0;
          g += kIlvTiles;
          if (g >= ilv_tend) {
            k_ = nblk;
            return;
          }
        }
        const int32_t nt = __builtin_amdgcn_readlane(iw_nt, k_);
        const int32_t t0 = __builtin_amdgcn_readlane(iw_t0, k_);
        const int64_t tb = g > t0 ? g : t0;
        const int64_t te = g + kIlvTiles < nt ? g + kIlvTiles : nt;
        if (tb < te) {
          w_.kv_start = readlane64(iw_kv, k_);
          w_.len_kv = __builtin_amdgcn_readlane(iw_len, k_);
          w_.diag = __builtin_amdgcn_readlane(iw_diag, k_);
          w_.ntiles = nt;
          w_.t0 = t0;
          w_.te = te;
          t_ = tb;
          return;
        }
      }
    }
    if (++t_ < w_.ntiles) return;
    ++k_;
    first(k_, w_);
    t_ = w_.t0;
  };
  int k = 0;
  BlockWalk cw{0, 0, 0, 0, 0, 0};
  int64_t t;
  if constexpr (ILV) {
    // one step before block 0's tiles of the first group (k = nblk - 1 wraps
    // to block 0 of group ilv_tbeg); nothing visible: ilv_tbeg >= ilv_tend
    k = nblk - 1;
    t = ilv_tbeg - kIlvTiles;
    cw.te = t + 1;
    next(k, t, cw);
  } else {
    first(k, cw);
    t = cw.t0;
  }

  // ---- K/V stream: NS LDS stages, the load cursor runs NS - 1 tiles ahead ----
  const TileStream<HD, NW> ld(wave, lane, 2 * G.ks[1] * rs, 2 * G.vs[1] * rs);
  const int per_tile = 2 * ld.count();
  const unsigned lds0 = lds_addr(smem);
  int kl = k;
  int64_t tl = t;
  BlockWalk lw = cw;
  int issued = 0;
  auto issue = [&](int stage) {
    const int64_t j0 = tl * BK;
    const int64_t p0 = tile_pos(lw.kv_start, tl);
    ld.load(kb + 2 * p0 * G.ks[1], vb + 2 * p0 * G.vs[1], lds0 + stage * STAGE,
            lds0 + stage * STAGE + TB, lw.len_kv - j0);
    ++issued;
    next(kl, tl, lw);
  };
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (kl < nblk) issue(s);
  // the Q fragments and the first tiles have landed; from here on the only
  // vector-memory operations in flight are the tile loads counted above
  vm_wait<0>();

  const int a_off = TL::a_off(lane);
  const int t_off = TL::t_off(lane);
  int it = 0;
  while (k < nblk) {
    // this wave's loads of tile `it` have landed once at most the loads of
    // the tiles issued after it are outstanding; the barrier then publishes
    // every wave's part and frees the stage read in the previous iteration
    vm_wait((issued - 1 - it) * per_tile);
    __syncthreads();
    if (kl < nblk) issue((it + NS - 1) % NS);

    const int64_t j0 = t * BK;
    // this wave's row ii sees the tile's key jj iff jj <= ii + dw (global
    // positions, in units of the row step)
    int64_t dw;
    if constexpr (RUNS) {
      const int64_t gk = tile_pos(cw.kv_start, t);
      dw = rs == 1 ? gq_w - gk : floor_div64(gq_w - gk, rs);
    } else {
      dw = i0w + cw.diag - j0;
    }
    if (dw + 31 >= 0) {  // some row of this wave sees a key of the tile
      const char *kt = smem + (it % NS) * STAGE;
      const char *vt = kt + TB;
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      // S at raised issue priority: while this wave feeds the matrix core,
      // the SIMD's other wave fills the VALU slots with its softmax
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s0 = mfma32(__builtin_bit_cast(bf16x8, ld16(kt + a_off + ks * 32)), qf[ks], s0);
        s1 = mfma32(__builtin_bit_cast(bf16x8, ld16(kt + a_off + 32 * RB + ks * 32)), qf[ks], s1);
      }
      sched_lds_ahead<2 * KS, 4>();
      __builtin_amdgcn_s_setprio(0);
      // element i of s0 / s1 is key j0 + 32*(i/16) + 16*((i%16)/8) + 8g + i%8
      // (global position of key jj of the tile: gk + jj * rs)
      const int64_t gk = DOCS ? tile_pos(cw.kv_start, t) : 0;
      const bool masked = (dw < BK - 1) || (j0 + BK > cw.len_kv) || (DOCS && gk < qlo_w);
      if (masked) {
        // key j0 + jj is visible iff lo <= jj <= lim: lim from the causal
        // rule and the piece's end, lo from the row's document start
        const int64_t lim64 = c32 + dw;
        const int64_t len64 = cw.len_kv - 1 - j0;
        const int64_t m64 = lim64 < len64 ? lim64 : len64;
        const int lim = static_cast<int>(m64 < -1 ? -1 : (m64 > BK ? BK : m64));
        if constexpr (DOCS) {
          int lo = 0;
          if (qlo > gk) {
            const unsigned ahead = static_cast<unsigned>(qlo - gk), step = static_cast<unsigned>(rs);
            const unsigned l = (ahead + step - 1) / step;
            lo = l > static_cast<unsigned>(BK) ? BK : static_cast<int>(l);
          }
          const unsigned span = static_cast<unsigned>(lim + 1 > lo ? lim + 1 - lo : 0);
          const int x = 8 * g - lo;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kc = 16 * (i / 8) + (i % 8);
            if (static_cast<unsigned>(x + kc) >= span) s0[i] = -INFINITY;
            if (static_cast<unsigned>(x + kc + 32) >= span) s1[i] = -INFINITY;
          }
        } else {
          const int x = 8 * g - lim;  // key jj = kc + 8g is masked iff jj > lim
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kc = 16 * (i / 8) + (i % 8);
            if (x + kc > 0) s0[i] = -INFINITY;
            if (x + kc + 32 > 0) s1[i] = -INFINITY;
          }
        }
      }
      // P = 2^(s c - m) with a per-row reference m.  Exact for any m (the
      // output and the row sum share it); m only has to keep P in range.
      // Tiles that need a mask, and every tile until all rows of the wave
      // have a reference, take the full path: the tile's row max raises the
      // reference when it grows by more than TAU, so P <= 2^TAU.  Otherwise
      // P is formed against the current reference right away and the tile
      // falls back to the full path only if some row half-sum exceeds
      // PSUM_MAX (every P of it is then <= PSUM_MAX as well).
      float psum = 0.f;
      bf16x8 pb[4];
      auto probs = [&](float m_use) {
        psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p0 = fast_exp2(__builtin_fmaf(s0[i], c, -m_use));
          const float p1 = fast_exp2(__builtin_fmaf(s1[i], c, -m_use));
          psum += p0 + p1;
          pb[i / 8][i % 8] = static_cast<__bf16>(p0);
          pb[2 + i / 8][i % 8] = static_cast<__bf16>(p1);
        }
      };
      bool full = masked || !ref_ok;
      if (!full) {
        probs(m_run);
        full = __any(psum > PSUM_MAX);
      }
      if (full) {
        // row max with the NaN-propagating maximum: v_maximum3_f32 needs no
        // operand canonicalisation (the scores hold no NaN; -inf is kept)
        float mx = __builtin_elementwise_maximum(s0[0], s1[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i)
          mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s0[i], s1[i]));
        mx = pair_max(mx) * c;
        // raise the reference max only when it grows by more than TAU
        if (__any(mx > m_run + TAU)) {
          const float m_new = __builtin_elementwise_maximum(m_run, mx);
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
        probs(m_run == -INFINITY ? 0.f : m_run);
        ref_ok = !__any(m_run == -INFINITY);
      }
      l_run += psum;
      // O^T += V^T P^T: A = V^T (d x 16 keys) read transposed from the V tile
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int o = t_off + 16 * kk * RB;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = mfma32(cat8(lds_read_tr(vt + o + 64 * dt), lds_read_tr(vt + o + 4 * RB + 64 * dt)),
                           pb[kk], acc[dt]);
      }
    }
    next(k, t, cw);
    ++it;
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  const int64_t row = i0w + c32;
  if (row < seg.len_q) {
    if (OUT == 0) {
      const int64_t pos = pos_of(seg.q_start, row);
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
    } else if (OUT == 2) {
      // merge this block's normalised partial into the accumulator row of the
      // same query (one ring step's blocks have distinct query rows)
      const int64_t arow = (static_cast<int64_t>(b) * G.hq + h) * G.seqlen + pos_of(seg.q_start, row);
      float *ao = static_cast<float *>(a.o) + arow * HD;
      float wa, wp, lnew;
      merge_weights(a.lse[arow], lse, wa, wp, lnew);
      wp *= inv;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 *p4 = reinterpret_cast<f32x4 *>(ao + 32 * dt + 8 * q4 + 4 * g);
          const f32x4 av = *p4;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = (wa == 0.f ? 0.f : wa * av[e]) + (wp == 0.f ? 0.f : wp * acc[dt][4 * q4 + e]);
          *p4 = v;
        }
      if (g == 0) a.lse[arow] = lnew;
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

template <int HD, bool RUNS, bool DOCS>
void launch_fwd_docs(const FwdArgs &a, dim3 gr, hipStream_t s) {
  const dim3 bl(NT);
  if (a.out_mode == 0 && a.interleave)
    hipLaunchKernelGGL((fwd_bf16_kernel<HD, 0, true, RUNS, DOCS, true>), gr, bl, 0, s, a);
  else if (a.out_mode == 0)
    hipLaunchKernelGGL((fwd_bf16_kernel<HD, 0, true, RUNS, DOCS>), gr, bl, 0, s, a);
  else if (a.out_mode == 2)
    hipLaunchKernelGGL((fwd_bf16_kernel<HD, 2, true, RUNS, DOCS>), gr, bl, 0, s, a);
  else if (a.segs)
    hipLaunchKernelGGL((fwd_bf16_kernel<HD, 1, true, RUNS, DOCS>), gr, bl, 0, s, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<HD, 1, false, RUNS, DOCS>), gr, bl, 0, s, a);
}

template <int HD, bool RUNS>
void launch_fwd_variant(const FwdArgs &a, dim3 gr, hipStream_t s) {
  if (a.g.n_docs)
    launch_fwd_docs<HD, RUNS, true>(a, gr, s);
  else
    launch_fwd_docs<HD, RUNS, false>(a, gr, s);
}

hipError_t launch_fwd_bf16(const FwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  grid = xcd_grid(grid);  // whole groups of 8 (see xcd_item)
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.out_mode != 1 && !a.segs) return hipErrorInvalidValue;
  const dim3 gr(static_cast<unsigned>(grid));
  if (hd == 128) {
    if (a.runs)
      launch_fwd_variant<128, true>(a, gr, s);
    else
      launch_fwd_variant<128, false>(a, gr, s);
  } else if (hd == 64) {
    if (a.runs)
      launch_fwd_variant<64, true>(a, gr, s);
    else
      launch_fwd_variant<64, false>(a, gr, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfa
