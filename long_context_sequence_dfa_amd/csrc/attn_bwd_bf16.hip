// attn_bwd_bf16.hip -- bf16 backward of blockwise causal attention on gfx950.
//
// The backward keeps no attention matrix: P is recomputed from the saved
// log-sum-exp (FlashAttention glossary page, first two paragraphs;
// "rematerialisation-aware gradient checkpointing" on the DistFlashAttn
// paper record).  With D_i = rowsum(dO_i * O_i):
//   P_ij = e^{scale q_i.k_j - LSE_i},  dP_ij = dO_i.v_j,  dS_ij = P_ij (dP_ij - D_i)
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
//
// Two kernels, no atomics, deterministic (8 waves, 32 rows per wave):
//  * dq: query-major, shaped like the forward -- a workgroup owns 256 query
//    rows, walks its query piece's blocks in the host table's order and computes
//    S^T = K Q^T, dP^T = V dO^T and dQ^T += K^T dS^T on the matrix cores.
//    Each lane owns one query column, so LSE_i and D_i are per-lane scalars.
//  * dkdv: key-major -- a workgroup owns 256 key rows, walks every block
//    that reads its key piece and every query head of its group, and
//    computes S = Q K^T, dV^T += dO^T P, dP = dO V^T and dK^T += Q^T dS, so
//    S and P are formed once for both gradients.  Each lane owns one key
//    column.  K lives in registers as an MFMA operand; the V operand is
//    parked in LDS, which keeps the two accumulator sets of a wave within
//    the 256 registers that let two waves share every SIMD.
// With packed documents (Striped Attention Guide, "Production Deployment and
// Best Practices", item 3) a pair is kept only inside one document: the
// query-major kernel masks keys before the row's document start, the
// key-major ones queries at or after the key's document end, and both skip
// the tiles no row of the workgroup can see.
// Both stream 64-row K/V (or Q/dO) tiles through LDS stages with direct
// loads issued one stage ahead of the oldest resident tile (stream_lds.h);
// transposed operands come from ds_read_b64_tr_b16 on the row-major tiles.
#include "dfa_internal.h"
#include "stream_lds.h"

#include <stdint.h>

namespace dfa {
namespace {

constexpr int NW = kBwdWaves;  // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int NS = kBwdStages; // tiles resident in LDS (NS - 1 in flight)

// ============================ dQ (query-major) ============================
constexpr int DQ_BQ = kDqTileQ;  // 32 query rows per wave
constexpr int DQ_BK = 64;
static_assert(DQ_BQ == 32 * NW, "one 32-query column block per wave");

// RUNS: pieces made of runs (stripe blocks), visibility from global
// positions; otherwise rows start + i*stride and each block's diagonal.
// ILV: the interleaved walk (groups of kIlvTiles key tiles, as in the forward).
template <int HD, bool RUNS, bool DOCS, bool ILV>
__global__ __launch_bounds__(NT, 8 / NW) void dq_bf16_kernel(BwdArgs a) {
  using TL = Tile64<HD>;
  static_assert(TL::ROWS == DQ_BK, "key tiles are 64 rows");
  constexpr int RB = TL::RB, TB = TL::TB, STAGE = 2 * TB;  // K, V
  constexpr int KS = HD / 16, DT = HD / 32;
  __shared__ __attribute__((aligned(16))) char smem[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const Geom &G = a.g;
  const float c = G.scale_log2;
  const int BH = G.batch * G.hq;
  int bh;
  int64_t ti;
  if (!xcd_item(blockIdx.x, a.n_qtiles, BH, bh, ti)) return;
  const Tile tl = ld_table(a.qtiles + ti);
  const QSeg seg = ld_table(a.qsegs + tl.seg);
  const int b = bh / G.hq, h = bh % G.hq, hk = h / G.group;
  const int64_t i0 = static_cast<int64_t>(tl.tile) * DQ_BQ;
  const int64_t i0w = i0 + wave * 32;
  const int64_t iend = (i0 + DQ_BQ < seg.len_q) ? i0 + DQ_BQ : seg.len_q;
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
    return start + t_ * (DQ_BK * seg.stride);
  };
  const int64_t q_last = RUNS ? pos_of(seg.q_start, iend - 1) : 0;
  const int64_t gq_w = RUNS ? pos_of(seg.q_start, i0w) : 0;
  // packed documents: this lane's row sees keys at positions >= qlo only;
  // qlo_w is the wave's largest bound, wlo the workgroup's smallest
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

  const char *kb = static_cast<const char *>(a.k) + 2 * (b * G.ks[0] + hk * G.ks[2]);
  const char *vb = static_cast<const char *>(a.v) + 2 * (b * G.vs[0] + hk * G.vs[2]);

  // walk over (block, key tile); t0 skips tiles before wlo
  struct Walk {
    int64_t kv_start, len_kv, diag, ntiles, t0, te;
  };
  auto walk_of = [&](const KvRef &r) {  // key tiles holding a key at or before the last row
    int64_t hi;
    if constexpr (RUNS) {
      hi = piece_count_le(r.kv_start, seg.stride, seg.run, r.len_kv, q_last);
    } else {
      hi = iend + r.diag_offset;
      if (hi > r.len_kv) hi = r.len_kv;
    }
    const int64_t t0 = wlo > 0 ? piece_count_le(r.kv_start, seg.stride, seg.run, r.len_kv, wlo - 1) / DQ_BK : 0;
    const int64_t nt = hi > 0 ? (hi + DQ_BK - 1) / DQ_BK : 0;
    return Walk{r.kv_start, r.len_kv, r.diag_offset, nt, t0, nt};
  };
  auto walk = [&](int k) { return walk_of(ld_table(a.qkv + seg.blk_begin + k)); };
  const int nblk = seg.blk_count;
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
      const auto w = walk_of(a.qkv[seg.blk_begin + lane]);
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
  auto first = [&](int &k_, Walk &w_) {
    while (k_ < nblk) {
      w_ = walk(k_);
      if (w_.ntiles > w_.t0) return;
      ++k_;
    }
  };
  auto next = [&](int &k_, int64_t &t_, Walk &w_) {
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
  Walk cw{0, 0, 0, 0, 0, 0};
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

  // K and V stream
  const TileStream<HD, NW> ld(wave, lane, 2 * G.ks[1] * rs, 2 * G.vs[1] * rs);
  const int per_tile = 2 * ld.count();
  const unsigned lds0 = lds_addr(smem);
  int kl = k;
  int64_t tl_ = t;
  Walk lw = cw;
  int issued = 0;
  auto issue = [&](int stage) {
    const int64_t jt = tl_ * DQ_BK;
    const int64_t p0 = tile_pos(lw.kv_start, tl_);
    ld.load(kb + 2 * p0 * G.ks[1], vb + 2 * p0 * G.vs[1], lds0 + stage * STAGE,
            lds0 + stage * STAGE + TB, lw.len_kv - jt);
    ++issued;
    next(kl, tl_, lw);
  };
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (kl < nblk) issue(st);

  // rows past the piece read its last row; they are never stored
  bf16x8 qf[KS], df[KS];
  const int64_t row = i0w + c32;
  const bool valid = row < seg.len_q;
  const int64_t pos = pos_of(seg.q_start, valid ? row : seg.len_q - 1);
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
  const float lse2 = a.lse2[lr];
  const float ndd = a.dd[lr];  // -D of this lane's row
  // the operands above and the first tiles have landed; from here on the only
  // vector-memory operations in flight are the tile loads
  vm_wait<0>();
  // dP^T accumulations start from -D, so they end at dP - D directly
  f32x16 nd;
#pragma unroll
  for (int i = 0; i < 16; ++i) nd[i] = ndd;

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  const int a_off = TL::a_off(lane);
  const int t_off = TL::t_off(lane);
  int it = 0;
  while (k < nblk) {
    vm_wait((issued - 1 - it) * per_tile);  // this wave's part of tile `it` landed
    __syncthreads();                        // every part landed; stage it-1 free
    if (kl < nblk) issue((it + NS - 1) % NS);

    const int64_t j0 = t * DQ_BK;
    // this wave's row ii sees the tile's key jj iff jj <= ii + dw
    int64_t dw;
    if constexpr (RUNS) {
      const int64_t gk = tile_pos(cw.kv_start, t);
      dw = rs == 1 ? gq_w - gk : floor_div64(gq_w - gk, rs);
    } else {
      dw = i0w + cw.diag - j0;
    }
    if (dw + 31 >= 0) {
      const char *kt = smem + (it % NS) * STAGE;
      const char *vt = kt + TB;
      const int64_t gk = DOCS ? tile_pos(cw.kv_start, t) : 0;  // position of key 0 of the tile
      const bool need_mask = (dw < DQ_BK - 1) || (j0 + DQ_BK > cw.len_kv) || (DOCS && gk < qlo_w);
      int x = 0;
      unsigned span = 0;
      if (need_mask) {
        // element i of half kh is local key jj = 32kh + 16(i/8) + 8g + i%8,
        // visible iff lo <= jj <= lim (causal rule and piece end give lim,
        // the row's document start gives lo); x = 8g - lo
        const int64_t lim64 = c32 + dw, len64 = cw.len_kv - 1 - j0;
        const int64_t m64 = lim64 < len64 ? lim64 : len64;
        const int lim = static_cast<int>(m64 < -1 ? -1 : (m64 > DQ_BK ? DQ_BK : m64));
        int lo = 0;
        if (DOCS && qlo > gk) {
          const unsigned ahead = static_cast<unsigned>(qlo - gk), step = static_cast<unsigned>(rs);
          const unsigned l = (ahead + step - 1) / step;
          lo = l > static_cast<unsigned>(DQ_BK) ? DQ_BK : static_cast<int>(l);
        }
        span = static_cast<unsigned>(lim + 1 > lo ? lim + 1 - lo : 0);
        x = 8 * g - lo;
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {  // two halves of 32 keys
        f32x16 sv = f32x16{}, pv = nd;
        // the S/dP products at raised issue priority: while this wave feeds
        // the matrix core, the SIMD's other wave fills the VALU slots
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int o = a_off + 32 * kh * RB + ks * 32;
          sv = mfma32(__builtin_bit_cast(bf16x8, ld16(kt + o)), qf[ks], sv);
          pv = mfma32(__builtin_bit_cast(bf16x8, ld16(vt + o)), df[ks], pv);
        }
        __builtin_amdgcn_s_setprio(0);
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (static_cast<unsigned>(x + 32 * kh + 16 * (i / 8) + (i % 8)) >= span) sv[i] = -INFINITY;
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pa = fast_exp2(__builtin_fmaf(sv[i], c, -lse2));
          dsb[i / 8][i % 8] = static_cast<__bf16>(pa * pv[i]);
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
    next(k, t, cw);
    ++it;
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
constexpr int KV_BK = kBwdTileKV;  // 32 key rows per wave
constexpr int KV_BQ = 64;          // query rows per streamed tile
constexpr int KV_NS = kKvStages;   // Q/dO tiles resident in LDS
static_assert(KV_BK == 32 * NW, "one 32-key column block per wave");

// Key-major gradient kernel: per (key tile, query tile) pair S, P, dV, dP,
// dS and dK, in that order.  Registers per lane: K operand 4 HD/16, two
// accumulator sets 2 HD/2, one 32-query slice of S and dP; the V operand
// (HD/16 fragments of 16 bytes per lane) waits in LDS, where each lane reads
// back only what it wrote.  LDS: KV_NS stages of Q, dO and the row
// statistics plus the parked V fragments of the workgroup.
template <int HD, bool RUNS, bool DOCS>
__global__ __launch_bounds__(NT, 8 / NW) void dkdv_bf16_kernel(BwdArgs a) {
  using TL = Tile64<HD>;
  static_assert(TL::ROWS == KV_BQ, "query tiles are 64 rows");
  constexpr int RB = TL::RB;
  constexpr int TB = TL::TB;
  constexpr int STAGE = 2 * TB + 2 * KV_BQ * 4;  // Q, dO, LSE*log2(e), -D
  constexpr int KS = HD / 16, DT = HD / 32;
  constexpr int VPARK = KS * 1024;               // parked V fragments per wave
  static_assert(KV_NS * STAGE + NW * VPARK <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) char smem[KV_NS * STAGE + NW * VPARK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const Geom &G = a.g;
  const float c = G.scale_log2;
  const int BH = G.batch * G.hkv;
  // batch-head fastest: splitting the XCDs by head measured no faster here
  const int64_t bid = blockIdx.x;
  if (bid >= static_cast<int64_t>(a.n_kvtiles) * BH) return;
  const int bh = static_cast<int>(bid % BH);
  const Tile tl = ld_table(a.kvtiles + bid / BH);
  const KvSeg seg = ld_table(a.kvsegs + tl.seg);
  const int b = bh / G.hkv, hk = bh % G.hkv;
  const int64_t j0 = static_cast<int64_t>(tl.tile) * KV_BK;
  const int64_t j0w = j0 + wave * 32;
  const int64_t col = j0w + c32;  // this lane's key row
  const bool valid = col < seg.len_kv;
  auto pos_of = [&](int64_t start, int64_t i) {
    return RUNS ? piece_pos(start, seg.stride, seg.run, i) : start + i * seg.stride;
  };
  const int64_t pos = pos_of(seg.kv_start, valid ? col : seg.len_kv - 1);
  const int64_t rs = RUNS ? piece_row_step(seg.stride, seg.run) : seg.stride;  // row step in a tile
  // global position of the first row of 64-row tile t of a piece (a run is
  // 64 * 2^tsh rows, so the tile's run and offset are a shift and a mask)
  const int tsh = RUNS && seg.run > 1 ? __builtin_ctzll(static_cast<uint64_t>(seg.run)) - 6 : 0;
  auto tile_pos = [&](int64_t start, int64_t t_) {
    if constexpr (RUNS) {
      if (seg.run > 1) return start + (t_ >> tsh) * seg.stride + ((t_ & ((int64_t{1} << tsh) - 1)) << 6);
    }
    return start + t_ * (KV_BQ * seg.stride);
  };
  // global positions of the workgroup's and this wave's first key
  const int64_t gk0 = RUNS ? pos_of(seg.kv_start, j0) : 0;
  const int64_t gk_w = RUNS ? pos_of(seg.kv_start, j0w) : 0;
  // packed documents: queries at positions >= khi cannot see this lane's
  // key; khi_w is the wave's smallest bound (its first key), whi the
  // workgroup's largest (its last key) -- positions rise with the row index
  int32_t khi = INT32_MAX, khi_w = INT32_MAX;
  int64_t whi = INT64_MAX;
  if constexpr (DOCS) {
    int64_t lo_, hi;
    doc_range(G.docs, G.n_docs, pos, lo_, hi);
    khi = static_cast<int32_t>(hi);
    khi_w = __builtin_amdgcn_readfirstlane(khi);
    const int64_t jl = (j0 + KV_BK < seg.len_kv ? j0 + KV_BK : seg.len_kv) - 1;
    doc_range(G.docs, G.n_docs, pos_of(seg.kv_start, jl), lo_, hi);
    whi = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(hi));
  }

  // walk over (group head, block, query tile)
  struct Walk {
    int64_t q_start, len_q, diag, t0, t1;  // query tiles [t0, t1)
    int h;
  };
  auto walk = [&](int gi, int k) {
    const QRef r = ld_table(a.kvq + seg.blk_begin + k);
    Walk w{r.q_start, r.len_q, r.diag_offset, 0, 0, hk * G.group + gi};
    // the first query row at or after the workgroup's first key
    int64_t lo;
    if constexpr (RUNS) {
      lo = piece_count_le(r.q_start, seg.stride, seg.run, r.len_q, gk0 - 1);
    } else {
      lo = j0 - r.diag_offset;
      if (lo < 0) lo = 0;
    }
    // the query rows before the first position after the last key's document
    const int64_t hi = DOCS ? piece_count_le(r.q_start, seg.stride, seg.run, r.len_q, whi - 1)
                                       : r.len_q;
    if (lo < hi) {
      w.t0 = lo / KV_BQ;
      w.t1 = (hi + KV_BQ - 1) / KV_BQ;
    }
    return w;
  };
  const int nblk = seg.blk_count, ngrp = G.group;
  auto first = [&](int &gi_, int &k_, Walk &w_) {
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
  auto next = [&](int &gi_, int &k_, int64_t &t_, Walk &w_) {
    if (++t_ < w_.t1) return;
    ++k_;
    first(gi_, k_, w_);
    t_ = w_.t0;
  };
  int gi = 0, k = 0;
  Walk cw{};
  first(gi, k, cw);
  int64_t t = cw.t0;

  // Q/dO stream; LSE*log2(e) and -D of the 64 rows go to LDS with one 4-byte
  // direct load each, issued by the last two waves (they have the fewest
  // tile instructions)
  const TileStream<HD, NW> ld(wave, lane, 2 * G.qs[1] * rs, 2 * G.os[1] * rs);
  const bool stats_wave = wave >= NW - 2;
  const int per_tile = 2 * ld.count() + (stats_wave ? 1 : 0);
  const unsigned lds0 = lds_addr(smem);
  int gl = gi, kl = k;
  int64_t tl_ = t;
  Walk lw = cw;
  int issued = 0;
  auto issue = [&](int stage) {
    const int64_t i0 = tl_ * KV_BQ;
    const int64_t p0 = tile_pos(lw.q_start, tl_);
    const char *qb = static_cast<const char *>(a.q) + 2 * (b * G.qs[0] + p0 * G.qs[1] + lw.h * G.qs[2]);
    const char *db = static_cast<const char *>(a.dout) + 2 * (b * G.os[0] + p0 * G.os[1] + lw.h * G.os[2]);
    const unsigned sb = lds0 + stage * STAGE;
    ld.load(qb, db, sb, sb + TB, lw.len_q - i0);
    if (stats_wave) {
      const int64_t rows = lw.len_q - i0;
      const unsigned r = static_cast<unsigned>(lane < rows ? lane : rows - 1);
      const int64_t row0 = (static_cast<int64_t>(b) * G.hq + lw.h) * G.seqlen + p0;
      const float *src = wave == NW - 2 ? a.lse2 : a.dd;
      dma4(src + row0, r * static_cast<unsigned>(rs) * 4u,
           sb + 2 * TB + (wave == NW - 2 ? 0 : KV_BQ * 4));
    }
    ++issued;
    next(gl, kl, tl_, lw);
  };
#pragma unroll
  for (int st = 0; st < KV_NS - 1; ++st)
    if (gl < ngrp) issue(st);

  // K and V as B operands of S = Q K^T and dP = dO V^T: lane (c32, g) holds
  // row c32's elements 16 ks + 8 g .. +8.  Rows past the key piece read its
  // last row and are never stored.  V's fragments go to this lane's own
  // 16-byte slots of the parking area (slot ks at 1024 ks: a wave's reads of
  // one slot cover 1 KB without bank conflicts).
  bf16x8 kf[KS];
  char *vpark = smem + KV_NS * STAGE + wave * VPARK + lane * 16;
  {
    const char *ksrc = static_cast<const char *>(a.k) + 2 * (b * G.ks[0] + pos * G.ks[1] + hk * G.ks[2]);
    const char *vsrc = static_cast<const char *>(a.v) + 2 * (b * G.vs[0] + pos * G.vs[1] + hk * G.vs[2]);
    bf16x8 vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, ld16(ksrc + (2 * ks + g) * 16));
      vf[ks] = __builtin_bit_cast(bf16x8, ld16(vsrc + (2 * ks + g) * 16));
    }
    vm_wait<0>();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<bf16x8 *>(vpark + ks * 1024) = vf[ks];
  }
  f32x16 acck[DT], accv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acck[dt] = accv[dt] = f32x16{};

  // per-lane operand offsets (independent of the tile); loop indices only
  // add compile-time constants to them
  const int a_off = TL::a_off(lane);
  const int t_off = TL::t_off(lane);
  int it = 0;
  while (gi < ngrp) {
    vm_wait((issued - 1 - it) * per_tile);  // this wave's part of tile `it` landed
    __syncthreads();                        // every part landed; stage it-1 free
    if (gl < ngrp) issue((it + KV_NS - 1) % KV_NS);

    const int64_t qi0 = t * KV_BQ;
    // query row qq of the tile sees this wave's key c32 iff c32 <= qq + dw
    int64_t dw;
    if constexpr (RUNS) {
      const int64_t gq = tile_pos(cw.q_start, t);
      dw = rs == 1 ? gq - gk_w : floor_div64(gq - gk_w, rs);
    } else {
      dw = qi0 + cw.diag - j0w;
    }
    // some pair of this wave visible: largest query row sees smallest key row
    if (KV_BQ - 1 + dw >= 0) {
      const char *qt = smem + (it % KV_NS) * STAGE;
      const char *dt_ = qt + TB;
      const float *lt = reinterpret_cast<const float *>(qt + 2 * TB);
      const float *ddt = lt + KV_BQ;
      // local query qq (0..63) of the tile is kept iff lo <= qq < hi
      // packed documents: global position of the tile's first and last query
      const int64_t gq0 = DOCS ? tile_pos(cw.q_start, t) : 0;
      // the tile's last row (tiles never straddle a run)
      const int64_t gql = DOCS ? gq0 + ((qi0 + KV_BQ < cw.len_q ? KV_BQ : cw.len_q - qi0) - 1) * rs : 0;
      const bool need_mask = (dw < 31) || (qi0 + KV_BQ > cw.len_q) || (DOCS && gql >= khi_w);
      int lo = 0, hi = KV_BQ;
      if (need_mask) {
        const int64_t lo64 = c32 - dw, hi64 = cw.len_q - qi0;
        lo = static_cast<int>(lo64 < 0 ? 0 : (lo64 > KV_BQ ? KV_BQ : lo64));
        hi = static_cast<int>(hi64 > KV_BQ ? KV_BQ : hi64);
        if (DOCS) {  // queries of the tile before the end of the key's document
          const int dh = khi <= gq0 ? 0
                                    : static_cast<int>((static_cast<unsigned>(khi - gq0) + static_cast<unsigned>(rs) - 1) /
                                                       static_cast<unsigned>(rs));
          hi = dh < hi ? dh : hi;
        }
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {  // two halves of 32 query rows
        const char *qa = qt + a_off + 32 * mt * RB, *da = dt_ + a_off + 32 * mt * RB;
        f32x16 s = f32x16{};
        __builtin_amdgcn_s_setprio(1);  // see the dQ kernel
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma32(__builtin_bit_cast(bf16x8, ld16(qa + ks * 32)), kf[ks], s);
        sched_lds_ahead<KS, 2>();
        __builtin_amdgcn_s_setprio(0);
        // element i is query row qi0 + 32mt + 16(i/8) + 8g + i%8; masked
        // scores become -inf (probability 0)
        if (need_mask) {
          const int x = 8 * g - lo;  // qq - lo without the element's constant part
          const unsigned span = static_cast<unsigned>(hi > lo ? hi - lo : 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const unsigned rel = static_cast<unsigned>(x + 32 * mt + 16 * (i / 8) + (i % 8));
            if (rel >= span) s[i] = -INFINITY;
          }
        }
        // P (fp32, in place of S: it is needed again for dS) and its bf16
        // copy, the B operand of dV
        bf16x8 pb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int qoff = 32 * mt + 16 * u + 8 * g;
          const f32x4 la = *reinterpret_cast<const f32x4 *>(lt + qoff);
          const f32x4 lb = *reinterpret_cast<const f32x4 *>(lt + qoff + 4);
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int i = 8 * u + w;
            s[i] = fast_exp2(__builtin_fmaf(s[i], c, -(w < 4 ? la[w] : lb[w - 4])));
            pb[u][w] = static_cast<__bf16>(s[i]);
          }
        }
        // dV^T += dO^T P: A operand read transposed from the dO tile
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int o = t_off + 16 * (2 * mt + u) * RB;
#pragma unroll
          for (int e = 0; e < DT; ++e)
            accv[e] = mfma32(cat8(lds_read_tr(dt_ + o + 64 * e), lds_read_tr(dt_ + o + 4 * RB + 64 * e)),
                             pb[u], accv[e]);
        }
        // dP = dO V^T, accumulated from -D (the tile's row statistics), so
        // that dS = P (dP - D) is one product per element
        f32x16 dpm;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int qoff = 32 * mt + 16 * u + 8 * g;
          const f32x4 da4 = *reinterpret_cast<const f32x4 *>(ddt + qoff);
          const f32x4 db4 = *reinterpret_cast<const f32x4 *>(ddt + qoff + 4);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            dpm[8 * u + w] = da4[w];
            dpm[8 * u + 4 + w] = db4[w];
          }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          dpm = mfma32(__builtin_bit_cast(bf16x8, ld16(da + ks * 32)),
                       *reinterpret_cast<const bf16x8 *>(vpark + ks * 1024), dpm);
        sched_lds_ahead<KS, 2, 2>();  // dO and V fragments
        __builtin_amdgcn_s_setprio(0);
        bf16x8 sb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int w = 0; w < 8; ++w) sb[u][w] = static_cast<__bf16>(s[8 * u + w] * dpm[8 * u + w]);
        // dK^T += Q^T dS: A operand read transposed from the Q tile
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int o = t_off + 16 * (2 * mt + u) * RB;
#pragma unroll
          for (int e = 0; e < DT; ++e)
            acck[e] = mfma32(cat8(lds_read_tr(qt + o + 64 * e), lds_read_tr(qt + o + 4 * RB + 64 * e)),
                             sb[u], acck[e]);
        }
      }
    }
    next(gi, k, t, cw);
    ++it;
  }
  if (!valid) return;
  // dK = scale * acck, dV = accv; element 4 q4 + e of block dt is column
  // 32 dt + 8 q4 + 4 g + e of this lane's key row
  char *dko = static_cast<char *>(a.dk) + 2 * (b * G.ks[0] + pos * G.ks[1] + hk * G.ks[2]);
  char *dvo = static_cast<char *>(a.dv) + 2 * (b * G.vs[0] + pos * G.vs[1] + hk * G.vs[2]);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 xk, xv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xk[e] = static_cast<__bf16>(acck[dt][4 * q4 + e] * G.scale);
        xv[e] = static_cast<__bf16>(accv[dt][4 * q4 + e]);
      }
      *reinterpret_cast<bf16x4 *>(dko + 2 * (32 * dt + 8 * q4 + 4 * g)) = xk;
      *reinterpret_cast<bf16x4 *>(dvo + 2 * (32 * dt + 8 * q4 + 4 * g)) = xv;
    }
}

}  // namespace

template <int HD, bool RUNS>
void launch_dq_variant(const BwdArgs &a, dim3 gr, hipStream_t s) {
  if (a.g.n_docs && a.interleave)
    hipLaunchKernelGGL((dq_bf16_kernel<HD, RUNS, true, true>), gr, dim3(NT), 0, s, a);
  else if (a.g.n_docs)
    hipLaunchKernelGGL((dq_bf16_kernel<HD, RUNS, true, false>), gr, dim3(NT), 0, s, a);
  else if (a.interleave)
    hipLaunchKernelGGL((dq_bf16_kernel<HD, RUNS, false, true>), gr, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((dq_bf16_kernel<HD, RUNS, false, false>), gr, dim3(NT), 0, s, a);
}

hipError_t launch_bwd_dq_bf16(const BwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  grid = xcd_grid(grid);  // whole groups of 8 (see xcd_item)
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 gr(static_cast<unsigned>(grid));
  if (hd == 128) {
    if (a.runs)
      launch_dq_variant<128, true>(a, gr, s);
    else
      launch_dq_variant<128, false>(a, gr, s);
  } else if (hd == 64) {
    if (a.runs)
      launch_dq_variant<64, true>(a, gr, s);
    else
      launch_dq_variant<64, false>(a, gr, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HD, bool RUNS>
void launch_dkdv_docs(const BwdArgs &a, dim3 gr, hipStream_t s) {
  if (a.g.n_docs)
    hipLaunchKernelGGL((dkdv_bf16_kernel<HD, RUNS, true>), gr, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((dkdv_bf16_kernel<HD, RUNS, false>), gr, dim3(NT), 0, s, a);
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs &a, int hd, int64_t grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 gr(static_cast<unsigned>(grid));
  if (hd == 128) {
    if (a.runs)
      launch_dkdv_docs<128, true>(a, gr, s);
    else
      launch_dkdv_docs<128, false>(a, gr, s);
  } else if (hd == 64) {
    if (a.runs)
      launch_dkdv_docs<64, true>(a, gr, s);
    else
      launch_dkdv_docs<64, false>(a, gr, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfa
