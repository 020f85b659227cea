// api.cpp -- host runtime behind the C ABI in include/dfa.h: argument
// validation, work planning over a block list, workspace layout and kernel
// launches on the caller's stream.
//
// Planning.  A block list is regrouped two ways:
//  * by query piece (q_start, len_q, stride, run): each piece keeps its blocks
//    ordered by the key piece's first position (ring step breaks ties) and is
//    cut into query tiles (forward, dQ);
//  * by key piece (kv_start, len_kv, stride, run): each keeps the blocks that
//    read it, ordered by the query piece's first position, cut into key tiles
//    (dK, dV).
// Fused kernels merge a row's blocks online, so their order changes only the
// rounding, and a position order shared by every piece makes workgroups of
// one head and of different virtual ranks that run side by side (similar
// cost) read the same tiles at about the same time, from L2 (with stripe
// blocks of 64 tokens the ring-step order left the L2 almost no reuse).
// Stepwise mode keeps ring-step order (one launch per step).
// Work tiles are sorted by decreasing cost so the heaviest start first.  The
// tables travel to the device in the caller's workspace; the kernels read
// key/value rows of the owning rank in place, so a ring step costs no copy
// (the buffer hand-off of the DistFlashAttn Guide, "Core Innovation 2").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <initializer_list>
#include <map>
#include <tuple>
#include <vector>

#include "dfa.h"
#include "dfa_internal.h"

namespace {

using dfa::KvRef;
using dfa::KvSeg;
using dfa::QRef;
using dfa::QSeg;
using dfa::Tile;

constexpr size_t kAlign = 256;
constexpr int kCostTileKV = 64;  // granularity of the cost estimate

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

dfa_status check_desc(const dfa_attn_desc *d) {
  if (!d) return DFA_E_NULL;
  if (d->dtype != DFA_BF16 && d->dtype != DFA_F32) return DFA_E_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return DFA_E_UNSUPPORTED;
  if (d->batch < 1 || d->heads_q < 1 || d->heads_kv < 1 || d->seqlen < 1) return DFA_E_SHAPE;
  if (d->heads_q % d->heads_kv) return DFA_E_SHAPE;
  // the kernels take each row's maximum of scale * q.k as its reference:
  // that is the largest score only for a positive scale
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return DFA_E_SHAPE;
  if (d->doc_bounds && (d->n_docs < 1 || d->n_docs > d->seqlen || d->seqlen > INT32_MAX))
    return DFA_E_SHAPE;
  const int64_t elems16 = d->dtype == DFA_BF16 ? 8 : 4;  // elements per 16 bytes
  const int64_t *all[4] = {d->q_strides, d->k_strides, d->v_strides, d->o_strides};
  for (auto s : all)
    for (int i = 0; i < 3; ++i) {
      if (s[i] < 0) return DFA_E_SHAPE;
      if (s[i] % elems16) return DFA_E_ALIGN;
    }
  return DFA_OK;
}

bool ptr_aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

dfa_status check_block(const dfa_attn_desc *d, const dfa_block &b) {
  const int64_t N = d->seqlen;
  if (b.len_q < 1 || b.len_kv < 1 || b.stride < 1 || b.run < 1) return DFA_E_SHAPE;
  if (b.q_start < 0 || b.kv_start < 0) return DFA_E_SHAPE;
  if (b.run > 1) {
    // whole runs that never overlap; the row tiles (64 rows) must not
    // straddle a run
    if (b.stride < b.run || b.len_q % b.run || b.len_kv % b.run) return DFA_E_SHAPE;
    if (b.run % 64 || ((b.run / 64) & (b.run / 64 - 1))) return DFA_E_UNSUPPORTED;  // 64 * 2^k
  }
  const int64_t rq = (b.len_q - 1) / b.run, rk = (b.len_kv - 1) / b.run;  // last run index
  if (b.q_start > N - 1 || rq > (N - 1 - b.q_start) / b.stride ||
      dfa::piece_pos(b.q_start, b.stride, b.run, b.len_q - 1) > N - 1)
    return DFA_E_SHAPE;
  if (b.kv_start > N - 1 || rk > (N - 1 - b.kv_start) / b.stride ||
      dfa::piece_pos(b.kv_start, b.stride, b.run, b.len_kv - 1) > N - 1)
    return DFA_E_SHAPE;
  // the block's run-level offset (for run = 1 the exact mask rule)
  if (b.diag_offset != floor_div(b.q_start - b.kv_start, b.stride)) return DFA_E_SHAPE;
  return DFA_OK;
}

// The bf16 kernels stream 64-row tiles of a piece into LDS with 32-bit byte
// offsets from the tile's first row: 64 rows (token stride times the row step
// inside a tile) must span less than 2^31 bytes in every streamed tensor.
dfa_status check_tile_span(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n,
                           std::initializer_list<int64_t> token_strides) {
  if (d->dtype != DFA_BF16) return DFA_OK;
  int64_t row_elems = 0;
  for (int64_t s : token_strides) row_elems = std::max(row_elems, s);
  const int64_t limit = (int64_t{1} << 31) / 64;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t step = dfa::piece_row_step(blocks[i].stride, blocks[i].run);
    // 2 * row_elems * step >= limit, without overflow for any int64 inputs
    if (row_elems >= limit || step >= limit || 2 * row_elems >= (limit + step - 1) / step)
      return DFA_E_UNSUPPORTED;
  }
  return DFA_OK;
}

bool any_runs(const dfa_block *blocks, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (blocks[i].run > 1) return true;
  return false;
}

using PieceKey = std::tuple<int64_t, int64_t, int64_t, int64_t>;  // start, len, stride, run

// Distinct pieces must not share rows.  Returns false on overlap; sets
// `full` when the pieces cover every position.
bool pieces_disjoint(const std::vector<PieceKey> &pieces, int64_t N, bool &full) {
  std::vector<uint8_t> seen(static_cast<size_t>(N), 0);
  int64_t covered = 0;
  for (const auto &p : pieces) {
    const int64_t s = std::get<0>(p), len = std::get<1>(p), st = std::get<2>(p), run = std::get<3>(p);
    for (int64_t i = 0; i < len; ++i) {
      uint8_t &x = seen[static_cast<size_t>(dfa::piece_pos(s, st, run, i))];
      if (x) return false;
      x = 1;
    }
    covered += len;
  }
  full = covered == N;
  return true;
}

// ---- query-major plan (forward, dQ) ----
struct QPlan {
  std::vector<QSeg> segs;
  std::vector<KvRef> kv;
  std::vector<Tile> tiles;
  bool full = false;
};

dfa_status plan_q(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n, int tileq,
                  QPlan &out) {
  std::map<PieceKey, std::vector<int64_t>> by_piece;
  std::vector<PieceKey> order;
  for (int64_t i = 0; i < n; ++i) {
    const dfa_block &b = blocks[i];
    PieceKey key{b.q_start, b.len_q, b.stride, b.run};
    auto it = by_piece.find(key);
    if (it == by_piece.end()) {
      order.push_back(key);
      by_piece[key] = {i};
    } else {
      it->second.push_back(i);
    }
  }
  if (!pieces_disjoint(order, d->seqlen, out.full)) return DFA_E_SHAPE;
  struct Cost {
    int64_t cost;
    Tile t;
  };
  std::vector<Cost> costs;
  for (const auto &key : order) {
    auto idx = by_piece[key];
    std::stable_sort(idx.begin(), idx.end(), [&](int64_t a, int64_t b) {
      return std::make_tuple(blocks[a].kv_start, blocks[a].step) <
             std::make_tuple(blocks[b].kv_start, blocks[b].step);
    });
    QSeg s{};
    s.q_start = std::get<0>(key);
    s.len_q = std::get<1>(key);
    s.stride = std::get<2>(key);
    s.run = std::get<3>(key);
    s.part_off = 0;
    s.blk_begin = static_cast<int32_t>(out.kv.size());
    s.blk_count = static_cast<int32_t>(idx.size());
    for (int64_t bi : idx)
      out.kv.push_back(KvRef{blocks[bi].kv_start, blocks[bi].len_kv, blocks[bi].diag_offset});
    const int32_t seg_id = static_cast<int32_t>(out.segs.size());
    out.segs.push_back(s);
    const int64_t nt = ceil_div(s.len_q, tileq);
    for (int64_t t = 0; t < nt; ++t) {
      const int64_t iend = std::min<int64_t>((t + 1) * tileq, s.len_q);
      const int64_t q_last = dfa::piece_pos(s.q_start, s.stride, s.run, iend - 1);
      int64_t c = 0;
      for (int64_t bi : idx) {
        const int64_t hi = dfa::piece_count_le(blocks[bi].kv_start, s.stride, s.run,
                                               blocks[bi].len_kv, q_last);
        c += ceil_div(hi, kCostTileKV);
      }
      costs.push_back(Cost{c, Tile{seg_id, static_cast<int32_t>(t)}});
    }
  }
  std::stable_sort(costs.begin(), costs.end(),
                   [](const Cost &a, const Cost &b) { return a.cost > b.cost; });
  out.tiles.reserve(costs.size());
  for (const auto &c : costs) out.tiles.push_back(c.t);
  return DFA_OK;
}

// The fused query-major walks (forward, dQ) interleave a piece's blocks in
// groups of kIlvTiles key tiles when every block is a near-triangle over
// single-token rows (|diag_offset| <= 1, run = 1: token striping), so that
// the query tiles of one head, whose costs differ, read the same key tiles
// at about the same time (from L2; the HBM traffic saved raises the clock);
// the kernels then keep one block per lane (at most 64 per piece, 32-bit
// lengths).  Other schedules keep the walk block after block: with stripe
// blocks of 64-128 tokens the position-ordered walk already shares L2 and
// the interleave's cursor measured slower.
bool interleavable(const dfa_block *blocks, int64_t n, const QPlan &qp) {
  for (int64_t i = 0; i < n; ++i)
    if (blocks[i].diag_offset < -1 || blocks[i].diag_offset > 1 || blocks[i].len_kv > INT32_MAX ||
        blocks[i].run != 1)
      return false;
  for (const auto &s : qp.segs)
    if (s.blk_count > 64) return false;
  return true;
}

// ---- key-major plan (dK, dV) ----
struct KvPlan {
  std::vector<KvSeg> segs;
  std::vector<QRef> q;
  std::vector<Tile> tiles;
  bool full = false;
};

dfa_status plan_kv(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n, int tilek,
                   KvPlan &out) {
  std::map<PieceKey, std::vector<int64_t>> by_piece;
  std::vector<PieceKey> order;
  for (int64_t i = 0; i < n; ++i) {
    const dfa_block &b = blocks[i];
    PieceKey key{b.kv_start, b.len_kv, b.stride, b.run};
    auto it = by_piece.find(key);
    if (it == by_piece.end()) {
      order.push_back(key);
      by_piece[key] = {i};
    } else {
      it->second.push_back(i);
    }
  }
  if (!pieces_disjoint(order, d->seqlen, out.full)) return DFA_E_SHAPE;
  struct Cost {
    int64_t cost;
    Tile t;
  };
  std::vector<Cost> costs;
  for (const auto &key : order) {
    auto idx = by_piece[key];
    std::stable_sort(idx.begin(), idx.end(), [&](int64_t a, int64_t b) {
      return std::make_tuple(blocks[a].q_start, blocks[a].step) <
             std::make_tuple(blocks[b].q_start, blocks[b].step);
    });
    KvSeg s{};
    s.kv_start = std::get<0>(key);
    s.len_kv = std::get<1>(key);
    s.stride = std::get<2>(key);
    s.run = std::get<3>(key);
    s.blk_begin = static_cast<int32_t>(out.q.size());
    s.blk_count = static_cast<int32_t>(idx.size());
    for (int64_t bi : idx)
      out.q.push_back(QRef{blocks[bi].q_start, blocks[bi].len_q, blocks[bi].diag_offset});
    const int32_t seg_id = static_cast<int32_t>(out.segs.size());
    out.segs.push_back(s);
    const int64_t nt = ceil_div(s.len_kv, tilek);
    for (int64_t t = 0; t < nt; ++t) {
      const int64_t gk0 = dfa::piece_pos(s.kv_start, s.stride, s.run, t * tilek);
      int64_t c = 0;
      for (int64_t bi : idx) {
        // query rows at or after the tile's first key see at least one key
        const int64_t lo = dfa::piece_count_le(blocks[bi].q_start, s.stride, s.run,
                                               blocks[bi].len_q, gk0 - 1);
        if (lo < blocks[bi].len_q) c += ceil_div(blocks[bi].len_q - lo, kCostTileKV);
      }
      costs.push_back(Cost{c, Tile{seg_id, static_cast<int32_t>(t)}});
    }
  }
  std::stable_sort(costs.begin(), costs.end(),
                   [](const Cost &a, const Cost &b) { return a.cost > b.cost; });
  out.tiles.reserve(costs.size());
  for (const auto &c : costs) out.tiles.push_back(c.t);
  return DFA_OK;
}

// ---- device table packing ----
struct Packer {
  std::vector<char> bytes;
  template <class T>
  size_t add(const std::vector<T> &v) {
    const size_t off = bytes.size();
    const size_t sz = align_up(v.size() * sizeof(T));
    bytes.resize(off + std::max<size_t>(sz, kAlign), 0);
    if (!v.empty()) std::memcpy(bytes.data() + off, v.data(), v.size() * sizeof(T));
    return off;
  }
};

dfa::Geom make_geom(const dfa_attn_desc *d) {
  dfa::Geom g{};
  for (int i = 0; i < 3; ++i) {
    g.qs[i] = d->q_strides[i];
    g.ks[i] = d->k_strides[i];
    g.vs[i] = d->v_strides[i];
    g.os[i] = d->o_strides[i];
  }
  g.seqlen = d->seqlen;
  g.batch = d->batch;
  g.hq = d->heads_q;
  g.hkv = d->heads_kv;
  g.group = d->heads_q / d->heads_kv;
  g.scale = d->softmax_scale;
  g.scale_log2 = d->softmax_scale * 1.4426950408889634f;
  g.docs = d->doc_bounds;
  g.n_docs = d->doc_bounds ? static_cast<int32_t>(d->n_docs) : 0;
  return g;
}

int fwd_tile(const dfa_attn_desc *d) { return d->dtype == DFA_BF16 ? dfa::kFwdTileQ : dfa::kF32TileQ; }
int dq_tile(const dfa_attn_desc *d) { return d->dtype == DFA_BF16 ? dfa::kDqTileQ : dfa::kF32TileQ; }
int kv_tile(const dfa_attn_desc *d) { return d->dtype == DFA_BF16 ? dfa::kBwdTileKV : dfa::kF32TileKV; }

dfa_status hip_status(hipError_t e) { return e == hipSuccess ? DFA_OK : DFA_E_HIP; }

dfa_status check_blocks(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n) {
  if (n < 0) return DFA_E_SHAPE;
  if (n > 0 && !blocks) return DFA_E_NULL;
  if (n > 0x3fffffff) return DFA_E_SHAPE;
  for (int64_t i = 0; i < n; ++i) {
    const dfa_status st = check_block(d, blocks[i]);
    if (st != DFA_OK) return st;
  }
  return DFA_OK;
}

// Stepwise forward: rounds of blocks whose query pieces are distinct, in
// ring-step order.  Each round's launch merges every block's partial into
// the accumulator rows of its queries (distinct rows: no two blocks of a
// round write the same row).
struct StepPlan {
  std::vector<QSeg> segs;   // one per block
  std::vector<KvRef> kv;    // one per block
  std::vector<Tile> tiles;  // per round, contiguous
  struct Round {
    int32_t tile_begin, tile_count;
  };
  std::vector<Round> rounds;
};

void plan_steps(const dfa_block *blocks, int64_t n, int tileq, StepPlan &sp) {
  std::vector<int64_t> idx(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](int64_t a, int64_t b) {
    return std::make_tuple(blocks[a].step, blocks[a].rank, blocks[a].kv_start) <
           std::make_tuple(blocks[b].step, blocks[b].rank, blocks[b].kv_start);
  });
  size_t pos = 0;
  while (pos < idx.size()) {
    const int64_t step = blocks[idx[pos]].step;
    size_t end = pos;
    while (end < idx.size() && blocks[idx[end]].step == step) ++end;
    std::vector<std::vector<int64_t>> rounds;
    std::vector<std::vector<PieceKey>> used;
    for (size_t p = pos; p < end; ++p) {
      const dfa_block &b = blocks[idx[p]];
      PieceKey key{b.q_start, b.len_q, b.stride, b.run};
      size_t r = 0;
      while (r < rounds.size() &&
             std::find(used[r].begin(), used[r].end(), key) != used[r].end())
        ++r;
      if (r == rounds.size()) {
        rounds.emplace_back();
        used.emplace_back();
      }
      rounds[r].push_back(idx[p]);
      used[r].push_back(key);
    }
    for (const auto &rb : rounds) {
      StepPlan::Round R{static_cast<int32_t>(sp.tiles.size()), 0};
      for (int64_t bi : rb) {
        const dfa_block &b = blocks[bi];
        QSeg s{};
        s.q_start = b.q_start;
        s.len_q = b.len_q;
        s.stride = b.stride;
        s.run = b.run;
        s.blk_begin = static_cast<int32_t>(sp.kv.size());
        s.blk_count = 1;
        sp.kv.push_back(KvRef{b.kv_start, b.len_kv, b.diag_offset});
        const int32_t sid = static_cast<int32_t>(sp.segs.size());
        sp.segs.push_back(s);
        const int64_t nt = ceil_div(b.len_q, tileq);
        for (int64_t t = 0; t < nt; ++t) sp.tiles.push_back(Tile{sid, static_cast<int32_t>(t)});
      }
      R.tile_count = static_cast<int32_t>(sp.tiles.size()) - R.tile_begin;
      sp.rounds.push_back(R);
    }
    pos = end;
  }
}

// Ring-faithful slots: the blocks of one (rank, step) slot in rounds of
// distinct query pieces, slots in (step, rank) order.  Same tables as
// plan_steps (one QSeg and KvRef per block), so the same workspace size.
void plan_slots(const dfa_block *blocks, int64_t n, int tileq, int P, StepPlan &sp,
                std::vector<int32_t> &round_slot) {
  std::vector<int64_t> idx(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](int64_t a, int64_t b) {
    return std::make_tuple(blocks[a].step, blocks[a].rank, blocks[a].kv_start) <
           std::make_tuple(blocks[b].step, blocks[b].rank, blocks[b].kv_start);
  });
  size_t pos = 0;
  while (pos < idx.size()) {
    const dfa_block &b0 = blocks[idx[pos]];
    size_t end = pos;
    while (end < idx.size() && blocks[idx[end]].step == b0.step && blocks[idx[end]].rank == b0.rank)
      ++end;
    std::vector<std::vector<int64_t>> rounds;
    std::vector<std::vector<PieceKey>> used;
    for (size_t p = pos; p < end; ++p) {
      const dfa_block &b = blocks[idx[p]];
      PieceKey key{b.q_start, b.len_q, b.stride, b.run};
      size_t r = 0;
      while (r < rounds.size() && std::find(used[r].begin(), used[r].end(), key) != used[r].end()) ++r;
      if (r == rounds.size()) {
        rounds.emplace_back();
        used.emplace_back();
      }
      rounds[r].push_back(idx[p]);
      used[r].push_back(key);
    }
    for (const auto &rb : rounds) {
      StepPlan::Round R{static_cast<int32_t>(sp.tiles.size()), 0};
      for (int64_t bi : rb) {
        const dfa_block &b = blocks[bi];
        QSeg s{};
        s.q_start = b.q_start;
        s.len_q = b.len_q;
        s.stride = b.stride;
        s.run = b.run;
        s.blk_begin = static_cast<int32_t>(sp.kv.size());
        s.blk_count = 1;
        sp.kv.push_back(KvRef{b.kv_start, b.len_kv, b.diag_offset});
        const int32_t sid = static_cast<int32_t>(sp.segs.size());
        sp.segs.push_back(s);
        const int64_t nt = ceil_div(b.len_q, tileq);
        for (int64_t t = 0; t < nt; ++t) sp.tiles.push_back(Tile{sid, static_cast<int32_t>(t)});
      }
      R.tile_count = static_cast<int32_t>(sp.tiles.size()) - R.tile_begin;
      sp.rounds.push_back(R);
      round_slot.push_back(static_cast<int32_t>(b0.step * P + b0.rank));
    }
    pos = end;
  }
}

// Workspace layouts (offsets in bytes).
struct FusedLayout {
  size_t segs, kv, tiles, total;
};
struct StepLayout {
  size_t segs, kv, tiles, acc_o, acc_lse, total;
};
struct BwdLayout {
  size_t qsegs, qkv, qtiles, kvsegs, kvq, kvtiles, dd, lse2, total;
};

template <class T>
size_t vbytes(const std::vector<T> &v) {
  return std::max<size_t>(align_up(v.size() * sizeof(T)), kAlign);
}

FusedLayout fused_layout(const QPlan &p) {
  FusedLayout L{};
  L.segs = 0;
  L.kv = L.segs + vbytes(p.segs);
  L.tiles = L.kv + vbytes(p.kv);
  L.total = L.tiles + vbytes(p.tiles);
  return L;
}

StepLayout step_layout(const dfa_attn_desc *d, const StepPlan &p) {
  StepLayout L{};
  const size_t hd = static_cast<size_t>(d->head_dim);
  const size_t rows = static_cast<size_t>(d->batch) * d->heads_q * d->seqlen;
  L.segs = 0;
  L.kv = L.segs + vbytes(p.segs);
  L.tiles = L.kv + vbytes(p.kv);
  L.acc_o = L.tiles + vbytes(p.tiles);
  L.acc_lse = L.acc_o + align_up(rows * hd * sizeof(float));
  L.total = L.acc_lse + align_up(rows * sizeof(float));
  return L;
}

BwdLayout bwd_layout(const dfa_attn_desc *d, const QPlan &qp, const KvPlan &kp) {
  BwdLayout L{};
  const size_t rows = static_cast<size_t>(d->batch) * d->heads_q * d->seqlen;
  L.qsegs = 0;
  L.qkv = L.qsegs + vbytes(qp.segs);
  L.qtiles = L.qkv + vbytes(qp.kv);
  L.kvsegs = L.qtiles + vbytes(qp.tiles);
  L.kvq = L.kvsegs + vbytes(kp.segs);
  L.kvtiles = L.kvq + vbytes(kp.q);
  L.dd = L.kvtiles + vbytes(kp.tiles);
  L.lse2 = L.dd + align_up(rows * sizeof(float));
  L.total = L.lse2 + align_up(rows * sizeof(float));
  return L;
}

template <class T>
void put(std::vector<char> &buf, size_t off, const std::vector<T> &v) {
  if (!v.empty()) std::memcpy(buf.data() + off, v.data(), v.size() * sizeof(T));
}

dfa_status upload(void *ws, const std::vector<char> &host, size_t bytes, hipStream_t s) {
  if (bytes == 0) return DFA_OK;
  return hip_status(hipMemcpyAsync(ws, host.data(), bytes, hipMemcpyHostToDevice, s));
}

dfa_status check_ws(void *ws, size_t have, size_t need) {
  if (need == 0) return DFA_OK;
  if (!ws) return DFA_E_WORKSPACE;
  if (have < need) return DFA_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return DFA_E_ALIGN;
  return DFA_OK;
}

// Stepwise forward over a planned list of rounds: accumulators set to the
// merge identity, each round's partials merged into the accumulator rows in
// the partial kernel's epilogue, then O and LSE written from them.  With
// events, events[slot] is recorded before the first round of each slot in
// slot order (empty slots included) and events[n_slots] at the end.
dfa_status run_stepwise(const dfa_attn_desc *d, const StepPlan &sp, const int32_t *round_slot,
                        int32_t n_slots, void *const *events, dfa::FwdArgs a, void *o, float *lse,
                        void *workspace, size_t ws_bytes, hipStream_t s) {
  const StepLayout L = step_layout(d, sp);
  dfa_status st = check_ws(workspace, ws_bytes, L.total);
  if (st != DFA_OK) return st;
  const int hd = d->head_dim;
  char *ws = static_cast<char *>(workspace);
  std::vector<char> host(L.acc_o, 0);
  put(host, L.segs, sp.segs);
  put(host, L.kv, sp.kv);
  put(host, L.tiles, sp.tiles);
  st = upload(workspace, host, L.acc_o, s);
  if (st != DFA_OK) return st;
  float *acc_o = reinterpret_cast<float *>(ws + L.acc_o);
  float *acc_lse = reinterpret_cast<float *>(ws + L.acc_lse);
  const int64_t BH = static_cast<int64_t>(d->batch) * d->heads_q;
  const int64_t rows = BH * d->seqlen;
  st = hip_status(dfa::launch_acc_init(acc_o, acc_lse, rows, hd, s));
  if (st != DFA_OK) return st;
  auto launch = [&](const dfa::FwdArgs &args, int64_t grid) {
    return d->dtype == DFA_BF16 ? dfa::launch_fwd_bf16(args, hd, grid, s)
                                : dfa::launch_fwd_f32(args, hd, grid, s);
  };
  bool mark_ok = true;
  auto mark = [&](int32_t slot) {
    if (hipEventRecord(static_cast<hipEvent_t>(events[slot]), s) != hipSuccess) mark_ok = false;
  };
  // per round: every block's partial, merged into its query rows (mode 2)
  a.o = acc_o;
  a.lse = acc_lse;
  a.out_mode = 2;
  a.segs = reinterpret_cast<const QSeg *>(ws + L.segs);
  a.kv = reinterpret_cast<const KvRef *>(ws + L.kv);
  int32_t next_slot = 0;
  for (size_t r = 0; r < sp.rounds.size(); ++r) {
    if (events)
      while (next_slot <= round_slot[r]) mark(next_slot++);
    const auto &R = sp.rounds[r];
    a.tiles = reinterpret_cast<const Tile *>(ws + L.tiles) + R.tile_begin;
    a.n_tiles = R.tile_count;
    st = hip_status(launch(a, static_cast<int64_t>(R.tile_count) * BH));
    if (st != DFA_OK) return st;
  }
  if (events)
    while (next_slot <= n_slots) mark(next_slot++);  // empty trailing slots, then the end
  st = hip_status(dfa::launch_finalize(acc_o, acc_lse, o, d->o_strides, d->dtype, lse, d->batch,
                                       d->heads_q, d->seqlen, hd, s));
  if (st != DFA_OK) return st;
  return mark_ok ? DFA_OK : DFA_E_HIP;
}

}  // namespace

extern "C" dfa_status dfa_rope(int32_t dtype, int32_t batch, int64_t seqlen, int32_t heads, int32_t head_dim,
                    const int64_t *x_strides, const void *x, const int64_t *y_strides, void *y,
                    int64_t pos_offset, double base, int32_t inverse, void *stream) {
  if (!x_strides || !y_strides) return DFA_E_NULL;
  if (dtype != DFA_BF16 && dtype != DFA_F32) return DFA_E_UNSUPPORTED;
  if (head_dim < 2 || head_dim > 512 || head_dim % 2) return DFA_E_UNSUPPORTED;
  if (batch < 1 || heads < 1 || seqlen < 0 || pos_offset < 0) return DFA_E_SHAPE;
  if (!(base > 0.0) || !std::isfinite(base) || (inverse != 0 && inverse != 1)) return DFA_E_SHAPE;
  if (seqlen == 0) return DFA_OK;
  if (!x || !y) return DFA_E_NULL;
  const uintptr_t pair = dtype == DFA_BF16 ? 4 : 8;
  if ((reinterpret_cast<uintptr_t>(x) % pair) || (reinterpret_cast<uintptr_t>(y) % pair))
    return DFA_E_ALIGN;
  bool same = true;
  for (int i = 0; i < 3; ++i) {
    if (x_strides[i] < 0 || y_strides[i] < 0) return DFA_E_SHAPE;
    if ((x_strides[i] % 2) || (y_strides[i] % 2)) return DFA_E_ALIGN;
    same = same && x_strides[i] == y_strides[i];
  }
  if (x == y && !same) return DFA_E_SHAPE;
  dfa::RopeArgs a{};
  a.x = x;
  a.y = y;
  for (int i = 0; i < 3; ++i) {
    a.xs[i] = x_strides[i];
    a.ys[i] = y_strides[i];
  }
  a.seqlen = seqlen;
  a.pos_offset = pos_offset;
  a.base = base;
  a.batch = batch;
  a.heads = heads;
  a.head_dim = head_dim;
  a.inverse = inverse;
  return hip_status(dfa::launch_rope(a, dtype == DFA_BF16, static_cast<hipStream_t>(stream)));
}

const char *dfa_status_string(dfa_status s) {
  switch (s) {
    case DFA_OK: return "ok";
    case DFA_E_NULL: return "a required pointer is NULL";
    case DFA_E_SHAPE: return "inconsistent sizes or block list";
    case DFA_E_UNSUPPORTED: return "unsupported head_dim, dtype, mode or schedule kind";
    case DFA_E_ALIGN: return "pointer or stride violates 16-byte row alignment";
    case DFA_E_CAPACITY: return "output array too small";
    case DFA_E_WORKSPACE: return "workspace missing or too small";
    case DFA_E_HIP: return "HIP runtime error or kernel launch failure";
    default: return "unknown status";
  }
}

extern "C" dfa_status dfa_workspace_size(const dfa_attn_desc *d, const dfa_block *blocks,
                                         int64_t n_blocks, int32_t op, size_t *bytes) {
  if (!bytes) return DFA_E_NULL;
  dfa_status st = check_desc(d);
  if (st != DFA_OK) return st;
  st = check_blocks(d, blocks, n_blocks);
  if (st != DFA_OK) return st;
  if (op == DFA_OP_FWD_FUSED) {
    QPlan p;
    st = plan_q(d, blocks, n_blocks, fwd_tile(d), p);
    if (st != DFA_OK) return st;
    *bytes = fused_layout(p).total;
  } else if (op == DFA_OP_FWD_STEPWISE) {
    QPlan p;  // validates piece disjointness
    st = plan_q(d, blocks, n_blocks, fwd_tile(d), p);
    if (st != DFA_OK) return st;
    StepPlan sp;
    plan_steps(blocks, n_blocks, fwd_tile(d), sp);
    *bytes = step_layout(d, sp).total;
  } else if (op == DFA_OP_BWD) {
    QPlan qp;
    KvPlan kp;
    st = plan_q(d, blocks, n_blocks, dq_tile(d), qp);
    if (st != DFA_OK) return st;
    st = plan_kv(d, blocks, n_blocks, kv_tile(d), kp);
    if (st != DFA_OK) return st;
    *bytes = bwd_layout(d, qp, kp).total;
  } else {
    return DFA_E_UNSUPPORTED;
  }
  return DFA_OK;
}

extern "C" dfa_status dfa_attn_block_fwd(const dfa_attn_desc *d, const dfa_block *blk,
                                         const void *q, const void *k, const void *v,
                                         float *o_part, float *lse_part, void *stream) {
  dfa_status st = check_desc(d);
  if (st != DFA_OK) return st;
  if (!blk || !q || !k || !v || !o_part || !lse_part) return DFA_E_NULL;
  st = check_block(d, *blk);
  if (st != DFA_OK) return st;
  if (!ptr_aligned(q) || !ptr_aligned(k) || !ptr_aligned(v) || !ptr_aligned(o_part))
    return DFA_E_ALIGN;
  st = check_tile_span(d, blk, 1, {d->k_strides[1], d->v_strides[1]});
  if (st != DFA_OK) return st;
  dfa::FwdArgs a{};
  a.g = make_geom(d);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o_part;
  a.lse = lse_part;
  a.out_mode = 1;
  a.runs = blk->run > 1;
  a.seg0 = QSeg{blk->q_start, blk->len_q, blk->stride, blk->run, 0, 0, 1};
  a.kv0 = KvRef{blk->kv_start, blk->len_kv, blk->diag_offset};
  const int tq = fwd_tile(d);
  const int64_t grid = ceil_div(blk->len_q, tq) * d->batch * d->heads_q;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->dtype == DFA_BF16) return hip_status(dfa::launch_fwd_bf16(a, d->head_dim, grid, s));
  return hip_status(dfa::launch_fwd_f32(a, d->head_dim, grid, s));
}

extern "C" dfa_status dfa_lse_merge(int64_t n_rows, int32_t head_dim, float *o_acc,
                                    float *lse_acc, const float *o_part, const float *lse_part,
                                    void *stream) {
  if (head_dim != 64 && head_dim != 128) return DFA_E_UNSUPPORTED;
  if (n_rows < 0) return DFA_E_SHAPE;
  if (n_rows == 0) return DFA_OK;
  if (!o_acc || !lse_acc || !o_part || !lse_part) return DFA_E_NULL;
  if (!ptr_aligned(o_acc) || !ptr_aligned(o_part)) return DFA_E_ALIGN;
  return hip_status(dfa::launch_merge_rows(o_acc, lse_acc, o_part, lse_part, n_rows, head_dim,
                                           static_cast<hipStream_t>(stream)));
}

extern "C" dfa_status dfa_attn_fwd(const dfa_attn_desc *d, const dfa_block *blocks,
                                   int64_t n_blocks, int32_t mode, const void *q, const void *k,
                                   const void *v, void *o, float *lse, void *workspace,
                                   size_t ws_bytes, void *stream) {
  dfa_status st = check_desc(d);
  if (st != DFA_OK) return st;
  if (!q || !k || !v || !o || !lse) return DFA_E_NULL;
  if (!ptr_aligned(q) || !ptr_aligned(k) || !ptr_aligned(v) || !ptr_aligned(o)) return DFA_E_ALIGN;
  if (mode != DFA_FWD_FUSED && mode != DFA_FWD_STEPWISE) return DFA_E_UNSUPPORTED;
  st = check_blocks(d, blocks, n_blocks);
  if (st != DFA_OK) return st;
  st = check_tile_span(d, blocks, n_blocks, {d->k_strides[1], d->v_strides[1]});
  if (st != DFA_OK) return st;
  QPlan qp;
  st = plan_q(d, blocks, n_blocks, fwd_tile(d), qp);
  if (st != DFA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int hd = d->head_dim;
  dfa::FwdArgs a{};
  a.runs = any_runs(blocks, n_blocks);
  a.g = make_geom(d);
  a.q = q;
  a.k = k;
  a.v = v;
  auto launch = [&](const dfa::FwdArgs &args, int64_t grid) {
    return d->dtype == DFA_BF16 ? dfa::launch_fwd_bf16(args, hd, grid, s)
                                : dfa::launch_fwd_f32(args, hd, grid, s);
  };
  const int64_t BH = static_cast<int64_t>(d->batch) * d->heads_q;

  if (mode == DFA_FWD_FUSED) {
    const FusedLayout L = fused_layout(qp);
    st = check_ws(workspace, ws_bytes, L.total);
    if (st != DFA_OK) return st;
    if (!qp.full) {
      st = hip_status(dfa::launch_zero_rows(o, d->o_strides, d->dtype, d->batch, d->seqlen,
                                            d->heads_q, hd, lse, s));
      if (st != DFA_OK) return st;
    }
    if (qp.tiles.empty()) return DFA_OK;
    std::vector<char> host(L.total, 0);
    put(host, L.segs, qp.segs);
    put(host, L.kv, qp.kv);
    put(host, L.tiles, qp.tiles);
    st = upload(workspace, host, L.tiles + qp.tiles.size() * sizeof(Tile), s);
    if (st != DFA_OK) return st;
    char *ws = static_cast<char *>(workspace);
    a.o = o;
    a.lse = lse;
    a.out_mode = 0;
    a.interleave = interleavable(blocks, n_blocks, qp);
    a.segs = reinterpret_cast<const QSeg *>(ws + L.segs);
    a.kv = reinterpret_cast<const KvRef *>(ws + L.kv);
    a.tiles = reinterpret_cast<const Tile *>(ws + L.tiles);
    a.n_tiles = static_cast<int32_t>(qp.tiles.size());
    return hip_status(launch(a, static_cast<int64_t>(qp.tiles.size()) * BH));
  }

  // stepwise
  StepPlan sp;
  plan_steps(blocks, n_blocks, fwd_tile(d), sp);
  return run_stepwise(d, sp, nullptr, 0, nullptr, a, o, lse, workspace, ws_bytes, s);
}

extern "C" dfa_status dfa_attn_fwd_slots(const dfa_attn_desc *d, const dfa_block *blocks,
                                         int64_t n_blocks, const void *q, const void *k,
                                         const void *v, void *o, float *lse, void *workspace,
                                         size_t ws_bytes, const dfa_slot_marks *marks,
                                         void *stream) {
  dfa_status st = check_desc(d);
  if (st != DFA_OK) return st;
  if (!q || !k || !v || !o || !lse || !marks || !marks->events) return DFA_E_NULL;
  if (!ptr_aligned(q) || !ptr_aligned(k) || !ptr_aligned(v) || !ptr_aligned(o)) return DFA_E_ALIGN;
  const int32_t P = marks->n_ranks;
  if (P < 1 || P > 46340) return DFA_E_SHAPE;  // P * P + 1 events fit an int32
  st = check_blocks(d, blocks, n_blocks);
  if (st != DFA_OK) return st;
  for (int64_t i = 0; i < n_blocks; ++i)
    if (blocks[i].rank < 0 || blocks[i].rank >= P || blocks[i].step < 0 || blocks[i].step >= P)
      return DFA_E_SHAPE;
  st = check_tile_span(d, blocks, n_blocks, {d->k_strides[1], d->v_strides[1]});
  if (st != DFA_OK) return st;
  QPlan qp;  // validates piece disjointness
  st = plan_q(d, blocks, n_blocks, fwd_tile(d), qp);
  if (st != DFA_OK) return st;
  StepPlan sp;
  std::vector<int32_t> round_slot;
  plan_slots(blocks, n_blocks, fwd_tile(d), P, sp, round_slot);
  dfa::FwdArgs a{};
  a.runs = any_runs(blocks, n_blocks);
  a.g = make_geom(d);
  a.q = q;
  a.k = k;
  a.v = v;
  return run_stepwise(d, sp, round_slot.data(), P * P, marks->events, a, o, lse, workspace,
                      ws_bytes, static_cast<hipStream_t>(stream));
}

extern "C" dfa_status dfa_attn_bwd(const dfa_attn_desc *d, const dfa_block *blocks,
                                   int64_t n_blocks, const void *q, const void *k, const void *v,
                                   const void *o, const void *d_o, const float *lse, void *dq,
                                   void *dk, void *dv, void *workspace, size_t ws_bytes,
                                   void *stream) {
  return dfa_attn_bwd_ex(d, blocks, n_blocks, q, k, v, o, d_o, lse, dq, dk, dv, workspace,
                         ws_bytes, nullptr, stream);
}

extern "C" dfa_status dfa_attn_bwd_ex(const dfa_attn_desc *d, const dfa_block *blocks,
                                      int64_t n_blocks, const void *q, const void *k,
                                      const void *v, const void *o, const void *d_o,
                                      const float *lse, void *dq, void *dk, void *dv,
                                      void *workspace, size_t ws_bytes,
                                      const dfa_kernel_marks *marks, void *stream) {
  dfa_status st = check_desc(d);
  if (st != DFA_OK) return st;
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return DFA_E_NULL;
  for (const void *p : {q, k, v, o, d_o, static_cast<const void *>(dq),
                        static_cast<const void *>(dk), static_cast<const void *>(dv)})
    if (!ptr_aligned(p)) return DFA_E_ALIGN;
  st = check_blocks(d, blocks, n_blocks);
  if (st != DFA_OK) return st;
  // the dQ kernel streams K and V, the dK/dV kernel Q and dO (strides of o)
  st = check_tile_span(d, blocks, n_blocks,
                       {d->q_strides[1], d->o_strides[1], d->k_strides[1], d->v_strides[1]});
  if (st != DFA_OK) return st;
  QPlan qp;
  KvPlan kp;
  st = plan_q(d, blocks, n_blocks, dq_tile(d), qp);
  if (st != DFA_OK) return st;
  st = plan_kv(d, blocks, n_blocks, kv_tile(d), kp);
  if (st != DFA_OK) return st;
  const BwdLayout L = bwd_layout(d, qp, kp);
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != DFA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int hd = d->head_dim;
  if (!qp.full) {
    st = hip_status(dfa::launch_zero_rows(dq, d->q_strides, d->dtype, d->batch, d->seqlen,
                                          d->heads_q, hd, nullptr, s));
    if (st != DFA_OK) return st;
  }
  if (!kp.full) {
    st = hip_status(dfa::launch_zero_rows(dk, d->k_strides, d->dtype, d->batch, d->seqlen,
                                          d->heads_kv, hd, nullptr, s));
    if (st != DFA_OK) return st;
    st = hip_status(dfa::launch_zero_rows(dv, d->v_strides, d->dtype, d->batch, d->seqlen,
                                          d->heads_kv, hd, nullptr, s));
    if (st != DFA_OK) return st;
  }
  if (n_blocks == 0) return DFA_OK;
  std::vector<char> host(L.dd, 0);
  put(host, L.qsegs, qp.segs);
  put(host, L.qkv, qp.kv);
  put(host, L.qtiles, qp.tiles);
  put(host, L.kvsegs, kp.segs);
  put(host, L.kvq, kp.q);
  put(host, L.kvtiles, kp.tiles);
  st = upload(workspace, host, L.dd, s);
  if (st != DFA_OK) return st;
  char *ws = static_cast<char *>(workspace);
  dfa::BwdArgs a{};
  a.runs = any_runs(blocks, n_blocks);
  a.g = make_geom(d);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = d_o;
  a.lse = lse;
  a.dd = reinterpret_cast<float *>(ws + L.dd);
  a.lse2 = reinterpret_cast<float *>(ws + L.lse2);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.qsegs = reinterpret_cast<const QSeg *>(ws + L.qsegs);
  a.qkv = reinterpret_cast<const KvRef *>(ws + L.qkv);
  a.qtiles = reinterpret_cast<const Tile *>(ws + L.qtiles);
  a.n_qtiles = static_cast<int32_t>(qp.tiles.size());
  a.interleave = interleavable(blocks, n_blocks, qp);
  a.kvsegs = reinterpret_cast<const KvSeg *>(ws + L.kvsegs);
  a.kvq = reinterpret_cast<const QRef *>(ws + L.kvq);
  a.kvtiles = reinterpret_cast<const Tile *>(ws + L.kvtiles);
  a.n_kvtiles = static_cast<int32_t>(kp.tiles.size());
  bool mark_ok = true;
  auto mark = [&](void *ev) {
    if (ev && hipEventRecord(static_cast<hipEvent_t>(ev), s) != hipSuccess) mark_ok = false;
  };
  if (marks) mark(marks->pre_begin);
  st = hip_status(dfa::launch_bwd_pre(a, d->dtype, hd, s));
  if (st != DFA_OK) return st;
  const int64_t BHq = static_cast<int64_t>(d->batch) * d->heads_q;
  const int64_t BHkv = static_cast<int64_t>(d->batch) * d->heads_kv;
  const bool bf = d->dtype == DFA_BF16;
  if (marks) mark(marks->dq_begin);
  st = hip_status(bf ? dfa::launch_bwd_dq_bf16(a, hd, a.n_qtiles * BHq, s)
                     : dfa::launch_bwd_dq_f32(a, hd, a.n_qtiles * BHq, s));
  if (st != DFA_OK) return st;
  // one kernel computes dK and dV: both marks precede it
  if (marks) mark(marks->dk_begin);
  if (marks) mark(marks->dv_begin);
  st = hip_status(bf ? dfa::launch_bwd_dkdv_bf16(a, hd, a.n_kvtiles * BHkv, s)
                     : dfa::launch_bwd_dkdv_f32(a, hd, a.n_kvtiles * BHkv, s));
  if (st != DFA_OK) return st;
  if (marks) mark(marks->end);
  return mark_ok ? DFA_OK : DFA_E_HIP;
}
