// dfa_internal.h -- device-side work tables and kernel launchers shared by the
// host runtime (api.cpp) and the HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfa {

// Global position of local row i of a piece: runs of `run` consecutive
// tokens, consecutive runs `stride` apart (run = 1: start + i*stride).
__host__ __device__ inline int64_t piece_pos(int64_t start, int64_t stride, int64_t run, int64_t i) {
  return run == 1 ? start + i * stride : start + (i / run) * stride + i % run;
}

// Number of rows of a piece of `len` rows whose global position is <= x
// (positions increase with the row index).
__host__ __device__ inline int64_t piece_count_le(int64_t start, int64_t stride, int64_t run,
                                                  int64_t len, int64_t x) {
  if (x < start) return 0;
  const int64_t d = x - start, u = d / stride, off = d - u * stride;
  const int64_t n = u * run + (off + 1 < run ? off + 1 : run);
  return n < len ? n : len;
}

// Distance between consecutive rows inside a 64-row tile of a piece (tiles
// never straddle a run: run is 1 or a multiple of 64).
__host__ __device__ inline int64_t piece_row_step(int64_t stride, int64_t run) {
  return run == 1 ? stride : 1;
}

__host__ __device__ inline int64_t floor_div64(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

// One distinct query piece (rows as in piece_pos).  Its blocks (key pieces
// in position order) are kv[blk_begin, blk_begin + blk_count); the key
// pieces share the query piece's stride and run.
struct QSeg {
  int64_t q_start, len_q, stride, run;
  int64_t part_off;  // single-block mode: float offset of this piece's partial buffer
  int32_t blk_begin, blk_count;
};

// One key piece seen by a query piece, with the block's diagonal offset:
// local key j is visible to local query i iff j <= i + diag_offset.
struct KvRef {
  int64_t kv_start, len_kv, diag_offset;
};

// One distinct key piece (backward, key-major walk) and the query pieces
// that read it: q[blk_begin, blk_begin + blk_count).
struct KvSeg {
  int64_t kv_start, len_kv, stride, run;
  int32_t blk_begin, blk_count;
};

struct QRef {
  int64_t q_start, len_q, diag_offset;
};

// A unit of work: tile `tile` of piece `seg`.
struct Tile {
  int32_t seg, tile;
};

// Geometry of one attention problem as the kernels see it.
struct Geom {
  int64_t qs[3], ks[3], vs[3], os[3];  // element strides (batch, token, head)
  int64_t seqlen;
  int32_t batch, hq, hkv, group;  // group = hq / hkv
  float scale_log2;               // softmax scale * log2(e)
  float scale;                    // softmax scale
  const int32_t *docs;            // packed documents: n_docs + 1 ascending bounds, or null
  int32_t n_docs;                 // 0: one document (plain causal)
};

// Packed documents: [lo, hi) = the document holding global position p, by
// binary search over the n + 1 cumulative bounds (document t holds
// [b[t], b[t+1])).  Every load stays inside b[0..n] whatever b holds.
__device__ inline void doc_range(const int32_t *b, int n, int64_t p, int64_t &lo, int64_t &hi) {
  int l = 0, r = n;
  while (r - l > 1) {
    const int m = (l + r) >> 1;
    if (b[m] <= p)
      l = m;
    else
      r = m;
  }
  lo = b[l];
  hi = b[l + 1];
}

// Forward over query pieces (fused walk, stepwise rounds, single block).
struct FwdArgs {
  Geom g;
  const void *q, *k, *v;
  void *o;        // out_mode 0: dtype O (strides g.os); 1: fp32 partial buffer base;
                  // 2: fp32 accumulator [B][Hq][N][hd]
  float *lse;     // out_mode 0 and 2: [B][Hq][N]; 1: partial LSE base (float offset part_off/hd)
  const QSeg *segs;
  const KvRef *kv;
  const Tile *tiles;
  int32_t n_tiles;
  int32_t out_mode;  // 0: final O/LSE at global rows; 1: fp32 partials per piece;
                     // 2: partials merged into the accumulator rows (rows of one
                     // launch are distinct)
  int32_t runs;      // some piece is made of runs (run > 1)
  int32_t interleave;  // fused walk in groups of kIlvTiles key tiles per block, block after
                       // block, group after group (every block a near-triangle:
                       // |diag_offset| <= 1, len_kv < 2^31, at most 64 blocks per piece)
  QSeg seg0;         // used when segs == nullptr (one block, no table)
  KvRef kv0;
};

// Backward arguments.
struct BwdArgs {
  Geom g;
  const void *q, *k, *v, *o, *dout;
  const float *lse;  // [B][Hq][N]
  float *dd;         // -D = -rowsum(dO*O): [B][Hq][N]
  float *lse2;       // LSE * log2(e): [B][Hq][N]
  void *dq, *dk, *dv;
  const QSeg *qsegs;
  const KvRef *qkv;    // key pieces per query piece (dq walk)
  const Tile *qtiles;
  int32_t n_qtiles;
  const KvSeg *kvsegs;
  const QRef *kvq;     // query pieces per key piece (dk/dv walk)
  const Tile *kvtiles;
  int32_t n_kvtiles;
  int32_t runs;  // some piece is made of runs (run > 1)
  int32_t interleave;  // dQ walk as FwdArgs::interleave
};


// Tile shapes (rows per work item).
constexpr int kFwdWaves = 8;                // bf16 forward: waves per workgroup
constexpr int kFwdTileQ = 32 * kFwdWaves;   // bf16 forward: query rows per workgroup
constexpr int kFwdStages = 4;               // bf16 forward: K/V tiles resident in LDS
constexpr int kBwdWaves = 8;                // bf16 dq, dk, dv: waves per workgroup
constexpr int kBwdStages = 4;               // bf16 dq: K/V tiles resident in LDS
constexpr int kDqTileQ = 32 * kBwdWaves;    // bf16 dq: query rows per workgroup
constexpr int kBwdTileKV = 32 * kBwdWaves;  // bf16 dk/dv: key rows per workgroup
constexpr int kKvStages = 2;                // bf16 dk/dv: Q/dO tiles resident in LDS
constexpr int kIlvTiles = 4;      // interleaved walks: key tiles per block and group (2^k)
constexpr int kF32TileQ = 64;    // fp32 kernels: rows per workgroup
constexpr int kF32TileKV = 64;

// Rotary position embedding over [batch][seqlen][heads][head_dim] (element
// strides xs / ys for batch, token, head; head_dim contiguous).
struct RopeArgs {
  const void *x;
  void *y;
  int64_t xs[3], ys[3];
  int64_t seqlen, pos_offset;
  double base;
  int32_t batch, heads, head_dim, inverse;
};

// ---- launchers (return hipError_t of the launch) ----
hipError_t launch_fwd_bf16(const FwdArgs &a, int hd, int64_t grid, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs &a, int hd, int64_t grid, hipStream_t s);
hipError_t launch_bwd_pre(const BwdArgs &a, int dtype, int hd, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const BwdArgs &a, int hd, int64_t grid, hipStream_t s);
// grid: work items (tiles x batch-heads); the bf16 forward and dQ launchers
// round it up to whole groups of 8 (xcd_item); the dK/dV kernel writes both
// gradients
hipError_t launch_bwd_dkdv_bf16(const BwdArgs &a, int hd, int64_t grid, hipStream_t s);
hipError_t launch_bwd_dq_f32(const BwdArgs &a, int hd, int64_t grid, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const BwdArgs &a, int hd, int64_t grid, hipStream_t s);
// head_dim even, 2..512
hipError_t launch_rope(const RopeArgs &a, int dtype_bf16, hipStream_t s);

// Fill rows of a [B][N][H][hd] tensor (strides) with zero; if lse != nullptr
// also set lse [B][H][N] to -inf.
hipError_t launch_zero_rows(void *x, const int64_t strides[3], int dtype, int batch, int64_t n,
                            int heads, int hd, float *lse, hipStream_t s);
// acc <- identity (O = 0, LSE = -inf) for [rows][hd] fp32 + [rows].
hipError_t launch_acc_init(float *o_acc, float *lse_acc, int64_t rows, int hd, hipStream_t s);
// Plain contiguous merge of n_rows rows (public dfa_lse_merge).
hipError_t launch_merge_rows(float *o_acc, float *lse_acc, const float *o_part,
                             const float *lse_part, int64_t n_rows, int hd, hipStream_t s);
// Accumulator [B][Hq][N][hd] fp32 -> O (dtype, strides) and lse [B][Hq][N].
hipError_t launch_finalize(const float *o_acc, const float *lse_acc, void *o,
                           const int64_t os[3], int dtype, float *lse, int batch, int hq,
                           int64_t n, int hd, hipStream_t s);

}  // namespace dfa
