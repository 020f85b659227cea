// schedule.cpp -- closed-form enumeration of the virtual-rank ring schedules
// and their balance accounting.  Pure host code.
//
// Chunk ownership:
//   RING      rank r owns [r*C, (r+1)*C), C = N/P (DistFlashAttn Guide, "The
//             Causal Imbalance Crisis").
//   BALANCED  2P chunks of C = N/(2P); rank r owns chunks r and 2P-1-r
//             (DistFlashAttn Guide, "Core Innovation 1", folded chunk
//             assignment).
//   STRIPED   rank r owns positions r, r+P, r+2P, ... (Striped Attention
//             Guide, "Mathematical Formulation of Token Striping").
//   STRIPED with stripe blocks of B tokens: rank r owns the runs
//             [(u*P + r)*B, (u*P + r + 1)*B), u = 0, 1, ... (the guide's
//             block-striped variant).
// At ring step s rank r holds the key/value shard of rank (r - s) mod P
// (Striped Attention Guide, "Workload Balance Theorem").
//
// Per block the visible-pair count follows from the chunk geometry:
//   a key chunk strictly before the query chunk   -> C*C pairs (full block)
//   the same chunk                                 -> C*(C+1)/2 (diagonal)
//   a key chunk after the query chunk              -> 0 (block omitted)
// and for striped shards, query m of rank r (position m*P+r) sees key n of
// rank j (position n*P+j) iff n <= m when j <= r, iff n <= m-1 when j > r:
// C*(C+1)/2 or C*(C-1)/2 pairs with diagonal offset 0 or -1 (the shifted
// diagonal of the striped mask, Striped Attention Guide, "Algorithmic
// Mechanics" 1, step 2).  With stripe blocks (R = C/B runs per rank), query
// (run u, offset e) of rank r sees every key of the runs v < u of rank j, and
// of run u all B keys when j < r, the first e+1 when j = r, none when j > r:
// B*B*R*(R-1)/2 + R*(B*B, B*(B+1)/2 or 0) pairs.
#include <cstring>
#include <vector>

#include "dfa.h"

namespace {

struct Emitter {
  dfa_block *out;
  int64_t capacity;
  int64_t n = 0;
  void emit(int64_t rank, int64_t step, int64_t kv_rank, int64_t q_start, int64_t kv_start,
            int64_t len, int64_t stride, int64_t diag, int64_t pairs, int64_t run = 1) {
    if (out && n < capacity) {
      dfa_block &b = out[n];
      b.rank = rank;
      b.step = step;
      b.kv_rank = kv_rank;
      b.q_start = q_start;
      b.kv_start = kv_start;
      b.len_q = len;
      b.len_kv = len;
      b.stride = stride;
      b.diag_offset = diag;
      b.pairs = pairs;
      b.run = run;
    }
    ++n;
  }
};

int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

}  // namespace

extern "C" dfa_status dfa_schedule_build(int32_t kind, int64_t seqlen, int32_t n_ranks,
                                         dfa_block *out, int64_t capacity, int64_t *n_out) {
  if (!n_out) return DFA_E_NULL;
  if (seqlen < 1 || n_ranks < 1 || capacity < 0) return DFA_E_SHAPE;
  const int64_t P = n_ranks, N = seqlen;
  Emitter em{out, capacity};
  switch (kind) {
    case DFA_SCHED_RING: {
      if (N % P) return DFA_E_SHAPE;
      const int64_t C = N / P;
      for (int64_t r = 0; r < P; ++r)
        for (int64_t s = 0; s < P; ++s) {
          const int64_t j = ((r - s) % P + P) % P;
          if (j > r) continue;
          em.emit(r, s, j, r * C, j * C, C, 1, (r - j) * C, j == r ? C * (C + 1) / 2 : C * C);
        }
      break;
    }
    case DFA_SCHED_BALANCED: {
      if (N % (2 * P)) return DFA_E_SHAPE;
      const int64_t C = N / (2 * P);
      for (int64_t r = 0; r < P; ++r) {
        const int64_t qc[2] = {r, 2 * P - 1 - r};  // ascending: r < P <= 2P-1-r
        for (int64_t s = 0; s < P; ++s) {
          const int64_t j = ((r - s) % P + P) % P;
          const int64_t kc[2] = {j, 2 * P - 1 - j};
          for (int a = 0; a < 2; ++a)
            for (int c = 0; c < 2; ++c) {
              if (kc[c] > qc[a]) continue;
              const bool diag = kc[c] == qc[a];
              em.emit(r, s, j, qc[a] * C, kc[c] * C, C, 1, (qc[a] - kc[c]) * C,
                      diag ? C * (C + 1) / 2 : C * C);
            }
        }
      }
      break;
    }
    case DFA_SCHED_STRIPED: {
      if (N % P) return DFA_E_SHAPE;
      const int64_t C = N / P;
      for (int64_t r = 0; r < P; ++r)
        for (int64_t s = 0; s < P; ++s) {
          const int64_t j = ((r - s) % P + P) % P;
          const int64_t pairs = j <= r ? C * (C + 1) / 2 : C * (C - 1) / 2;
          if (pairs == 0) continue;
          em.emit(r, s, j, r, j, C, P, floor_div(r - j, P), pairs);
        }
      break;
    }
    default:
      return DFA_E_UNSUPPORTED;
  }
  *n_out = em.n;
  if (out && em.n > capacity) return DFA_E_CAPACITY;
  return DFA_OK;
}

extern "C" dfa_status dfa_schedule_build_striped_blocks(int64_t seqlen, int32_t n_ranks,
                                                        int64_t stripe, dfa_block *out,
                                                        int64_t capacity, int64_t *n_out) {
  if (!n_out) return DFA_E_NULL;
  if (seqlen < 1 || n_ranks < 1 || stripe < 1 || capacity < 0) return DFA_E_SHAPE;
  const int64_t P = n_ranks, N = seqlen, B = stripe;
  if (N % (P * B)) return DFA_E_SHAPE;
  const int64_t C = N / P, R = C / B;
  Emitter em{out, capacity};
  for (int64_t r = 0; r < P; ++r)
    for (int64_t s = 0; s < P; ++s) {
      const int64_t j = ((r - s) % P + P) % P;
      const int64_t same_run = j < r ? B * B : (j == r ? B * (B + 1) / 2 : 0);
      const int64_t pairs = B * B * (R * (R - 1) / 2) + R * same_run;
      if (pairs == 0) continue;
      em.emit(r, s, j, r * B, j * B, C, P * B, floor_div(r - j, P), pairs, B);
    }
  *n_out = em.n;
  if (out && em.n > capacity) return DFA_E_CAPACITY;
  return DFA_OK;
}

extern "C" dfa_status dfa_schedule_balance(const dfa_block *blocks, int64_t n_blocks,
                                           int32_t n_ranks, int64_t *rank_pairs,
                                           int64_t *step_max, dfa_balance *out) {
  if (n_blocks < 0 || n_ranks < 1) return DFA_E_SHAPE;
  if (n_blocks > 0 && !blocks) return DFA_E_NULL;
  const int64_t P = n_ranks;
  std::vector<int64_t> load(static_cast<size_t>(P * P), 0);  // [rank][step]
  for (int64_t i = 0; i < n_blocks; ++i) {
    const dfa_block &b = blocks[i];
    if (b.rank < 0 || b.rank >= P || b.step < 0 || b.step >= P || b.pairs < 0) return DFA_E_SHAPE;
    load[b.rank * P + b.step] += b.pairs;
  }
  int64_t total = 0, sum_max = 0, busy = 0;
  for (int64_t r = 0; r < P; ++r) {
    int64_t t = 0;
    for (int64_t s = 0; s < P; ++s) {
      t += load[r * P + s];
      busy += load[r * P + s] > 0;
    }
    if (rank_pairs) rank_pairs[r] = t;
    total += t;
  }
  for (int64_t s = 0; s < P; ++s) {
    int64_t m = 0;
    for (int64_t r = 0; r < P; ++r) m = load[r * P + s] > m ? load[r * P + s] : m;
    if (step_max) step_max[s] = m;
    sum_max += m;
  }
  if (out) {
    out->total_pairs = total;
    out->busy_slots = busy;
    out->bubble = sum_max ? 1.0 - static_cast<double>(total) / (static_cast<double>(P) * sum_max) : 0.0;
    out->eta_blocks = static_cast<double>(busy) / static_cast<double>(P * P);
  }
  return DFA_OK;
}
