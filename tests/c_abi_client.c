/* A plain C99 client of libdfa's host-side calls, built by
 * tests/test_c_client.py: it proves the boundary is usable from C (header
 * compiles as C, symbols link, structs and enums match) without a GPU.
 * Output, one record per line:
 *   S <kind> <N> <P> <stripe> <n_blocks> <total_pairs> <busy_slots> <bubble> <eta>
 *   B <11 int64 fields of each block>              (after each S line)
 *   R <rank_pairs[0..P-1]> | <step_max[0..P-1]>
 *   E <what> <status> <n_out>                      (error paths)
 *   W <op> <bytes>                                 (workspace sizes)
 *   T <status> <text>                              (status strings)
 */
#include <stdio.h>
#include <stdlib.h>

#include "dfa.h"

static int show(int32_t kind, int64_t n, int32_t p, int64_t stripe) {
  int64_t count = 0;
  dfa_status st = stripe > 1 ? dfa_schedule_build_striped_blocks(n, p, stripe, NULL, 0, &count)
                             : dfa_schedule_build(kind, n, p, NULL, 0, &count);
  if (st != DFA_OK) return st;
  dfa_block *b = (dfa_block *)calloc((size_t)(count > 0 ? count : 1), sizeof(dfa_block));
  int64_t got = 0;
  st = stripe > 1 ? dfa_schedule_build_striped_blocks(n, p, stripe, b, count, &got)
                  : dfa_schedule_build(kind, n, p, b, count, &got);
  if (st != DFA_OK || got != count) return st != DFA_OK ? st : -100;
  int64_t *rp = (int64_t *)calloc((size_t)p, sizeof(int64_t));
  int64_t *sm = (int64_t *)calloc((size_t)p, sizeof(int64_t));
  dfa_balance bal;
  st = dfa_schedule_balance(b, got, p, rp, sm, &bal);
  if (st != DFA_OK) return st;
  printf("S %d %lld %d %lld %lld %lld %lld %.17g %.17g\n", kind, (long long)n, p, (long long)stripe,
         (long long)got, (long long)bal.total_pairs, (long long)bal.busy_slots, bal.bubble, bal.eta_blocks);
  for (int64_t i = 0; i < got; ++i)
    printf("B %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld\n", (long long)b[i].rank,
           (long long)b[i].step, (long long)b[i].kv_rank, (long long)b[i].q_start,
           (long long)b[i].kv_start, (long long)b[i].len_q, (long long)b[i].len_kv,
           (long long)b[i].stride, (long long)b[i].diag_offset, (long long)b[i].pairs,
           (long long)b[i].run);
  printf("R");
  for (int r = 0; r < p; ++r) printf(" %lld", (long long)rp[r]);
  printf(" |");
  for (int s = 0; s < p; ++s) printf(" %lld", (long long)sm[s]);
  printf("\n");
  /* workspace sizes of a bf16 problem over this block list (host only) */
  if (stripe == 1 && n % 64 == 0) {
    dfa_attn_desc d = {0};
    d.dtype = DFA_BF16;
    d.batch = 1;
    d.heads_q = 4;
    d.heads_kv = 2;
    d.head_dim = 128;
    d.softmax_scale = 0.08838834764831845f;
    d.seqlen = n;
    int64_t qs[3] = {n * 4 * 128, 4 * 128, 128}, ks[3] = {n * 2 * 128, 2 * 128, 128};
    for (int i = 0; i < 3; ++i) {
      d.q_strides[i] = qs[i];
      d.o_strides[i] = qs[i];
      d.k_strides[i] = ks[i];
      d.v_strides[i] = ks[i];
    }
    const int32_t ops[3] = {DFA_OP_FWD_FUSED, DFA_OP_FWD_STEPWISE, DFA_OP_BWD};
    for (int o = 0; o < 3; ++o) {
      size_t bytes = 0;
      st = dfa_workspace_size(&d, b, got, ops[o], &bytes);
      printf("W %d %d %zu\n", ops[o], st, bytes);
    }
  }
  free(b);
  free(rp);
  free(sm);
  return DFA_OK;
}

int main(void) {
  const int32_t kinds[3] = {DFA_SCHED_RING, DFA_SCHED_BALANCED, DFA_SCHED_STRIPED};
  const int32_t ps[4] = {1, 2, 4, 8};
  for (int k = 0; k < 3; ++k)
    for (int i = 0; i < 4; ++i) {
      dfa_status st = show(kinds[k], 1024, ps[i], 1);
      if (st != DFA_OK) {
        printf("FAIL %d %d %d\n", kinds[k], ps[i], st);
        return 1;
      }
    }
  if (show(DFA_SCHED_STRIPED, 2048, 4, 64) != DFA_OK || show(DFA_SCHED_STRIPED, 2048, 2, 128) != DFA_OK) {
    printf("FAIL stripe blocks\n");
    return 1;
  }
  /* error paths: a length the schedule cannot split, too small an output */
  /* (each call before its printf: argument evaluation order is unspecified) */
  int64_t n_out = -1;
  dfa_status st = dfa_schedule_build(DFA_SCHED_BALANCED, 1000, 8, NULL, 0, &n_out);
  printf("E shape %d %lld\n", st, (long long)n_out);
  dfa_block one;
  n_out = -1;
  st = dfa_schedule_build(DFA_SCHED_RING, 1024, 4, &one, 1, &n_out);
  printf("E capacity %d %lld\n", st, (long long)n_out);
  printf("E null %d\n", dfa_schedule_build(DFA_SCHED_RING, 1024, 4, NULL, 0, NULL));
  const dfa_status codes[8] = {DFA_OK, DFA_E_NULL, DFA_E_SHAPE, DFA_E_UNSUPPORTED,
                               DFA_E_ALIGN, DFA_E_CAPACITY, DFA_E_WORKSPACE, DFA_E_HIP};
  for (int i = 0; i < 8; ++i) printf("T %d %s\n", codes[i], dfa_status_string(codes[i]));
  return 0;
}
