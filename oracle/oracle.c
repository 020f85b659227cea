/*
 * oracle.c -- fp64 CPU reference for blockwise exact causal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the "oracle": a plain, slow and
 * deliberately unoptimised implementation of what the GPU library computes.
 * Only the test-suite, the package smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no code, header or constant with the HIP
 * library and must never be used as a fallback for it.
 *
 * Everything is double precision.  Callers pass the exact stored input values
 * (bf16 or fp32 values widened to double), so a comparison measures kernel
 * error, not input rounding.
 *
 * Tensor layout for every function: q and dO are [B][N][Hq][d], k and v are
 * [B][N][Hkv][d], contiguous.  Query head h reads key/value head
 * h / (Hq/Hkv) (contiguous groups; the pages only name grouped-query
 * attention, FlashAttention glossary page, "variants" list).
 *
 * Sources (the pages' text):
 *  - causal score matrix: a key at position j is visible to the query at
 *    position i iff j <= i, score q_i.k_j / sqrt(d)  (Striped Attention Guide,
 *    "The Fatal Flaw: Causal Workload Imbalance", the masked score equation;
 *    DistFlashAttn Guide, "The Causal Imbalance Crisis", tau <= t).
 *  - softmax with row max m, row sum l and output sum_j e^{S-m} v_j / l
 *    (Striped Attention Guide, "Algorithmic Mechanics" 1, first equation).
 *  - visibility inside a block is decided on global positions: masked iff
 *    GlobalPos(query) < GlobalPos(key)  (same section, step 2).
 *  - the merged blockwise result equals monolithic attention (same page,
 *    "Algorithmic Mechanics" opening paragraph; FlashAttention glossary page,
 *    "exact same attention matrix").
 *  - gradients are recomputed from the saved output and row statistics
 *    (FlashAttention glossary page, first two paragraphs).  The pages give no
 *    backward formulas; the functions below are the plain vector-Jacobian
 *    product of softmax attention written out element by element.
 *
 *  - packed documents: when several documents are concatenated into one
 *    sequence, a query attends only to keys of its own document (Striped
 *    Attention Guide, "Production Deployment and Best Practices", item 3,
 *    "Document Packing and Boundary Alignment").  Every function below takes
 *    an optional doc[N] (document id of each position; NULL = one document)
 *    and applies that rule on top of the causal one.
 *
 * Natural logarithms throughout: LSE_i = m_i + ln(l_i).  A row with no visible
 * key has O = 0 and LSE = -inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EARG -1
#define ORC_ENOMEM -2

static const double *vec(const double *x, int64_t N, int64_t H, int64_t d,
                         int64_t b, int64_t t, int64_t h) {
  return x + (((b * N) + t) * H + h) * d;
}

static double dot(const double *a, const double *b, int64_t d) {
  double s = 0.0;
  for (int64_t c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/* the key at position j is visible to the query at position i: not after it,
 * and (with packed documents) in the same document */
static int visible(int64_t i, int64_t j, const int64_t *doc) {
  return j <= i && (doc == NULL || doc[j] == doc[i]);
}

static int dims_ok(int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d) {
  return B >= 1 && N >= 0 && Hq >= 1 && Hkv >= 1 && d >= 1 && Hq % Hkv == 0;
}

/*
 * Attention of one query vector against the keys listed in keys[0..nk).
 * Two passes over the keys: the row maximum first, then the exponentials.
 * s_buf must hold nk doubles.  Writes o[0..d) and returns LSE (ln).
 */
static double attend_one(const double *qi, const double *kbase, const double *vbase,
                         int64_t key_stride, const int64_t *keys, int64_t nk, int64_t d,
                         double scale, double *s_buf, double *o) {
  for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
  if (nk == 0) return -INFINITY;
  double m = -INFINITY;
  for (int64_t t = 0; t < nk; ++t) {
    s_buf[t] = scale * dot(qi, kbase + keys[t] * key_stride, d);
    if (s_buf[t] > m) m = s_buf[t];
  }
  double l = 0.0;
  for (int64_t t = 0; t < nk; ++t) {
    double p = exp(s_buf[t] - m);
    l += p;
    const double *vj = vbase + keys[t] * key_stride;
    for (int64_t c = 0; c < d; ++c) o[c] += p * vj[c];
  }
  for (int64_t c = 0; c < d; ++c) o[c] /= l;
  return m + log(l);
}

/*
 * O1 -- full causal attention for selected query rows and heads.
 *   rows[r]  : global position of output row r (query at that position)
 *   heads[h] : query head of output head slot h
 *   o   : [B][n_heads][n_rows][d]     lse : [B][n_heads][n_rows]
 * Visible keys of the query at position i: every j in [0, i] (of i's
 * document when doc != NULL).
 */
int orc_attn_rows(int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                  const double *q, const double *k, const double *v,
                  int64_t n_rows, const int64_t *rows, int64_t n_heads, const int64_t *heads,
                  double *o, double *lse, const int64_t *doc) {
  if (!dims_ok(B, N, Hq, Hkv, d)) return ORC_EARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return ORC_EARG;
  for (int64_t h = 0; h < n_heads; ++h)
    if (heads[h] < 0 || heads[h] >= Hq) return ORC_EARG;
  int64_t group = Hq / Hkv;
  int err = ORC_OK;
  int64_t total = B * n_heads * n_rows;
#pragma omp parallel
  {
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    if (!s_buf || !keys) {
#pragma omp atomic write
      err = ORC_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t w = 0; w < total; ++w) {
        int64_t b = w / (n_heads * n_rows);
        int64_t hs = (w / n_rows) % n_heads;
        int64_t r = w % n_rows;
        int64_t h = heads[hs], hk = h / group, i = rows[r], nk = 0;
        for (int64_t j = 0; j <= i; ++j)
          if (visible(i, j, doc)) keys[nk++] = j;
        const double *qi = vec(q, N, Hq, d, b, i, h);
        const double *kb = vec(k, N, Hkv, d, b, 0, hk);
        const double *vb = vec(v, N, Hkv, d, b, 0, hk);
        double *oi = o + ((b * n_heads + hs) * n_rows + r) * d;
        lse[(b * n_heads + hs) * n_rows + r] =
            attend_one(qi, kb, vb, Hkv * d, keys, nk, d, scale, s_buf, oi);
      }
    }
    free(s_buf);
    free(keys);
  }
  return err;
}

/* position of local row i of a shard: runs of `run` consecutive tokens,
 * consecutive runs `stride` apart (run 1: start + i*stride; stripe blocks of
 * B tokens over P ranks: run B, stride P*B -- Striped Attention Guide,
 * "Mathematical Formulation of Token Striping", block-striped set) */
static int64_t piece_position(int64_t start, int64_t stride, int64_t run, int64_t i) {
  return start + (i / run) * stride + i % run;
}

/*
 * O2 -- partial attention of one (query-shard, key-shard) block.
 * Query row i of the block sits at global position
 * piece_position(q_start, stride, run, i), key row j at
 * piece_position(kv_start, stride, run, j).  Key j is visible to query i iff
 * its global position is not after the query's (GlobalPos rule) and, with
 * doc != NULL, both lie in the same document.  Each row is normalised over
 * the block's visible keys only.
 *   o_part : [B][Hq][len_q][d]     lse_part : [B][Hq][len_q]
 */

int orc_block_partial(int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                      const double *q, const double *k, const double *v,
                      int64_t q_start, int64_t kv_start, int64_t len_q, int64_t len_kv,
                      int64_t stride, int64_t run, double *o_part, double *lse_part,
                      const int64_t *doc) {
  if (!dims_ok(B, N, Hq, Hkv, d) || stride < 1 || run < 1 || len_q < 0 || len_kv < 0)
    return ORC_EARG;
  if (run > 1 && stride < run) return ORC_EARG;
  if (q_start < 0 || kv_start < 0) return ORC_EARG;
  if (len_q > 0 && piece_position(q_start, stride, run, len_q - 1) >= N) return ORC_EARG;
  if (len_kv > 0 && piece_position(kv_start, stride, run, len_kv - 1) >= N) return ORC_EARG;
  int64_t group = Hq / Hkv;
  int err = ORC_OK;
  int64_t total = B * Hq * len_q;
#pragma omp parallel
  {
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)(len_kv > 0 ? len_kv : 1));
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(len_kv > 0 ? len_kv : 1));
    if (!s_buf || !keys) {
#pragma omp atomic write
      err = ORC_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t w = 0; w < total; ++w) {
        int64_t b = w / (Hq * len_q), h = (w / len_q) % Hq, i = w % len_q;
        int64_t qpos = piece_position(q_start, stride, run, i), nk = 0;
        for (int64_t j = 0; j < len_kv; ++j) {
          int64_t kpos = piece_position(kv_start, stride, run, j);
          if (visible(qpos, kpos, doc)) keys[nk++] = kpos;
        }
        const double *qi = vec(q, N, Hq, d, b, qpos, h);
        const double *kb = vec(k, N, Hkv, d, b, 0, h / group);
        const double *vb = vec(v, N, Hkv, d, b, 0, h / group);
        double *oi = o_part + ((b * Hq + h) * len_q + i) * d;
        lse_part[(b * Hq + h) * len_q + i] =
            attend_one(qi, kb, vb, Hkv * d, keys, nk, d, scale, s_buf, oi);
      }
    }
    free(s_buf);
    free(keys);
  }
  return err;
}

/*
 * O3 -- merge normalised partials of the same rows.
 *   o_parts : [n_parts][n_rows][d]   lse_parts : [n_parts][n_rows]
 *   o       : [n_rows][d]            lse       : [n_rows]
 * With M = max_b LSE_b: LSE = M + ln sum_b e^{LSE_b - M} and
 * O = sum_b e^{LSE_b - LSE} O_b.  This is the pages' alpha/beta rescaling
 * (Striped Attention Guide, "Algorithmic Mechanics" 1, steps 4-7) with each
 * partial already divided by its own row sum.  All partials at -inf give
 * O = 0, LSE = -inf.
 */
int orc_merge(int64_t n_parts, int64_t n_rows, int64_t d,
              const double *o_parts, const double *lse_parts, double *o, double *lse) {
  if (n_parts < 0 || n_rows < 0 || d < 1) return ORC_EARG;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    double M = -INFINITY;
    for (int64_t p = 0; p < n_parts; ++p)
      if (lse_parts[p * n_rows + r] > M) M = lse_parts[p * n_rows + r];
    double *orow = o + r * d;
    for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
    if (M == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int64_t p = 0; p < n_parts; ++p) sum += exp(lse_parts[p * n_rows + r] - M);
    double L = M + log(sum);
    for (int64_t p = 0; p < n_parts; ++p) {
      double wgt = exp(lse_parts[p * n_rows + r] - L);
      const double *op = o_parts + (p * n_rows + r) * d;
      for (int64_t c = 0; c < d; ++c) orow[c] += wgt * op[c];
    }
    lse[r] = L;
  }
  return ORC_OK;
}

/*
 * O5, row half -- per query row of the loss  L = sum_{i in R} dO_i . O_i :
 *   P_ij  = e^{S_ij - LSE_i}           on visible pairs (j <= i, same document), 0 elsewhere
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   rows[r] : global position of row r       heads[h] : query head
 *   lse, dd : [B][n_heads][n_rows]           dq : [B][n_heads][n_rows][d]
 * Optional (NULL to skip) -- rounding-error magnitudes used by tests to set
 * tolerances, not results of the method:
 *   aa     : A_i = sum_c |dO_ic O_ic|, the size of D_i's terms   [B][n_heads][n_rows]
 *   dq_abs : scale * sum_j P_ij (|dP_ij - D_i| + A_i) |k_jc|     [B][n_heads][n_rows][d]
 */
int orc_grad_rows(int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                  const double *q, const double *k, const double *v, const double *dout,
                  int64_t n_rows, const int64_t *rows, int64_t n_heads, const int64_t *heads,
                  double *lse, double *dd, double *dq, double *aa, double *dq_abs,
                  const int64_t *doc) {
  if (!dims_ok(B, N, Hq, Hkv, d)) return ORC_EARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return ORC_EARG;
  for (int64_t h = 0; h < n_heads; ++h)
    if (heads[h] < 0 || heads[h] >= Hq) return ORC_EARG;
  int64_t group = Hq / Hkv;
  int err = ORC_OK;
  int64_t total = B * n_heads * n_rows;
#pragma omp parallel
  {
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *dp_buf = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!s_buf || !dp_buf) {
#pragma omp atomic write
      err = ORC_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t w = 0; w < total; ++w) {
        int64_t b = w / (n_heads * n_rows), hs = (w / n_rows) % n_heads, r = w % n_rows;
        int64_t h = heads[hs], hk = h / group, i = rows[r];
        const double *qi = vec(q, N, Hq, d, b, i, h);
        const double *doi = vec(dout, N, Hq, d, b, i, h);
        int64_t idx = (b * n_heads + hs) * n_rows + r;
        double *dqi = dq + idx * d;
        /* scores and the row statistics */
        double m = -INFINITY;
        for (int64_t j = 0; j <= i; ++j) {
          /* a key of another document gets score -inf: P_ij = 0, dS_ij = 0 */
          s_buf[j] = visible(i, j, doc) ? scale * dot(qi, vec(k, N, Hkv, d, b, j, hk), d) : -INFINITY;
          if (s_buf[j] > m) m = s_buf[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j <= i; ++j) l += exp(s_buf[j] - m);
        double L = m + log(l);
        /* probabilities, dP and D */
        double D = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
          s_buf[j] = exp(s_buf[j] - L); /* now P_ij */
          dp_buf[j] = dot(doi, vec(v, N, Hkv, d, b, j, hk), d);
          D += s_buf[j] * dp_buf[j];
        }
        for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
          double ds = s_buf[j] * (dp_buf[j] - D);
          const double *kj = vec(k, N, Hkv, d, b, j, hk);
          for (int64_t c = 0; c < d; ++c) dqi[c] += scale * ds * kj[c];
        }
        lse[idx] = L;
        dd[idx] = D;
        if (aa || dq_abs) {
          /* A_i = sum_c |dO_ic O_ic| and the absolute term sums of dQ_i */
          double A = 0.0;
          for (int64_t c = 0; c < d; ++c) {
            double oc = 0.0;
            for (int64_t j = 0; j <= i; ++j) oc += s_buf[j] * vec(v, N, Hkv, d, b, j, hk)[c];
            A += fabs(doi[c] * oc);
          }
          if (aa) aa[idx] = A;
          if (dq_abs) {
            double *ai = dq_abs + idx * d;
            for (int64_t c = 0; c < d; ++c) ai[c] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
              double w = s_buf[j] * (fabs(dp_buf[j] - D) + A);
              const double *kj = vec(k, N, Hkv, d, b, j, hk);
              for (int64_t c = 0; c < d; ++c) ai[c] += scale * w * fabs(kj[c]);
            }
          }
        }
      }
    }
    free(s_buf);
    free(dp_buf);
  }
  return err;
}

/*
 * O5, column half -- per key row j and key/value head hk:
 *   dK_j = scale * sum_{h in group(hk)} sum_{i in R, j visible to i} dS_ij q_i
 *   dV_j =         sum_{h in group(hk)} sum_{i in R, j visible to i} P_ij dO_i
 * with P and dS rebuilt from the row statistics LSE_i and D_i that
 * orc_grad_rows produced for the same row set R.
 *   rows[r]          : global positions of R
 *   lse, dd          : [B][Hq][n_rows]   (every query head)
 *   keys[t]          : global position of output key row t
 *   kv_heads[h]      : key/value head of output head slot h
 *   dk, dv           : [B][n_kv_heads][n_keys][d]
 * Optional (all three or none): aa = A_i from orc_grad_rows ([B][Hq][n_rows])
 * and the magnitudes
 *   dk_abs = scale * sum P_ij (|dP_ij - D_i| + A_i) |q_ic|,  dv_abs = sum P_ij |dO_ic|.
 */
int orc_grad_cols(int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t d, double scale,
                  const double *q, const double *k, const double *v, const double *dout,
                  int64_t n_rows, const int64_t *rows, const double *lse, const double *dd,
                  int64_t n_keys, const int64_t *keys, int64_t n_kv_heads, const int64_t *kv_heads,
                  double *dk, double *dv, const double *aa, double *dk_abs, double *dv_abs,
                  const int64_t *doc) {
  if (!dims_ok(B, N, Hq, Hkv, d)) return ORC_EARG;
  if ((dk_abs || dv_abs) && !(dk_abs && dv_abs && aa)) return ORC_EARG;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return ORC_EARG;
  for (int64_t t = 0; t < n_keys; ++t)
    if (keys[t] < 0 || keys[t] >= N) return ORC_EARG;
  for (int64_t h = 0; h < n_kv_heads; ++h)
    if (kv_heads[h] < 0 || kv_heads[h] >= Hkv) return ORC_EARG;
  int64_t group = Hq / Hkv;
  int64_t total = B * n_kv_heads * n_keys;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t w = 0; w < total; ++w) {
    int64_t b = w / (n_kv_heads * n_keys), hs = (w / n_keys) % n_kv_heads, t = w % n_keys;
    int64_t hk = kv_heads[hs], j = keys[t];
    const double *kj = vec(k, N, Hkv, d, b, j, hk);
    const double *vj = vec(v, N, Hkv, d, b, j, hk);
    double *dkj = dk + ((b * n_kv_heads + hs) * n_keys + t) * d;
    double *dvj = dv + ((b * n_kv_heads + hs) * n_keys + t) * d;
    for (int64_t c = 0; c < d; ++c) dkj[c] = dvj[c] = 0.0;
    double *dka = dk_abs ? dk_abs + ((b * n_kv_heads + hs) * n_keys + t) * d : NULL;
    double *dva = dv_abs ? dv_abs + ((b * n_kv_heads + hs) * n_keys + t) * d : NULL;
    if (dka)
      for (int64_t c = 0; c < d; ++c) dka[c] = dva[c] = 0.0;
    for (int64_t g = 0; g < group; ++g) {
      int64_t h = hk * group + g;
      for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = rows[r];
        if (!visible(i, j, doc)) continue;
        const double *qi = vec(q, N, Hq, d, b, i, h);
        const double *doi = vec(dout, N, Hq, d, b, i, h);
        int64_t idx = (b * Hq + h) * n_rows + r;
        double p = exp(scale * dot(qi, kj, d) - lse[idx]);
        double dpd = dot(doi, vj, d) - dd[idx]; /* dP_ij - D_i */
        double ds = p * dpd;
        for (int64_t c = 0; c < d; ++c) {
          dkj[c] += scale * ds * qi[c];
          dvj[c] += p * doi[c];
        }
        if (dka) {
          double w = p * (fabs(dpd) + aa[idx]);
          for (int64_t c = 0; c < d; ++c) {
            dka[c] += scale * w * fabs(qi[c]);
            dva[c] += p * fabs(doi[c]);
          }
        }
      }
    }
  }
  return ORC_OK;
}

/*
 * O6 -- rotary position embedding at absolute positions (Striped Attention
 * Guide, "Preserving Rotary Position Embeddings (RoPE)": each token vector is
 * rotated by its absolute sequence index, q_rot = R(Theta, i) q).  The pages
 * name the rotation but not its parameters; this is the RoFormer form with
 * interleaved pairs: pair c = (x[2c], x[2c+1]) turns by the angle
 * pos * base^(-2c/d), pos = pos_offset + token index.  inverse != 0 turns by
 * minus that angle (the transpose, used for gradients).
 *   x, y : [B][N][H][d] contiguous (y may equal x)
 */
int orc_rope(int64_t B, int64_t N, int64_t H, int64_t d, const double *x, double *y,
             int64_t pos_offset, double base, int inverse) {
  if (B < 1 || N < 0 || H < 1 || d < 2 || d % 2 || base <= 0.0) return ORC_EARG;
  double sgn = inverse ? -1.0 : 1.0;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < N; ++t) {
    double pos = (double)(pos_offset + t);
    for (int64_t c = 0; c < d / 2; ++c) {
      double theta = pos * pow(base, -2.0 * (double)c / (double)d);
      double cs = cos(theta), sn = sgn * sin(theta);
      for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
          const double *xi = x + ((b * N + t) * H + h) * d;
          double *yi = y + ((b * N + t) * H + h) * d;
          double a0 = xi[2 * c], a1 = xi[2 * c + 1];
          yi[2 * c] = a0 * cs - a1 * sn;
          yi[2 * c + 1] = a0 * sn + a1 * cs;
        }
    }
  }
  return ORC_OK;
}

/* Number of OpenMP threads a parallel region of this library uses. */
int orc_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
