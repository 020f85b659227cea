/*
 * dfa.h -- C ABI of libdfa: blockwise exact causal attention with an online
 * softmax, run as P virtual ranks of a context-parallel ring on one AMD
 * Instinct MI355X (gfx950).
 *
 * Method (from the pages this library follows):
 *  - Causal attention: a key at position j is visible to the query at
 *    position i iff j <= i; scores are q_i.k_j * scale with scale = 1/sqrt(d)
 *    (Striped Attention Guide, "The Fatal Flaw: Causal Workload Imbalance",
 *    masked score equation).
 *  - Per (query chunk, key chunk) block the kernel keeps a running row max,
 *    a running row sum of exponentials and a running output, rescaling them
 *    as new key tiles arrive, and normalises at the end (Striped Attention
 *    Guide, "Algorithmic Mechanics" 1, steps 1-7).
 *  - Partial results of the blocks of one query chunk are combined by
 *    log-sum-exp rescaling; the result is exact attention (same section;
 *    FlashAttention glossary page, "exact same attention matrix").
 *  - The backward pass keeps only the output and the per-row log-sum-exp and
 *    recomputes the probabilities (FlashAttention glossary page, first two
 *    paragraphs; DistFlashAttn paper record, "rematerialisation-aware
 *    gradient checkpointing").
 *  - Schedules: the contiguous ring, DistFlashAttn's folded chunk pairs and
 *    round-robin token striping (DistFlashAttn Guide, "The Causal Imbalance
 *    Crisis" and "Core Innovation 1"; Striped Attention Guide, "Round-Robin
 *    Permutation" and "Mathematical Formulation of Token Striping").  At ring
 *    step s rank r holds the key/value shard of rank (r - s) mod P (Striped
 *    Attention Guide, "Workload Balance Theorem").  On one GPU a ring step is
 *    a pointer hand-off: a block simply reads the owner's rows in place.
 *
 * Conventions for every call:
 *  - Every call returns a dfa_status: DFA_OK (0) or a negative error.  No C++
 *    exception crosses the ABI.  On an error nothing has been enqueued.
 *  - Device pointers are plain HIP device addresses; the caller allocates,
 *    owns and frees every buffer, including the workspace.  The library
 *    never allocates, frees or synchronises device memory.
 *  - "stream" is the caller's hipStream_t passed as void*; NULL means the
 *    default stream.  Calls other than dfa_schedule_build,
 *    dfa_schedule_balance, dfa_workspace_size and dfa_status_string only
 *    enqueue work and return; device faults surface at the caller's next
 *    synchronisation.  Launch failures return DFA_E_HIP.
 *  - Inputs are never modified.  Outputs must not alias inputs.
 *  - Tensors are logically [batch, token, head, head_dim] with head_dim
 *    contiguous; the descriptor gives element strides for batch, token and
 *    head.  Row pointers must be 16-byte aligned (strides multiples of 8
 *    elements for bf16, 4 for fp32).
 *  - Not thread-safe per stream: calls that share a stream are ordered by it;
 *    calls on different streams must not share output or workspace buffers.
 */
#ifndef DFA_H_
#define DFA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dfa_status;

enum {
  DFA_OK = 0,
  DFA_E_NULL = -1,        /* a required pointer is NULL */
  DFA_E_SHAPE = -2,       /* sizes inconsistent (e.g. P does not divide N, Hq % Hkv != 0) */
  DFA_E_UNSUPPORTED = -3, /* head_dim, dtype, mode or schedule kind not supported */
  DFA_E_ALIGN = -4,       /* pointer or stride violates the 16-byte row alignment */
  DFA_E_CAPACITY = -5,    /* output array too small */
  DFA_E_WORKSPACE = -6,   /* workspace missing or smaller than dfa_workspace_size() */
  DFA_E_HIP = -7          /* a HIP runtime call or kernel launch failed */
};

/* Schedule kinds. */
enum {
  DFA_SCHED_RING = 0,     /* rank p owns tokens [p*N/P, (p+1)*N/P) */
  DFA_SCHED_BALANCED = 1, /* 2P chunks of N/(2P); rank p owns chunks p and 2P-1-p */
  DFA_SCHED_STRIPED = 2   /* rank p owns tokens i with i mod P == p */
};

/* Element types of Q, K, V, O, dO, dQ, dK, dV.  Accumulation is always fp32. */
enum { DFA_F32 = 0, DFA_BF16 = 1 };

/* Forward modes of dfa_attn_fwd. */
enum {
  DFA_FWD_FUSED = 0,   /* one launch; each query tile walks its rank's blocks in ring-step
                          order with the running max/sum/output in registers */
  DFA_FWD_STEPWISE = 1 /* ring-faithful: per step, every rank's blocks compute partial
                          (O, LSE) pairs that are merged into fp32 accumulators (the merge
                          runs in the partial kernel's epilogue; one launch per round of
                          blocks with distinct query rows) */
};

/* Operations for dfa_workspace_size. */
enum { DFA_OP_FWD_FUSED = 0, DFA_OP_FWD_STEPWISE = 1, DFA_OP_BWD = 2 };

/*
 * One block of a schedule: the queries of one shard of rank `rank` against
 * the keys of one shard of rank `kv_rank` at ring step `step`.  Eleven
 * little-endian int64 fields (88 bytes).  A shard is a sequence of runs of
 * `run` consecutive tokens, consecutive runs `stride` apart: local row i sits
 * at global position start + (i / run) * stride + i % run.  run = 1 gives the
 * rows start + i * stride (contiguous chunks: stride 1; token stripes:
 * stride P); block stripes of B tokens have run = B, stride = P * B.  Key j is
 * visible to query i iff its global position is not after the query's; for
 * run = 1 that is j <= i + diag_offset.  Only blocks with at least one visible
 * pair exist.
 */
typedef struct dfa_block {
  int64_t rank;        /* virtual rank computing the block (owns the query rows) */
  int64_t step;        /* ring step s in [0, P) */
  int64_t kv_rank;     /* (rank - step) mod P: owner of the key/value rows */
  int64_t q_start;     /* global position of local query row 0 */
  int64_t kv_start;    /* global position of local key row 0 */
  int64_t len_q;       /* number of query rows */
  int64_t len_kv;      /* number of key rows */
  int64_t stride;      /* global distance between consecutive runs: 1 (chunks), P (token
                          stripes), P * B (block stripes) */
  int64_t diag_offset; /* floor((q_start - kv_start) / stride) */
  int64_t pairs;       /* number of visible (query, key) pairs */
  int64_t run;         /* consecutive tokens per run: 1, or B for block stripes */
} dfa_block;

/*
 * Attention problem.  q: [batch][seqlen][heads_q][head_dim], k and v:
 * [batch][seqlen][heads_kv][head_dim], o: like q.  Strides are in elements,
 * ordered (batch, token, head).  Query head h reads key/value head
 * h / (heads_q / heads_kv) (grouped-query attention, FlashAttention glossary
 * page, "variants").  Gradients use their primal's strides: dq like q, dk like
 * k, dv like v, d_o like o.  LSE arrays are fp32 [batch][heads_q][seqlen],
 * contiguous, natural logarithm.
 *
 * Packed documents (Striped Attention Guide, "Production Deployment and Best
 * Practices", item 3): when doc_bounds is not NULL the sequence is a
 * concatenation of n_docs documents and a query attends only to keys of its
 * own document (on top of the causal rule).  doc_bounds is a DEVICE array of
 * n_docs + 1 int32 positions, doc_bounds[0] = 0 < doc_bounds[1] < ... <
 * doc_bounds[n_docs] = seqlen; document t holds positions [doc_bounds[t],
 * doc_bounds[t+1]).  The same boundaries apply to every batch entry.  The
 * host cannot read them: calls check only 1 <= n_docs <= seqlen < 2^31
 * (else DFA_E_SHAPE); boundaries that break the rule above give unspecified
 * results (no out-of-bounds access).  With doc_bounds NULL, n_docs is ignored.
 */
typedef struct dfa_attn_desc {
  int32_t dtype;         /* DFA_BF16 or DFA_F32 */
  int32_t batch;         /* >= 1 */
  int32_t heads_q;       /* >= 1 */
  int32_t heads_kv;      /* >= 1, divides heads_q */
  int32_t head_dim;      /* 64 or 128 */
  float softmax_scale;   /* finite and > 0, else DFA_E_SHAPE; the caller passes
                            1/sqrt(head_dim) for standard attention */
  int64_t seqlen;        /* global N; every pointer indexes global token order */
  int64_t q_strides[3];
  int64_t k_strides[3];
  int64_t v_strides[3];
  int64_t o_strides[3];
  const int32_t *doc_bounds; /* device, n_docs + 1 entries, or NULL (one document) */
  int64_t n_docs;
} dfa_attn_desc;

/*
 * Per-schedule balance figures (host-side accounting over dfa_block.pairs).
 *   rank_pairs[r]  : visible pairs computed by rank r (array of n_ranks)
 *   step_max[s]    : largest per-rank load in ring step s (array of n_ranks)
 *   bubble         : 1 - total / (P * sum_s step_max[s]) -- share of rank-time
 *                    idle in a lock-step ring (Striped Attention Guide, "The
 *                    Fatal Flaw", point 2)
 *   eta_blocks     : busy (rank, step) slots / P^2 -- the pages' block-count
 *                    utilisation (DistFlashAttn Guide, "The Causal Imbalance
 *                    Crisis", eta_util)
 */
typedef struct dfa_balance {
  int64_t total_pairs;
  int64_t busy_slots;
  double bubble;
  double eta_blocks;
} dfa_balance;

/*
 * dfa_schedule_build -- enumerate the blocks of a schedule (host only).
 *   kind      : DFA_SCHED_*.
 *   seqlen    : N >= 1.  RING and STRIPED need N % n_ranks == 0, BALANCED
 *               N % (2*n_ranks) == 0 ("P divides the sequence length",
 *               DistFlashAttn Guide, "Operational Checklist"); else DFA_E_SHAPE.
 *   n_ranks   : P >= 1.
 *   out       : host array of `capacity` blocks, or NULL to only count.
 *   n_out     : receives the number of blocks (always set on DFA_OK and on
 *               DFA_E_CAPACITY).
 * Blocks are written in (rank, step, q_start, kv_start) order.  Defined by the
 * folded chunk assignment (DistFlashAttn Guide, "Core Innovation 1"), the
 * contiguous split ("The Causal Imbalance Crisis") and token striping
 * (Striped Attention Guide, "Mathematical Formulation of Token Striping").
 */
dfa_status dfa_schedule_build(int32_t kind, int64_t seqlen, int32_t n_ranks, dfa_block *out,
                              int64_t capacity, int64_t *n_out);

/*
 * dfa_schedule_build_striped_blocks -- the striped schedule with stripe blocks
 * of `stripe` tokens (host only): rank p owns the tokens i with
 * floor(i / stripe) = p (mod P) (Striped Attention Guide, "Mathematical
 * Formulation of Token Striping", block-striped variant, and its "Block
 * Stripe Size" recommendation of 64 or 128).  At step s rank r holds the keys
 * of rank (r - s) mod P, as in DFA_SCHED_STRIPED.  Blocks have run = stripe and
 * stride = P * stripe; stripe = 1 reproduces DFA_SCHED_STRIPED exactly.
 *   seqlen : N with N % (n_ranks * stripe) == 0, else DFA_E_SHAPE.
 *   stripe : >= 1.  The attention calls take run = 1 or run = 64 * 2^k (their
 *            row tiles are 64 rows, and a tile's run is found by a shift);
 *            other stripes are only enumerated.
 * Other arguments as dfa_schedule_build.
 */
dfa_status dfa_schedule_build_striped_blocks(int64_t seqlen, int32_t n_ranks, int64_t stripe,
                                             dfa_block *out, int64_t capacity, int64_t *n_out);

/*
 * dfa_schedule_balance -- per-rank and per-step loads of a block list (host).
 *   rank_pairs, step_max : host arrays of n_ranks int64, or NULL.
 *   out                  : receives the totals (may be NULL).
 * Blocks with rank or step outside [0, n_ranks) give DFA_E_SHAPE.
 */
dfa_status dfa_schedule_balance(const dfa_block *blocks, int64_t n_blocks, int32_t n_ranks,
                                int64_t *rank_pairs, int64_t *step_max, dfa_balance *out);

/*
 * dfa_attn_block_fwd -- one block's partial attention (Striped Attention
 * Guide, "Algorithmic Mechanics" 1, steps 1-3 and 7 for a single block).
 *   o_part   : device fp32 [batch][heads_q][len_q][head_dim], contiguous; row i
 *              is the block's query row i normalised over the block's visible
 *              keys only.
 *   lse_part : device fp32 [batch][heads_q][len_q]; LSE of those keys.
 * A row with no visible key gets O = 0 and LSE = -inf.  bf16: the 2^31-byte
 * limit on 64 rows of k and v of dfa_attn_fwd applies.
 */
dfa_status dfa_attn_block_fwd(const dfa_attn_desc *d, const dfa_block *blk, const void *q,
                              const void *k, const void *v, float *o_part, float *lse_part,
                              void *stream);

/*
 * dfa_lse_merge -- in place (o_acc, lse_acc) <- (o_acc, lse_acc) (+) (o_part, lse_part).
 * With M = max(lse_acc, lse_part) and LSE = M + ln(e^{lse_acc-M} + e^{lse_part-M}):
 * o_acc = e^{lse_acc-LSE} o_acc + e^{lse_part-LSE} o_part (the normalised form
 * of the alpha/beta rescaling, Striped Attention Guide, "Algorithmic
 * Mechanics" 1, steps 4-6).  The identity element is (0, -inf); merging two
 * (., -inf) rows gives (0, -inf), never NaN.
 *   n_rows   : number of rows; o arrays are fp32 [n_rows][head_dim], lse fp32 [n_rows].
 */
dfa_status dfa_lse_merge(int64_t n_rows, int32_t head_dim, float *o_acc, float *lse_acc,
                         const float *o_part, const float *lse_part, void *stream);

/*
 * dfa_attn_fwd -- forward over a block list (a whole schedule or any subset,
 * e.g. one rank's share): exact causal attention of every query row over the
 * keys its blocks give it, O = softmax(scale Q K^T) V per row with the
 * running max / sum / output of the online softmax and LSE = m + ln l
 * (Striped Attention Guide, "Algorithmic Mechanics" 1, steps 1-7; the page's
 * opening of "Algorithmic Mechanics" states that the result is exact, equal to
 * one monolithic attention pass, as does the FlashAttention glossary page,
 * first two paragraphs).
 *   blocks/n_blocks : host array (as built by dfa_schedule_build or a subset).
 *                     The distinct query pieces (q_start, len_q, stride, run) must
 *                     not share rows, nor the distinct key pieces.
 *   mode            : DFA_FWD_FUSED or DFA_FWD_STEPWISE.
 *   o               : device, dtype, strides o_strides.
 *   lse             : device fp32 [batch][heads_q][seqlen].
 *   workspace       : device buffer of at least dfa_workspace_size() bytes,
 *                     256-byte aligned (may be NULL if that size is 0).
 * Output rows that no block touches are written as O = 0, LSE = -inf.
 * bf16: 64 consecutive rows of one piece must span less than 2^31 bytes in
 * each of k and v (64 * 2 * token stride * row step, the row step being the
 * block's stride for run = 1 and 1 otherwise), else DFA_E_UNSUPPORTED.
 */
dfa_status dfa_attn_fwd(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n_blocks,
                        int32_t mode, const void *q, const void *k, const void *v, void *o,
                        float *lse, void *workspace, size_t ws_bytes, void *stream);

/*
 * dfa_attn_bwd -- gradients of the forward over the same block list:
 * dS = P (dP - D) with P recomputed from the saved LSE and D = rowsum(dO*O)
 * (the backward keeps only O and the per-row statistics and recomputes the
 * attention matrix: FlashAttention glossary page, first two paragraphs;
 * DistFlashAttn paper record, "rematerialisation-aware gradient
 * checkpointing").  The gradient formulas are the vector-Jacobian product of
 * the forward's definition; the pages give none.
 *   o, lse      : the forward's outputs for the same block list.
 *   dq, dk, dv  : device, dtype, strides of q, k, v.  Overwritten; rows no
 *                 block touches are written as 0.  For grouped-query
 *                 attention dk and dv sum over the query heads of a group.
 * bf16 only: 64 consecutive rows of one piece must span less than 2^31
 * bytes in each of q, k, v and d_o (64 * 2 * token stride * row step, the row
 * step being the block's stride for run = 1 and 1 otherwise), else
 * DFA_E_UNSUPPORTED.
 */
dfa_status dfa_attn_bwd(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n_blocks,
                        const void *q, const void *k, const void *v, const void *o,
                        const void *d_o, const float *lse, void *dq, void *dk, void *dv,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * Optional timing marks for dfa_attn_bwd_ex.  Each non-NULL member is a
 * hipEvent_t (passed as void*) created by the caller; the call records it on
 * its stream right before the named kernel is launched, or (end) right after
 * its last launch.  Recording changes no result and skips no work.  The
 * backward launches, in order: D = rowsum(dO*O), the dQ kernel, and one
 * kernel that computes both dK and dV: dk_begin and dv_begin are recorded
 * back to back before it, so the dK-to-dV interval is empty and dv_begin to
 * end times the dK/dV kernel.
 */
typedef struct dfa_kernel_marks {
  void *pre_begin;
  void *dq_begin;
  void *dk_begin;
  void *dv_begin;
  void *end;
} dfa_kernel_marks;

/*
 * dfa_attn_bwd_ex -- dfa_attn_bwd plus per-kernel timing marks (marks may be
 * NULL, which makes it identical to dfa_attn_bwd).  An event that fails to
 * record returns DFA_E_HIP after the work is enqueued.
 */
dfa_status dfa_attn_bwd_ex(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n_blocks,
                           const void *q, const void *k, const void *v, const void *o,
                           const void *d_o, const float *lse, void *dq, void *dk, void *dv,
                           void *workspace, size_t ws_bytes, const dfa_kernel_marks *marks,
                           void *stream);

/*
 * Timing marks of a ring-faithful forward, one per (rank, step) slot.
 * events is a host array of n_ranks * n_ranks + 1 hipEvent_t handles (as
 * void*) created by the caller.
 */
typedef struct dfa_slot_marks {
  void **events;
  int32_t n_ranks;
} dfa_slot_marks;

/*
 * dfa_attn_fwd_slots -- the stepwise forward (DFA_FWD_STEPWISE semantics
 * and results) launched one (rank, step) slot at a time, as P devices of a
 * synchronous ring would run it: the slots go out in (step, rank) order,
 * events[s * P + r] is recorded on the stream right before slot (r, s) --
 * also for a slot without blocks -- and events[P * P] after the last, so
 * the elapsed time between consecutive events is one slot's time on the
 * GPU (the per-rank timeline behind the idle-bubble figures of the
 * DistFlashAttn Guide, "Breakdown of Idle Time and Bubble Elimination", and
 * the Striped Attention Guide, "End-to-End Throughput Scaling").  Blocks must have rank and step
 * in [0, n_ranks) (else DFA_E_SHAPE); marks and marks->events must not be
 * NULL; n_ranks >= 1.  Workspace: dfa_workspace_size(DFA_OP_FWD_STEPWISE).
 * An event that fails to record returns DFA_E_HIP after the work is
 * enqueued.
 */
dfa_status dfa_attn_fwd_slots(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n_blocks,
                              const void *q, const void *k, const void *v, void *o, float *lse,
                              void *workspace, size_t ws_bytes, const dfa_slot_marks *marks,
                              void *stream);

/*
 * dfa_attn_bwd_noalloc -- dfa_attn_bwd without a workspace argument, for
 * callers that cannot allocate device memory (tight serving loops, harnesses
 * that forbid hipMalloc): the call allocates no device memory and uses the
 * library's fixed scratch of 80 MiB per GPU instead (a device array each GPU
 * holds from the first use until the process ends).  Not for HIP graph
 * capture: like every call here it uploads its planning tables with an
 * asynchronous host-to-device copy from a host buffer that is released when
 * the call returns, which a captured graph would replay.
 * Same arguments, results and errors as dfa_attn_bwd, plus:
 *   - DFA_E_WORKSPACE when the problem needs more than the scratch
 *     (dfa_workspace_size(DFA_OP_BWD) > 80 MiB; about 8 bytes per
 *     batch x heads_q x seqlen row plus the planning tables), checked on the
 *     host before anything is enqueued;
 *   - DFA_E_UNSUPPORTED when `stream` belongs to another device than the
 *     current one (the scratch used is the current device's).
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (other streams, other host threads) race and must be ordered by
 * the caller.  Nothing in the scratch has to start at zero; each call
 * rewrites what it reads.
 */
dfa_status dfa_attn_bwd_noalloc(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n_blocks,
                                const void *q, const void *k, const void *v, const void *o,
                                const void *d_o, const float *lse, void *dq, void *dk, void *dv,
                                void *stream);

/*
 * dfa_workspace_size -- bytes of workspace `op` (DFA_OP_*) needs for this
 * descriptor and block list.  Pure host computation.
 */
dfa_status dfa_workspace_size(const dfa_attn_desc *d, const dfa_block *blocks, int64_t n_blocks,
                              int32_t op, size_t *bytes);

/*
 * dfa_rope -- rotary position embedding at absolute positions (Striped
 * Attention Guide, "Preserving Rotary Position Embeddings (RoPE)": each token
 * vector turns by its absolute sequence index, applied before the ring
 * exchange).  The pages name the rotation without its parameters; this is
 * the RoFormer form with interleaved pairs: pair c = (x[2c], x[2c+1]) of the
 * token with index t turns by (pos_offset + t) * base^(-2c/head_dim)
 * (base 10000 in the usual models).  inverse = 1 turns by minus that angle:
 * the transpose, which maps gradients of the rotated tensor back
 * (dq = dfa_rope(dq_rot, inverse = 1)).  Tensors of this library hold global
 * token order, so a striped shard's row m of rank p already sits at its
 * absolute position m*P + p.
 *   dtype          : DFA_BF16 or DFA_F32 (x and y alike).
 *   x, y           : device [batch][seqlen][heads][head_dim], element strides
 *                    x_strides / y_strides (batch, token, head; host arrays of
 *                    3), head_dim contiguous.  y == x (same strides) rotates in
 *                    place; other overlaps are not allowed.
 *   head_dim       : even, 2..512.  Strides even; x and y aligned to one pair
 *                    (4 bytes bf16, 8 bytes fp32), else DFA_E_ALIGN.
 *   pos_offset     : position of token 0 (>= 0).
 * The angle and its sine and cosine are computed in fp64; each output is
 * rounded once (to fp32, then for bf16 to bf16, nearest even).
 */
dfa_status dfa_rope(int32_t dtype, int32_t batch, int64_t seqlen, int32_t heads, int32_t head_dim,
                    const int64_t *x_strides, const void *x, const int64_t *y_strides, void *y,
                    int64_t pos_offset, double base, int32_t inverse, void *stream);

/* Static English text for a status code (never NULL). */
const char *dfa_status_string(dfa_status s);

#ifdef __cplusplus
}
#endif

#endif /* DFA_H_ */
