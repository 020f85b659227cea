"""Brute-force enumerator of the virtual-rank schedules -- TEST INFRASTRUCTURE.

Part of the oracle: only tests, the smoke check and the benchmark's CPU
baseline may import it.  It shares no code with the library's schedule
builder.  Every block is derived by listing token positions and counting
visible (query, key) pairs one by one; nothing here uses the closed forms the
library uses.

Definitions taken from the pages:

* RING -- rank p owns the contiguous positions [p*N/P, (p+1)*N/P)
  (DistFlashAttn Guide, "The Causal Imbalance Crisis"; Striped Attention
  Guide, "The Rise of Context Parallelism").
* BALANCED -- the sequence is cut into 2P chunks; rank i owns chunk i and
  chunk 2P-1-i (DistFlashAttn Guide, "Core Innovation 1", "The Folded Chunk
  Assignment", and the worker listing's folded chunk indices).
* STRIPED -- rank p owns the positions i with i mod P == p (Striped Attention
  Guide, "Mathematical Formulation of Token Striping", first set).
* STRIPED_BLOCK (stripe B) -- rank p owns the positions i with
  floor(i / B) mod P == p (the same section, block-striped set).
* Ring rotation -- at step s rank p holds the key/value shard of rank
  (p - s) mod P: shards move to rank p+1 each step (Striped Attention Guide,
  "Workload Balance Theorem"; DistFlashAttn worker listing, next/prev ranks).
* Visibility -- key at position j is visible to the query at position i iff
  j <= i (Striped Attention Guide, masked score equation; the GlobalPos rule
  of "Algorithmic Mechanics" 1, step 2).

A block is one (query piece of rank p) x (key piece of rank (p-s) mod P) with
at least one visible pair.  A piece is a sorted list of positions, described
by (start, length, stride, run): runs of `run` consecutive positions, runs
`stride` apart.  RING has one piece per rank, BALANCED two (its low and high
chunk), STRIPED one with stride P (run 1), STRIPED_BLOCK one with stride P*B
and run B; the description is checked against the listed positions.

Block record (11 little-endian int64): rank, step, kv_rank, q_start, kv_start,
len_q, len_kv, stride, diag_offset, pairs, run.  For run 1, diag_offset is the
integer o with "local key j visible to local query i iff j <= i + o"; when
several o fit (a block where every pair is visible) the record uses
floor((q_start-kv_start)/stride).  For run > 1 visibility is not one shifted
diagonal and the record carries floor((q_start-kv_start)/stride) as well.
Blocks are listed in (rank, step, q_start, kv_start) order.
"""
from __future__ import annotations

import numpy as np

RING, BALANCED, STRIPED, STRIPED_BLOCK = 0, 1, 2, 3
KIND_NAMES = {RING: "ring", BALANCED: "balanced", STRIPED: "striped",
              STRIPED_BLOCK: "striped_block"}
FIELDS = ("rank", "step", "kv_rank", "q_start", "kv_start", "len_q", "len_kv",
          "stride", "diag_offset", "pairs", "run")


def rank_pieces(kind: int, n: int, p: int, stripe: int = 1):
    """List, per rank, of its (start, length, stride, run) position runs."""
    if p < 1 or n < 1:
        raise ValueError("need N >= 1 and P >= 1")
    if kind == RING:
        if n % p:
            raise ValueError("P must divide N")
        c = n // p
        return [[(r * c, c, 1, 1)] for r in range(p)]
    if kind == BALANCED:
        if n % (2 * p):
            raise ValueError("2P must divide N")
        c = n // (2 * p)
        return [[(r * c, c, 1, 1), ((2 * p - 1 - r) * c, c, 1, 1)] for r in range(p)]
    if kind == STRIPED:
        if n % p:
            raise ValueError("P must divide N")
        return [[(r, n // p, p, 1)] for r in range(p)]
    if kind == STRIPED_BLOCK:
        if stripe < 1 or n % (p * stripe):
            raise ValueError("P * stripe must divide N")
        out = []
        for r in range(p):
            # the definition, listed: positions whose stripe block belongs to r
            own = np.nonzero((np.arange(n, dtype=np.int64) // stripe) % p == r)[0]
            piece = (int(own[0]), int(own.size), p * stripe, stripe)
            if not np.array_equal(positions(piece), own):
                raise AssertionError("stripe-block piece description does not list its positions")
            out.append([piece])
        return out
    raise ValueError("unknown schedule kind")


def positions(piece) -> np.ndarray:
    start, length, stride, run = piece
    i = np.arange(length, dtype=np.int64)
    return start + (i // run) * stride + i % run


def _diag_offset(qpos: np.ndarray, kpos: np.ndarray, q_start, kv_start, stride) -> int:
    """Find by brute force the offsets o that reproduce every row's visible
    count, then return the conventional one (checked to be among them)."""
    counts = np.searchsorted(kpos, qpos, side="right")  # visible keys per query row
    len_kv = kpos.size
    i = np.arange(qpos.size)
    # rows strictly inside (0 < count < len_kv) pin o exactly; edge rows bound it
    inside = (counts > 0) & (counts < len_kv)
    cand = set((counts[inside] - 1 - i[inside]).tolist())
    if len(cand) > 1:
        raise AssertionError("block visibility is not a shifted diagonal")
    conventional = (q_start - kv_start) // stride
    if cand:
        (o,) = cand
        if o != conventional:
            raise AssertionError("diagonal offset disagrees with its definition")
        return o
    # every row sees all keys or none: all o with clamp(i+o+1, 0, len_kv) == counts fit
    if not np.array_equal(np.clip(i + conventional + 1, 0, len_kv), counts):
        raise AssertionError("conventional diagonal offset does not fit the block")
    return conventional


def enumerate_schedule(kind: int, n: int, p: int, stripe: int = 1) -> np.ndarray:
    """All non-empty blocks of a schedule as an int64 array [n_blocks, 11]."""
    pieces = rank_pieces(kind, n, p, stripe)
    out = []
    for r in range(p):
        for s in range(p):
            j = (r - s) % p
            for qp in pieces[r]:
                for kp in pieces[j]:
                    qpos, kpos = positions(qp), positions(kp)
                    pairs = int(np.searchsorted(kpos, qpos, side="right").sum())
                    if pairs == 0:
                        continue
                    if qp[3] == 1:
                        off = _diag_offset(qpos, kpos, qp[0], kp[0], qp[2])
                    else:
                        off = (qp[0] - kp[0]) // qp[2]
                    out.append((r, s, j, qp[0], kp[0], qp[1], kp[1], qp[2], off, pairs, qp[3]))
    out.sort(key=lambda t: (t[0], t[1], t[3], t[4]))
    return np.array(out, dtype=np.int64).reshape(-1, 11)


def to_bytes(blocks: np.ndarray) -> bytes:
    return np.ascontiguousarray(blocks, dtype="<i8").tobytes()


def balance(blocks: np.ndarray, p: int) -> dict:
    """Per-rank totals, per-step maxima and the idle-bubble ratio.

    bubble = 1 - (sum of all pairs) / (P * sum over steps of the largest rank
    load in that step): the share of rank-time spent waiting in a lock-step
    ring where each step lasts as long as its busiest rank (Striped Attention
    Guide, "The Fatal Flaw", point 2).  eta_blocks counts busy (rank, step)
    slots over P^2, the pages' block-count utilisation (DistFlashAttn Guide,
    "The Causal Imbalance Crisis", eta_util).
    """
    load = np.zeros((p, p), dtype=np.int64)  # [rank, step]
    for b in blocks:
        load[b[0], b[1]] += b[9]
    total = int(load.sum())
    step_max = load.max(axis=0)
    denom = p * int(step_max.sum())
    bubble = 1.0 - total / denom if denom else 0.0
    return {
        "rank_pairs": load.sum(axis=1),
        "step_max": step_max,
        "total_pairs": total,
        "bubble": bubble,
        "eta_blocks": float((load > 0).sum()) / (p * p),
        "load": load,
    }
