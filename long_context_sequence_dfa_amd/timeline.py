"""Measured per-virtual-rank timeline of one forward pass.

The pages assess a schedule by how long each rank computes at each ring step:
a step lasts as long as its slowest rank, and the time the other ranks wait
is the idle bubble (DistFlashAttn Guide, "Breakdown of Idle Time and Bubble
Elimination"; Striped Attention Guide, "Why Striping Solves Load Imbalance"
and "End-to-End Throughput Scaling").  On one GPU every (rank, step) slot
can be timed on its own.  slot_times runs one ring-faithful stepwise
forward (dfa_attn_fwd_slots) whose slots are launched one after the other
in (step, rank) order between HIP events, so each slot's time is its own
launches' time on the GPU.  rank_step_times instead times each block alone
through dfa_attn_block_fwd (median of repeats) and sums a slot's blocks.
The slot times, combined the way a synchronous ring combines them
(measured_balance), give the measured counterpart of the pair-count balance
that dfa_schedule_balance computes from the block list.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import binding


class HipEvents:
    """HIP events through libamdhip64 (the runtime torch already loaded)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.h.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def destroy(self, e) -> None:
        self.h.hipEventDestroy(e)

    def elapsed(self, a, b) -> float:
        """Milliseconds from event a to event b (waits for b)."""
        if self.h.hipEventSynchronize(b) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


def slot_times(q, k, v, blocks, n_ranks: int, stream=None, docs=None, warmup: int = 1, runs: int = 5):
    """Milliseconds per (rank, step) slot, shape [n_ranks, n_ranks]: the
    median over ``runs`` ring-faithful stepwise forwards (after ``warmup``
    untimed ones) of the time between the events recorded right before the
    slot's launches and right before the next slot's.  The median per slot
    keeps launch and clock jitter out of the per-step maxima; slots without
    blocks cost only the gap between two event records."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    P = int(n_ranks)
    hip = HipEvents()
    ev = [hip.create() for _ in range(P * P + 1)]
    try:
        o = torch.empty_like(q)
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
        desc = binding.make_desc(q, k, v, o, docs=docs)
        ws = torch.empty(max(binding.dfa_workspace_size(desc, blocks, binding.DFA_OP_FWD_STEPWISE), 256),
                         dtype=torch.uint8, device=q.device)
        for _ in range(max(warmup, 0)):
            binding.dfa_attn_fwd_slots(q, k, v, blocks, ev, P, o=o, lse=lse, workspace=ws,
                                       stream=stream, docs=docs)
        samples = np.zeros((max(int(runs), 1), P, P), dtype=np.float64)
        for n in range(samples.shape[0]):
            binding.dfa_attn_fwd_slots(q, k, v, blocks, ev, P, o=o, lse=lse, workspace=ws,
                                       stream=stream, docs=docs)
            for s in range(P):
                for r in range(P):
                    i = s * P + r
                    samples[n, r, s] = hip.elapsed(ev[i], ev[i + 1])
        return np.median(samples, axis=0)
    finally:
        torch.cuda.synchronize()
        for e in ev:
            hip.destroy(e)


def rank_step_times(q, k, v, blocks, n_ranks: int, repeats: int = 3, scale=None, stream=None,
                    docs=None):
    """Milliseconds per (rank, step) slot, shape [n_ranks, n_ranks]: each block
    timed alone (median of ``repeats`` launches after one warm-up launch),
    summed over the blocks of its slot.  Slots without blocks cost 0.
    ``docs``: optional int32 device tensor of packed-document boundaries."""
    import torch
    arr = binding._blocks_arg(blocks)
    if stream is None:
        stream = torch.cuda.current_stream()
    B, _, Hq, D = q.shape
    times = np.zeros((n_ranks, n_ranks), dtype=np.float64)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * repeats)]
    for blk in arr:
        rank, step, len_q = int(blk[0]), int(blk[1]), int(blk[5])
        op = torch.empty((B, Hq, len_q, D), dtype=torch.float32, device=q.device)
        lp = torch.empty((B, Hq, len_q), dtype=torch.float32, device=q.device)
        binding.dfa_attn_block_fwd(q, k, v, blk, op, lp, scale=scale, stream=stream, docs=docs)
        for r in range(repeats):
            ev[2 * r].record(stream)
            binding.dfa_attn_block_fwd(q, k, v, blk, op, lp, scale=scale, stream=stream, docs=docs)
            ev[2 * r + 1].record(stream)
        stream.synchronize()
        times[rank, step] += float(np.median([ev[2 * r].elapsed_time(ev[2 * r + 1])
                                              for r in range(repeats)]))
    return times


def measured_balance(times) -> dict:
    """Synchronous-ring accounting of slot costs ``times[rank, step]``: per-rank
    busy time, per-step maximum, makespan (sum of the step maxima) and the
    idle bubble 1 - sum(times) / (P * makespan)."""
    t = np.asarray(times, dtype=np.float64)
    P = t.shape[0]
    step_max = t.max(axis=0)
    makespan = float(step_max.sum())
    busy = float(t.sum())
    bubble = 1.0 - busy / (P * makespan) if makespan > 0 else 0.0
    return {"rank_busy": t.sum(axis=1), "step_max": step_max, "makespan": makespan,
            "busy": busy, "bubble": bubble}


def pair_times(blocks, n_ranks: int, pairs=None):
    """The pair counts of the block list in the same [rank, step] layout (the
    cost model in which dfa_schedule_balance measures the bubble); ``pairs``
    overrides the blocks' own counts (e.g. doc_pair_counts)."""
    arr = binding._blocks_arg(blocks)
    t = np.zeros((n_ranks, n_ranks), dtype=np.float64)
    for n, blk in enumerate(arr):
        t[int(blk[0]), int(blk[1])] += float(blk[9] if pairs is None else pairs[n])
    return t


def _piece_positions(start, length, stride, run):
    i = np.arange(length, dtype=np.int64)
    return start + (i // run) * stride + i % run


def doc_pair_counts(blocks, bounds):
    """Visible pairs of each block when the sequence packs documents with
    cumulative boundaries ``bounds`` (host array): pairs (query, key) with the
    key not after the query and both in one document (Striped Attention Guide,
    "Production Deployment and Best Practices", item 3)."""
    arr = binding._blocks_arg(blocks)
    b = np.asarray(bounds, dtype=np.int64).reshape(-1)
    out = np.zeros(len(arr), dtype=np.int64)
    for n, blk in enumerate(arr):
        qp = _piece_positions(blk[3], blk[5], blk[7], blk[10])
        kp = _piece_positions(blk[4], blk[6], blk[7], blk[10])
        lo = b[np.searchsorted(b, qp, side="right") - 1]
        seen = np.searchsorted(kp, qp, side="right") - np.searchsorted(kp, lo, side="left")
        out[n] = int(np.maximum(seen, 0).sum())
    return out
