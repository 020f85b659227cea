#!/usr/bin/env python3
"""Benchmark: causal attention forward+backward throughput on one MI355X.

One step = dfa_attn_fwd (fused) + dfa_attn_bwd over the whole DistFlashAttn
folded schedule (P = 8 virtual ranks) of a Llama-7B attention layer:
batch 1, 32 heads, head_dim 128, N = 32768, bf16, Q/K/V iid N(0,1) scaled by
1/sqrt(d), dO iid N(0,1).  Inputs are generated before timing and stay
resident in HBM.

Throughput counts causal-effective FLOPs over the exact visible pairs:
4*d per pair forward (QK^T and PV) and 10*d per pair backward (the recompute
of S plus dP, dV, dK, dQ).  Per kernel the algorithmic share is: forward
4*d; dK/dV kernel 8*d (the recompute of S, dV, dP and dK); dQ kernel 2*d
(dQ).  Recomputations beyond those five backward products (S and dP again
in the dQ kernel) are extra work and not counted.  The dominant kernel's roofline figure uses that share and the
kernel's own average duration, read from HIP events recorded on the stream
right before and after it (dfa_attn_bwd_ex marks).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "causal attention fwd+bwd TFLOP/s and % bf16 MFMA peak, Llama-7B shape N=32K"

WORKLOADS = {
    "llama7b-n32k-balanced-p8": dict(B=1, N=32768, Hq=32, Hkv=32, D=128, kind=1, P=8, seed=1003,
                                     scaled=True, rank=None),
    "llama7b-n131k-striped-p16-rank0": dict(B=1, N=131072, Hq=32, Hkv=32, D=128, kind=2, P=16,
                                            seed=1004, scaled=False, rank=0),
    "gqa-32-8-n256k-balanced-p32": dict(B=1, N=262144, Hq=32, Hkv=8, D=128, kind=1, P=32,
                                        seed=1005, scaled=False, rank=None),
    # stripe blocks of 64 / 128 tokens (the striped-attention page's block sizes)
    "llama7b-n32k-striped64-p8": dict(B=1, N=32768, Hq=32, Hkv=32, D=128, kind=2, P=8, seed=1003,
                                      scaled=True, rank=None, stripe=64),
    "llama7b-n32k-striped128-p8": dict(B=1, N=32768, Hq=32, Hkv=32, D=128, kind=2, P=8, seed=1003,
                                       scaled=True, rank=None, stripe=128),
    # packed documents of 1K-8K tokens (the striped-attention page's document
    # packing), attention kept inside each document
    "llama7b-n32k-docs-balanced-p8": dict(B=1, N=32768, Hq=32, Hkv=32, D=128, kind=1, P=8,
                                          seed=1003, scaled=True, rank=None, docs=(1024, 8192)),
    "llama7b-n32k-docs-striped64-p8": dict(B=1, N=32768, Hq=32, Hkv=32, D=128, kind=2, P=8,
                                           seed=1003, scaled=True, rank=None, stripe=64,
                                           docs=(1024, 8192)),
    # rotary embedding of q and k at absolute positions before the ring (the
    # striped-attention page's RoPE placement), gradients turned back after it
    "llama7b-n32k-rope-striped64-p8": dict(B=1, N=32768, Hq=32, Hkv=32, D=128, kind=2, P=8,
                                           seed=1003, scaled=True, rank=None, stripe=64,
                                           rope=10000.0),
}


def doc_bounds(wl):
    """The workload's packed-document boundaries (host int64), or None."""
    if "docs" not in wl:
        return None
    from long_context_sequence_dfa_amd import inputs
    return inputs.doc_bounds(wl["seed"], wl["N"], *wl["docs"])


def schedule(dfa, wl):
    """The workload's full block list (every rank)."""
    if wl.get("stripe", 1) > 1:
        return dfa.dfa_schedule_build_striped_blocks(wl["N"], wl["P"], wl["stripe"])
    return dfa.dfa_schedule_build(wl["kind"], wl["N"], wl["P"])


def source_hash(kernel_file: str) -> str:
    """sha256[:16] over a kernel source file and every header in csrc/ (the
    kernels include all of them), so any change to the code that builds the
    kernel changes the hash."""
    import hashlib
    csrc = os.path.join(ROOT, "long_context_sequence_dfa_amd", "csrc")
    h = hashlib.sha256(open(os.path.join(csrc, kernel_file), "rb").read())
    for f in sorted(os.listdir(csrc)):
        if f.endswith(".h"):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch of ``kernel`` from the committed counter summary
    (profiles/traffic.txt: FETCH_SIZE + WRITE_SIZE scaled by a plain copy),
    or None when absent or when the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        parts = line.split()
        if len(parts) == 4 and parts[0] == kernel and parts[1] == workload:
            fname, want = parts[2].split(":")
            src = os.path.join(ROOT, "long_context_sequence_dfa_amd", "csrc", fname)
            if not os.path.exists(src) or source_hash(fname) != want:
                return None
            return float(parts[3])
    return None


def cpu_baseline(wl: dict, budget_s: float = 20.0) -> dict:
    """The fp64 oracle on a bounded sample of the workload: forward and full
    gradients of head 0 over the first n tokens (a complete causal
    sub-problem: those rows see only keys < n), timed on the host cores."""
    import numpy as np

    import oracle
    from long_context_sequence_dfa_amd import inputs
    oracle.build(force=False)
    D = wl["D"]
    scale = 1.0 / math.sqrt(D)
    qs = scale if wl["scaled"] else None
    best = None
    n = 1024
    full_docs = doc_bounds(wl)
    while True:
        q = inputs.normal_tensor(wl["seed"], 0, (1, n, 1, D), "bf16", qs)
        k = inputs.normal_tensor(wl["seed"], 1, (1, n, 1, D), "bf16", qs)
        v = inputs.normal_tensor(wl["seed"], 2, (1, n, 1, D), "bf16", qs)
        do = inputs.normal_tensor(wl["seed"], 3, (1, n, 1, D), "bf16")
        docs = None
        if full_docs is not None:  # the documents cut at n
            docs = np.append(full_docs[full_docs < n], n)
        t0 = time.perf_counter()
        oracle.attn_rows(q, k, v, scale, docs=docs)
        oracle.attn_grads(q, k, v, do, scale, docs=docs)
        dt = time.perf_counter() - t0
        lens = [n] if docs is None else np.diff(docs)
        pairs = sum(int(x) * (int(x) + 1) // 2 for x in lens)
        best = (n, dt, 14.0 * D * pairs / dt / 1e12)
        if dt * 4.2 > budget_s or n >= 32768:  # next doubling would exceed the budget
            break
        n *= 2
    n, dt, tflops = best
    return {"value": tflops, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"head 0, first {n} tokens (complete causal prefix"
                      f"{', its documents' if full_docs is not None else ''}), fwd + full grads, "
                      f"fp64, {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b-n32k-balanced-p8", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="fused", choices=["fused", "stepwise"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy first (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus "
              f"{args.gpus}); the schedules run as virtual ranks on one device.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import long_context_sequence_dfa_amd as dfa
    from long_context_sequence_dfa_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    binding.lib()
    wl = WORKLOADS[args.workload]
    B, N, Hq, Hkv, D = wl["B"], wl["N"], wl["Hq"], wl["Hkv"], wl["D"]
    dev = torch.device("cuda:0")
    scale = 1.0 / math.sqrt(D)
    qs = scale if wl["scaled"] else None
    q, k, v, do = inputs.workload_tensors(wl["seed"], B, N, Hq, Hkv, D, "bf16", qs, with_do=True)
    tq, tk, tv, tdo = (inputs.to_torch(x, "bf16", dev) for x in (q, k, v, do))
    del q, k, v, do
    from long_context_sequence_dfa_amd import timeline
    blocks = schedule(dfa, wl)
    if wl["rank"] is not None:
        blocks = blocks[blocks[:, 0] == wl["rank"]]
    docs = doc_bounds(wl)
    td = None if docs is None else torch.tensor(docs, dtype=torch.int32, device=dev)
    if docs is None:
        pairs = int(blocks[:, 9].sum()) * B * Hq
        bal = dfa.dfa_schedule_balance(schedule(dfa, wl), wl["P"])
    else:  # visible pairs and the ring balance under the document mask
        pairs = int(timeline.doc_pair_counts(blocks, docs).sum()) * B * Hq
        full = schedule(dfa, wl)
        bal = timeline.measured_balance(timeline.pair_times(full, wl["P"],
                                                            timeline.doc_pair_counts(full, docs)))
    fwd_flops = 4.0 * D * pairs
    bwd_flops = 10.0 * D * pairs
    mode = dfa.DFA_FWD_FUSED if args.mode == "fused" else dfa.DFA_FWD_STEPWISE

    o = torch.empty_like(tq)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    desc = dfa.make_desc(tq, tk, tv, o, docs=td)
    op_f = dfa.DFA_OP_FWD_FUSED if mode == dfa.DFA_FWD_FUSED else dfa.DFA_OP_FWD_STEPWISE
    ws_f = torch.empty(max(dfa.dfa_workspace_size(desc, blocks, op_f), 256), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(dfa.dfa_workspace_size(desc, blocks, dfa.DFA_OP_BWD), 256), dtype=torch.uint8,
                       device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    from long_context_sequence_dfa_amd.timeline import HipEvents
    ev = HipEvents()
    # per step: fwd begin, fwd end, then the backward's marks
    ev_all = [[ev.create() for _ in range(9)] for _ in range(args.steps)]
    rope = wl.get("rope")
    qr, kr = (torch.empty_like(tq), torch.empty_like(tk)) if rope else (tq, tk)

    def step(m=None):
        # events: 7 forward begin (rotation of q, k first), 0 attention
        # forward begin, 1 forward end, 2-6 backward marks, 8 after the
        # gradients are turned back (rotations only: 7 == 0, 8 == 6)
        if m is not None:
            ev.h.hipEventRecord(m[7], sp)
        if rope:
            dfa.dfa_rope(tq, qr, base=rope)
            dfa.dfa_rope(tk, kr, base=rope)
        if m is not None:
            ev.h.hipEventRecord(m[0], sp)
        dfa.dfa_attn_fwd(qr, kr, tv, blocks, mode, o=o, lse=lse, workspace=ws_f, docs=td)
        marks = None
        if m is not None:
            ev.h.hipEventRecord(m[1], sp)
            marks = binding.DfaKernelMarks(m[2], m[3], m[4], m[5], m[6])
        dfa.dfa_attn_bwd(qr, kr, tv, o, tdo, lse, blocks, dq=dq, dk=dk, dv=dv, workspace=ws_b,
                         marks=marks, docs=td)
        if rope:
            dfa.dfa_rope(dq, dq, base=rope, inverse=True)
            dfa.dfa_rope(dk, dk, base=rope, inverse=True)
        if m is not None:
            ev.h.hipEventRecord(m[8], sp)

    if args.calibrate_copy:
        # one plain device copy of known size: the scale for HBM byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev_all[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the other forward mode, timed on its own (a few launches): the pages'
    # per-step partial-plus-merge form when the timed mode is fused, and back
    alt_mode = dfa.DFA_FWD_STEPWISE if mode == dfa.DFA_FWD_FUSED else dfa.DFA_FWD_FUSED
    alt_op = dfa.DFA_OP_FWD_STEPWISE if alt_mode == dfa.DFA_FWD_STEPWISE else dfa.DFA_OP_FWD_FUSED
    ws_alt = torch.empty(max(dfa.dfa_workspace_size(desc, blocks, alt_op), 256), dtype=torch.uint8,
                         device=dev)
    o_alt = torch.empty_like(tq)
    lse_alt = torch.empty_like(lse)
    dfa.dfa_attn_fwd(tq, tk, tv, blocks, alt_mode, o=o_alt, lse=lse_alt, workspace=ws_alt, docs=td)
    e0, e1 = ev.create(), ev.create()
    n_alt = 3
    ev.h.hipEventRecord(e0, sp)
    for _ in range(n_alt):
        dfa.dfa_attn_fwd(tq, tk, tv, blocks, alt_mode, o=o_alt, lse=lse_alt, workspace=ws_alt, docs=td)
    ev.h.hipEventRecord(e1, sp)
    alt_ms = ev.elapsed(e0, e1) / n_alt
    del ws_alt, o_alt, lse_alt

    # measured per-(rank, step) slot times of one ring-faithful stepwise
    # forward (each slot launched on its own between events): the idle
    # bubble a synchronous ring of P devices would see with these slot costs
    full = schedule(dfa, wl)  # every rank, also for a rank's share
    slot_ms = timeline.slot_times(tq, tk, tv, full, wl["P"], stream=stream, docs=td)
    bubble_measured = timeline.measured_balance(slot_ms)["bubble"]

    per = {name: float(np.mean([ev.elapsed(m[a], m[b]) for m in ev_all]))
           for name, a, b in (("fwd", 0, 1), ("bwd", 1, 6), ("bwd_pre", 2, 3), ("dq", 3, 4),
                              ("dkdv", 5, 6), ("rope_in", 7, 0), ("rope_back", 6, 8))}
    ms_step = elapsed * 1e3 / args.steps
    total_flops = (fwd_flops + bwd_flops) * args.steps
    value = total_flops / elapsed / 1e12
    fwd_avg, bwd_avg = per["fwd"], per["bwd"]

    # the dominant kernel by time, with its algorithmic FLOP share
    kernels = {"attn_fwd_bf16_fused": (per["fwd"], fwd_flops),
               "attn_bwd_dq_bf16": (per["dq"], 2.0 * D * pairs),
               "attn_bwd_dkdv_bf16": (per["dkdv"], 8.0 * D * pairs)}
    dom = max(kernels, key=lambda n: kernels[n][0])
    dom_ms, dom_flops = kernels[dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": stored_traffic(dom, args.workload), "launch_ms": dom_ms,
                "algorithmic_flop": dom_flops}

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "fwd_ms": fwd_avg,
        "bwd_ms": bwd_avg,
        "kernel_ms": {k_: per[k_] for k_ in ("fwd", "bwd_pre", "dq", "dkdv")},
        **({"rope_ms": {"q_k_forward": per["rope_in"], "dq_dk_back": per["rope_back"]},
            # q and k forward, dq and dk back: each pass reads and writes its bf16 tensor once
            "rope_gbs": 8.0 * (tq.numel() + tk.numel()) / ((per["rope_in"] + per["rope_back"]) * 1e-3) / 1e9}
           if rope else {}),
        "fwd_tflops": fwd_flops / (fwd_avg * 1e-3) / 1e12,
        f"fwd_{'stepwise' if mode == dfa.DFA_FWD_FUSED else 'fused'}_ms": alt_ms,
        f"fwd_{'stepwise' if mode == dfa.DFA_FWD_FUSED else 'fused'}_tflops": fwd_flops / (alt_ms * 1e-3) / 1e12,
        "bwd_tflops": bwd_flops / (bwd_avg * 1e-3) / 1e12,
        "idle_bubble_ratio": bal["bubble"],
        "idle_bubble_ratio_measured": bubble_measured,
        "comm_latency_ms": 0.0,
        "config": {"workload": args.workload, "global_batch": B, "seq_len": N, "heads_q": Hq,
                   "heads_kv": Hkv, "head_dim": D,
                   "schedule": {0: "ring", 1: "balanced", 2: "striped"}[wl["kind"]],
                   "stripe": wl.get("stripe", 1),
                   "documents": None if docs is None else {"count": len(docs) - 1,
                                                            "lengths": list(wl["docs"])},
                   "rope_base": rope,
                   "virtual_ranks": wl["P"], "rank_share": wl["rank"], "mode": args.mode,
                   "parallelism": "none: virtual ranks on one GPU"},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
