"""GPU parity at the full workload sizes, on outputs the fp64 oracle computes
one by one: output rows and LSE of sampled query rows (random, first, last,
chunk edges), dQ of those rows, and dK/dV of the last key rows (whose query
rows the oracle can afford); for the benchmark's workload (and the
grouped-query schedule at a length the oracle affords) every dQ row of one
head and the first 64 keys of every chunk -- the keys read by the most
query pieces, the key-major kernel's longest walks -- against every query
row that sees them.  Heads are sampled as whole grouped-query groups so the
oracle sees a consistent sub-problem.  Whole-tensor invariants (sum_j dK_j =
0, sum_j dV_j = sum_i dO_i) cover every head, with bounds computed from the
inputs alone.  The launch configuration is the benchmark's (fused forward,
the same block lists)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import schedule_ref as sr
from tests.parity_util import bhnd, check_grad, check_out, rows_of, sum_invariant_bounds, to_np

pytestmark = pytest.mark.gpu

# name: (N, Hq, Hkv, kind, P, seed, qkv_scaled, rank, heads_sampled)
WORKLOADS = {
    "llama7b-n32k-balanced-p8": (32768, 32, 32, sr.BALANCED, 8, 1003, True, None, [0, 17]),
    "llama7b-n131k-striped-p16-rank0": (131072, 32, 32, sr.STRIPED, 16, 1004, False, 0, [5]),
    "gqa-32-8-n256k-balanced-p32": (262144, 32, 8, sr.BALANCED, 32, 1005, False, None, [1]),
    # stripe blocks of 64 tokens at the Llama-7B shape (kind STRIPED_BLOCK)
    "llama7b-n32k-striped64-p8": (32768, 32, 32, sr.STRIPED_BLOCK, 8, 1003, True, None, [9]),
    # packed documents of 1K-8K tokens over the folded schedule
    "llama7b-n32k-docs-balanced-p8": (32768, 32, 32, sr.BALANCED, 8, 1003, True, None, [4]),
    # head_dim 64 (its own tile pitch and load split) over a long folded walk
    "d64-n64k-balanced-p8": (65536, 16, 16, sr.BALANCED, 8, 1006, False, None, [3]),
}
HEAD_DIM = {"d64-n64k-balanced-p8": 64}
STRIPE = {"llama7b-n32k-striped64-p8": 64}
DOCS = {"llama7b-n32k-docs-balanced-p8": (1024, 8192)}


@pytest.fixture(scope="module")
def dfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sequence_dfa_amd as m
    from long_context_sequence_dfa_amd import binding
    binding.lib()
    return m


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_sampled_parity(dfa, name):
    from long_context_sequence_dfa_amd import inputs
    N, Hq, Hkv, kind, P, seed, scaled, rank, kv_heads = WORKLOADS[name]
    D, group = HEAD_DIM.get(name, 128), Hq // Hkv
    print(f"case: {name} generating inputs", flush=True)
    qs = 1 / math.sqrt(D) if scaled else None
    q, k, v, do = inputs.workload_tensors(seed, 1, N, Hq, Hkv, D, "bf16", qs, with_do=True)
    dev = torch.device("cuda:0")
    tq, tk, tv, tdo = (inputs.to_torch(x, "bf16", dev) for x in (q, k, v, do))
    if kind == sr.STRIPED_BLOCK:
        blocks = dfa.dfa_schedule_build_striped_blocks(N, P, STRIPE[name])
    else:
        blocks = dfa.dfa_schedule_build(kind, N, P)
    if rank is not None:
        blocks = blocks[blocks[:, 0] == rank]
    docs = inputs.doc_bounds(seed, N, *DOCS[name]) if name in DOCS else None
    td = None if docs is None else torch.tensor(docs, dtype=torch.int32, device=dev)
    print(f"case: {name} forward + backward on the GPU ({len(blocks)} blocks)", flush=True)
    o, lse = dfa.dfa_attn_fwd(tq, tk, tv, blocks, docs=td)
    dq, dk, dv = dfa.dfa_attn_bwd(tq, tk, tv, o, tdo, lse, blocks, docs=td)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(dq.float()).all()
    assert torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()

    rows_all = rows_of(blocks)
    rng = np.random.default_rng(seed)
    chunk = {sr.BALANCED: N // (2 * P), sr.STRIPED_BLOCK: STRIPE.get(name, 1)}.get(kind, N // P)
    edges = [x for c in range(1, N // chunk) for x in (c * chunk - 1, c * chunk)]
    if docs is not None:  # both sides of every document boundary
        edges += [x for b in docs[1:-1] for x in (b - 1, b)]
    cand = np.concatenate([rng.choice(rows_all, 40, replace=False), rows_all[:4], rows_all[-4:],
                           np.array(edges[:8] + edges[-8:], dtype=np.int64)]
                          + ([] if docs is None else [np.array(edges[-2 * (len(docs) - 2):], dtype=np.int64)]))
    rows = np.intersect1d(np.unique(cand), rows_all)
    scale = 1 / math.sqrt(D)
    for hk in kv_heads:
        heads = list(range(hk * group, (hk + 1) * group))
        print(f"case: {name} oracle, kv head {hk}, {rows.size} rows", flush=True)
        qh, doh = q[:, :, heads], do[:, :, heads]
        kh, vh = k[:, :, [hk]], v[:, :, [hk]]
        ro, rl = oracle.attn_rows(qh, kh, vh, scale, rows=rows, docs=docs)
        ra, _ = oracle.attn_rows(qh, kh, np.abs(vh), scale, rows=rows, docs=docs)  # error magnitudes of O
        go = bhnd(to_np(o[:, rows][:, :, heads]))
        gl = to_np(lse[:, heads][:, :, rows])
        check_out(go, ro, gl, rl, "bf16", f"{name} O", oabs=ra, n_keys=N)
        lse_r, dd_r, rdq, aa, adq = oracle.grad_rows(qh, kh, vh, doh, scale, rows=rows, with_abs=True,
                                                     docs=docs)
        gq = bhnd(to_np(dq[:, rows][:, :, heads]))
        # the rms of a sampled gradient set stands in for the tensor's
        check_grad(gq, rdq, adq, "bf16", f"{name} dQ")
        # last key rows: their query rows are the tail of the row set
        tail_rows = rows_all[rows_all >= N - 96]
        keys = np.arange(N - 64, N)
        l2, d2, _, a2, _ = oracle.grad_rows(qh, kh, vh, doh, scale, rows=tail_rows, with_abs=True,
                                            docs=docs)
        rdk, rdv, adk, adv = oracle.grad_cols(qh, kh, vh, doh, scale, tail_rows, l2, d2, keys=keys,
                                              aa=a2, docs=docs)
        gk = bhnd(to_np(dk[:, keys][:, :, [hk]]))
        gv = bhnd(to_np(dv[:, keys][:, :, [hk]]))
        check_grad(gk, rdk, adk, "bf16", f"{name} dK")
        check_grad(gv, rdv, adv, "bf16", f"{name} dV")
    check_sum_invariants(name, q, k, v, do, scale, rows_all, dk, dv)
    print(f"case: {name} done", flush=True)


def check_sum_invariants(name, q, k, v, do, scale, rows, dk, dv):
    """Whole-tensor invariants, valid at any size: softmax is shift invariant
    in k (sum_j dK_j = 0), and sum_j dV_j is the sum of dO over the rows and
    the group's heads; bounds from the inputs alone (sum_invariant_bounds:
    2^-7 times the summed error magnitudes, no GPU value in them)."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if len(rows) == N:  # every row: no copies of the full tensors
        rows = slice(None)
    bk, bv = sum_invariant_bounds(q, k, v, do, scale, rows=None if isinstance(rows, slice) else rows)
    sk = dk.double().sum(dim=1).cpu().numpy()                 # [B, Hkv, D]
    sv = dv.double().sum(dim=1).cpu().numpy()
    want = np.zeros((B, Hkv, D))
    for h in range(Hq):
        want[:, h // (Hq // Hkv)] += np.asarray(do[:, rows, h], np.float64).sum(axis=1)
    rk, rv = float((np.abs(sk) / bk).max()), float((np.abs(sv - want) / bv).max())
    print(f"case: {name} sum dK error / bound {rk:.4f}, sum dV error / bound {rv:.4f}", flush=True)
    assert rk <= 1.0, f"{name} sum dK"
    assert rv <= 1.0, f"{name} sum dV"


# the benchmark's workload at full length, and the grouped-query folded
# schedule at a length whose every query row the oracle affords (P = 32,
# 64 chunks of 256, so the first chunk's keys are read by 64 query pieces):
# name, N, Hq, Hkv, P, seed, scaled, kv head checked
HEAVY = [
    ("llama7b-n32k-balanced-p8", 32768, 32, 32, 8, 1003, True, 0),
    ("gqa-32-8-n16k-balanced-p32", 16384, 32, 8, 32, 1005, False, 1),
]


@pytest.mark.parametrize("case", HEAVY, ids=[c[0] for c in HEAVY])
def test_heavy_keys_full_length(dfa, case):
    """dK and dV of the first 64 keys of every chunk of the folded schedule
    (each read by every later query piece: the longest key-major walks,
    many query tiles summed in the kernel's cost-sorted order, the group's
    query heads summed for grouped-query attention) against every query row
    that sees them; and every dQ row of the group's heads.  Mean and
    elementwise bounds."""
    from long_context_sequence_dfa_amd import inputs
    name, N, Hq, Hkv, P, seed, scaled, hk = case
    D, group = 128, Hq // Hkv
    print(f"case: heavy keys {name} generating inputs", flush=True)
    scale = 1 / math.sqrt(D)
    q, k, v, do = inputs.workload_tensors(seed, 1, N, Hq, Hkv, D, "bf16", scale if scaled else None,
                                          with_do=True)
    dev = torch.device("cuda:0")
    tq, tk, tv, tdo = (inputs.to_torch(x, "bf16", dev) for x in (q, k, v, do))
    blocks = dfa.dfa_schedule_build(sr.BALANCED, N, P)
    print(f"case: heavy keys {name} forward + backward on the GPU", flush=True)
    o, lse = dfa.dfa_attn_fwd(tq, tk, tv, blocks)
    dq, dk, dv = dfa.dfa_attn_bwd(tq, tk, tv, o, tdo, lse, blocks)
    torch.cuda.synchronize()
    heads = list(range(hk * group, (hk + 1) * group))
    qh, doh = q[:, :, heads], do[:, :, heads]
    kh, vh = k[:, :, [hk]], v[:, :, [hk]]
    C = N // (2 * P)
    keys = np.concatenate([np.arange(c * C, c * C + 64) for c in range(2 * P)])
    rows = np.arange(N)
    print(f"case: heavy keys {name} oracle: {len(heads)} heads x {N} rows", flush=True)
    lse_r, dd_r, rdq, aa, adq = oracle.grad_rows(qh, kh, vh, doh, scale, rows=rows, with_abs=True)
    print(f"case: heavy keys {name} oracle: {keys.size} keys", flush=True)
    rdk, rdv, adk, adv = oracle.grad_cols(qh, kh, vh, doh, scale, rows, lse_r, dd_r, keys=keys, aa=aa)
    check_grad(bhnd(to_np(dq[:, :, heads])), rdq, adq, "bf16", f"{name} dQ (all rows)")
    check_grad(bhnd(to_np(dk[:, keys][:, :, [hk]])), rdk, adk, "bf16", f"{name} dK (chunk heads)")
    check_grad(bhnd(to_np(dv[:, keys][:, :, [hk]])), rdv, adv, "bf16", f"{name} dV (chunk heads)")
    check_sum_invariants(name, q, k, v, do, scale, rows, dk, dv)
    print(f"case: heavy keys {name} done", flush=True)


# stepwise forward (per-ring-step partials merged in the kernel epilogue) at
# full size: the forward workload's shape and schedule, the token-striped
# rank share, and stripe blocks of 64
STEPWISE = ["llama7b-n32k-balanced-p8", "llama7b-n131k-striped-p16-rank0", "llama7b-n32k-striped64-p8"]


@pytest.mark.parametrize("name", STEPWISE)
def test_stepwise_forward_full_shape(dfa, name):
    """The stepwise forward at the workload's full size against the oracle on
    sampled rows (random, first, last, both sides of every chunk edge) of
    the sampled heads; every row of every head against the fused forward
    (the same mathematics through another merge order: agreement within the
    bf16 output bounds)."""
    from long_context_sequence_dfa_amd import inputs
    N, Hq, Hkv, kind, P, seed, scaled, rank, kv_heads = WORKLOADS[name]
    D, group = 128, Hq // Hkv
    print(f"case: stepwise {name} generating inputs", flush=True)
    q, k, v = inputs.workload_tensors(seed, 1, N, Hq, Hkv, D, "bf16", 1 / math.sqrt(D) if scaled else None)
    dev = torch.device("cuda:0")
    tq, tk, tv = (inputs.to_torch(x, "bf16", dev) for x in (q, k, v))
    if kind == sr.STRIPED_BLOCK:
        blocks = dfa.dfa_schedule_build_striped_blocks(N, P, STRIPE[name])
    else:
        blocks = dfa.dfa_schedule_build(kind, N, P)
    if rank is not None:
        blocks = blocks[blocks[:, 0] == rank]
    print(f"case: stepwise {name} forward on the GPU ({len(blocks)} blocks)", flush=True)
    o, lse = dfa.dfa_attn_fwd(tq, tk, tv, blocks, mode=dfa.DFA_FWD_STEPWISE)
    of, lf = dfa.dfa_attn_fwd(tq, tk, tv, blocks)
    torch.cuda.synchronize()
    rows_all = rows_of(blocks)
    ridx = torch.as_tensor(rows_all, device=dev)
    eo = (o[:, ridx].float() - of[:, ridx].float()).abs()
    el = (lse[:, :, ridx] - lf[:, :, ridx]).abs()
    print(f"case: stepwise {name} vs fused: O max {eo.max().item():.3e} mean {eo.mean().item():.3e}, "
          f"LSE max {el.max().item():.3e}", flush=True)
    assert eo.max().item() <= 2e-2 and eo.mean().item() <= 2e-3 and el.max().item() <= 1e-3
    rng = np.random.default_rng(seed + 7)
    chunk = {sr.BALANCED: N // (2 * P), sr.STRIPED_BLOCK: STRIPE.get(name, 1)}.get(kind, N // P)
    edges = [x for c in range(1, N // chunk) for x in (c * chunk - 1, c * chunk)]
    cand = np.concatenate([rng.choice(rows_all, 48, replace=False), rows_all[:4], rows_all[-4:],
                           np.array(edges[:8] + edges[-8:], dtype=np.int64)])
    rows = np.intersect1d(np.unique(cand), rows_all)
    scale = 1 / math.sqrt(D)
    for hk in kv_heads:
        heads = list(range(hk * group, (hk + 1) * group))
        print(f"case: stepwise {name} oracle, kv head {hk}, {rows.size} rows", flush=True)
        ro, rl = oracle.attn_rows(q[:, :, heads], k[:, :, [hk]], v[:, :, [hk]], scale, rows=rows)
        ra, _ = oracle.attn_rows(q[:, :, heads], k[:, :, [hk]], np.abs(v[:, :, [hk]]), scale, rows=rows)
        check_out(bhnd(to_np(o[:, rows][:, :, heads])), ro, to_np(lse[:, heads][:, :, rows]), rl, "bf16",
                  f"stepwise {name} O", oabs=ra, n_keys=N)
    print(f"case: stepwise {name} done", flush=True)
