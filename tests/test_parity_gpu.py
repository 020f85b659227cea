"""GPU parity: the HIP library through the C ABI against the fp64 oracle on
the same seeded inputs, element by element, at sizes that span several tiles
and a ragged tail; plus edge cases and run-to-run determinism."""
import numpy as np
import pytest
import torch

import oracle
from oracle import schedule_ref as sr
from tests.parity_util import (bhnd, check_grad, check_out, kv_rows_of, rows_of, to_np)

pytestmark = pytest.mark.gpu

RING, BAL, STR = sr.RING, sr.BALANCED, sr.STRIPED


@pytest.fixture(scope="module")
def dfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sequence_dfa_amd as m
    from long_context_sequence_dfa_amd import binding
    binding.lib()
    return m


def make(seed, B, N, Hq, Hkv, D, dtype, qkv_scale=None):
    from long_context_sequence_dfa_amd import inputs
    q, k, v, do = inputs.workload_tensors(seed, B, N, Hq, Hkv, D, dtype, qkv_scale, with_do=True)
    dev = torch.device("cuda:0")
    t = tuple(inputs.to_torch(x, dtype, dev) for x in (q, k, v, do))
    return (q, k, v, do), t


def say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- workload 1
def test_ring_fp32_blocks_merge_and_full(dfa):
    """N=1024, d=64, one head, fp32, contiguous ring with P=4: every block's
    partial, the step-order merge per rank, and the full forward."""
    say("case: ring fp32 N=1024 d=64 P=4 blocks/merge/full")
    N, D, P = 1024, 64, 4
    (q, k, v, do), (tq, tk, tv, tdo) = make(1001, 1, N, 1, 1, D, "f32")
    scale = 1 / np.sqrt(D)
    blocks = dfa.dfa_schedule_build(RING, N, P)
    ro, rl = oracle.attn_rows(q, k, v, scale)
    for r in range(P):
        rb = blocks[blocks[:, 0] == r]
        acc_o = torch.zeros((1, 1, N // P, D), dtype=torch.float32, device="cuda")
        acc_l = torch.full((1, 1, N // P), float("-inf"), device="cuda")
        for b in rb:  # step order
            op, lp = dfa.dfa_attn_block_fwd(tq, tk, tv, b)
            torch.cuda.synchronize()
            xo, xl = oracle.block_partial(q, k, v, scale, *b[3:8])
            check_out(to_np(op), xo, to_np(lp), xl, "f32", f"block {b[:3]}")
            dfa.dfa_lse_merge(acc_o, acc_l, op, lp)
        torch.cuda.synchronize()
        rows = slice(r * N // P, (r + 1) * N // P)
        check_out(to_np(acc_o), ro[:, :, rows], to_np(acc_l), rl[:, :, rows], "f32", f"rank {r}")
    for mode in (dfa.DFA_FWD_FUSED, dfa.DFA_FWD_STEPWISE):
        o, lse = dfa.dfa_attn_fwd(tq, tk, tv, blocks, mode)
        torch.cuda.synchronize()
        check_out(bhnd(to_np(o)), ro, to_np(lse), rl, "f32", f"fwd mode {mode}")
    dq, dk, dv = dfa.dfa_attn_bwd(tq, tk, tv, o, tdo, lse, blocks)
    torch.cuda.synchronize()
    (rdq, rdk, rdv), (adq, adk, adv) = oracle.attn_grads(q, k, v, do, scale, with_abs=True)
    for n, g, r, a in (("dq", dq, rdq, adq), ("dk", dk, rdk, adk), ("dv", dv, rdv, adv)):
        check_grad(bhnd(to_np(g)), r, a, "f32", n, n_terms=N)


# ------------------------------------------------------------ bf16 matrix
CASES = [
    # kind, N, P, B, Hq, Hkv, D, subset rank
    (BAL, 1024, 4, 1, 2, 2, 128, None),
    (BAL, 1000, 4, 2, 4, 2, 128, None),     # ragged chunks (125 rows)
    (RING, 768, 3, 2, 2, 1, 64, None),
    (RING, 640, 5, 1, 3, 3, 128, None),
    (STR, 1024, 8, 1, 2, 2, 128, None),
    (STR, 1024, 8, 1, 4, 1, 128, 0),        # rank 0's share (diag offsets 0 and -1)
    (STR, 1152, 16, 1, 2, 2, 64, 15),       # last rank's share
    (BAL, 2048, 8, 1, 2, 1, 64, 3),         # one folded rank
    (BAL, 96, 1, 1, 1, 1, 128, None),       # P = 1: one diagonal block
]


def with_dtypes(cases, f32_ok):
    """Every case in bf16; in fp32 only the cases f32_ok accepts (the fp32
    path is covered on the smaller ones)."""
    out = []
    for dtype in ("bf16", "f32"):
        for c in cases:
            if dtype == "bf16" or f32_ok(c):
                out.append(pytest.param(c, dtype, id=dtype + "-" + "-".join(str(x) for x in c)))
    return out


@pytest.mark.parametrize("case,dtype", with_dtypes(CASES, lambda c: True))
def test_forward_backward_parity(dfa, case, dtype):
    kind, N, P, B, Hq, Hkv, D, sub = case
    say(f"case: {sr.KIND_NAMES[kind]} N={N} P={P} B={B} Hq={Hq} Hkv={Hkv} D={D} rank={sub} {dtype}")
    blocks = dfa.dfa_schedule_build(kind, N, P)
    if sub is not None:
        blocks = blocks[blocks[:, 0] == sub]
    check_schedule(dfa, blocks, 2000 + N + P, N, B, Hq, Hkv, D, dtype)


# stripe blocks of 64 or 128 tokens (the striped-attention page's recommended
# block stripe sizes): N, P, stripe, batch, Hq, Hkv, d, subset rank
STRIPE_CASES = [
    (2048, 4, 64, 1, 2, 1, 128, None),
    (1280, 4, 64, 2, 2, 2, 64, None),      # 5 runs per rank: a ragged 256-row workgroup
    (4096, 8, 128, 1, 4, 2, 128, 5),       # one rank's share
    (1536, 2, 128, 1, 2, 2, 128, 0),
    (512, 8, 64, 1, 1, 1, 128, None),      # one run per rank
]


@pytest.mark.parametrize("case,dtype", with_dtypes(STRIPE_CASES, lambda c: True))
def test_stripe_block_parity(dfa, case, dtype):
    N, P, stripe, B, Hq, Hkv, D, sub = case
    say(f"case: stripe blocks N={N} P={P} stripe={stripe} B={B} Hq={Hq} Hkv={Hkv} D={D} "
        f"rank={sub} {dtype}")
    blocks = dfa.dfa_schedule_build_striped_blocks(N, P, stripe)
    if sub is not None:
        blocks = blocks[blocks[:, 0] == sub]
    (q, k, v, _), (tq, tk, tv, _) = make(4000 + N + P, B, N, Hq, Hkv, D, dtype)
    scale = 1 / np.sqrt(D)
    for b in blocks[:6]:  # single-block partials (a diagonal run block among them)
        op, lp = dfa.dfa_attn_block_fwd(tq, tk, tv, b)
        torch.cuda.synchronize()
        xo, xl = oracle.block_partial(q, k, v, scale, *b[3:8], run=b[10])
        xa, _ = oracle.block_partial(q, k, np.abs(v), scale, *b[3:8], run=b[10])
        check_out(to_np(op), xo, to_np(lp), xl, dtype, f"block {b[:3]}", oabs=xa, n_keys=N)
    check_schedule(dfa, blocks, 4000 + N + P, N, B, Hq, Hkv, D, dtype)


def check_schedule(dfa, blocks, seed, N, B, Hq, Hkv, D, dtype, docs=None, arrays=None,
                   grad_mean=True):
    """Fused and stepwise forward and the backward of a block list against the
    oracle on the rows it touches; every other row must come out zero.
    ``docs``: optional cumulative document boundaries (packed documents).
    ``arrays``: optional (q, k, v, dO) fp32 arrays exact in ``dtype`` used in
    place of the seeded normal inputs; ``grad_mean`` False drops the mean
    statistic of the bf16 gradient check (the elementwise bound stays)."""
    if arrays is None:
        (q, k, v, do), (tq, tk, tv, tdo) = make(seed, B, N, Hq, Hkv, D, dtype)
    else:
        from long_context_sequence_dfa_amd import inputs
        q, k, v, do = arrays
        tq, tk, tv, tdo = (inputs.to_torch(x, dtype, torch.device("cuda:0")) for x in arrays)
    scale = 1 / np.sqrt(D)
    td = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda")
    rows, krows = rows_of(blocks), kv_rows_of(blocks)
    ro, rl = oracle.attn_rows(q, k, v, scale, rows=rows, docs=docs)
    ra, _ = oracle.attn_rows(q, k, np.abs(v), scale, rows=rows, docs=docs)  # error magnitudes of O
    outs = {}
    for mode in (dfa.DFA_FWD_FUSED, dfa.DFA_FWD_STEPWISE):
        o, lse = dfa.dfa_attn_fwd(tq, tk, tv, blocks, mode, docs=td)
        torch.cuda.synchronize()
        go, gl = bhnd(to_np(o)), to_np(lse)
        check_out(go[:, :, rows], ro, gl[:, :, rows], rl, dtype, f"mode {mode}", oabs=ra, n_keys=N)
        other = np.setdiff1d(np.arange(N), rows)
        assert np.all(go[:, :, other] == 0) and np.all(np.isneginf(gl[:, :, other]))
        outs[mode] = (o, lse)
    o, lse = outs[dfa.DFA_FWD_FUSED]
    dq, dk, dv = dfa.dfa_attn_bwd(tq, tk, tv, o, tdo, lse, blocks, docs=td)
    torch.cuda.synchronize()
    (rdq, rdk, rdv), (adq, adk, adv) = oracle.attn_grads(q, k, v, do, scale, rows=rows, with_abs=True,
                                                          docs=docs)
    gq, gk, gv = bhnd(to_np(dq)), bhnd(to_np(dk)), bhnd(to_np(dv))
    nq, nk = N, N * (Hq // Hkv)  # terms per dQ element, per dK/dV element (at most)
    check_grad(gq[:, :, rows], rdq, adq, dtype, "dq", check_mean=grad_mean, n_terms=nq)
    check_grad(gk[:, :, krows], rdk[:, :, krows], adk[:, :, krows], dtype, "dk", check_mean=grad_mean,
               n_terms=nk)
    check_grad(gv[:, :, krows], rdv[:, :, krows], adv[:, :, krows], dtype, "dv", check_mean=grad_mean,
               n_terms=nk)
    # rows no block touches are zero, including key rows of other ranks
    for g, touched in ((gq, rows), (gk, krows), (gv, krows)):
        assert np.all(g[:, :, np.setdiff1d(np.arange(N), touched)] == 0)


# packed documents (the striped-attention page's document-packing practice):
# schedule kind, N, P, stripe, batch, Hq, Hkv, d, subset rank, document lengths
DOC_CASES = [
    (BAL, 2048, 4, 1, 1, 2, 1, 128, None, (1, 700)),
    (RING, 1024, 4, 1, 2, 2, 2, 64, None, (64, 64)),      # boundaries on tile edges
    (RING, 1024, 4, 1, 1, 2, 2, 128, None, (63, 65)),     # boundaries next to tile edges
    (STR, 1024, 8, 1, 1, 4, 2, 128, None, (1, 300)),
    (sr.STRIPED_BLOCK, 2048, 4, 64, 1, 2, 2, 128, None, (100, 900)),
    (BAL, 2048, 8, 1, 1, 2, 1, 128, 3, (1, 500)),          # one folded rank's share
    (BAL, 512, 2, 1, 1, 2, 2, 128, None, (1, 1)),         # every token its own document
    (BAL, 1000, 4, 1, 2, 2, 2, 128, None, (1000, 1000)),  # one document: plain causal
]


@pytest.mark.parametrize("case,dtype", with_dtypes(DOC_CASES, lambda c: True))
def test_document_mask_parity(dfa, case, dtype):
    from long_context_sequence_dfa_amd import inputs
    kind, N, P, stripe, B, Hq, Hkv, D, sub, (lmin, lmax) = case
    docs = inputs.doc_bounds(5000 + N + P, N, lmin, lmax)
    say(f"case: documents {sr.KIND_NAMES[kind]} N={N} P={P} stripe={stripe} B={B} Hq={Hq} "
        f"Hkv={Hkv} D={D} rank={sub} docs={len(docs) - 1} {dtype}")
    if kind == sr.STRIPED_BLOCK:
        blocks = dfa.dfa_schedule_build_striped_blocks(N, P, stripe)
    else:
        blocks = dfa.dfa_schedule_build(kind, N, P)
    if sub is not None:
        blocks = blocks[blocks[:, 0] == sub]
    seed = 5000 + N + P
    (q, k, v, _), (tq, tk, tv, _) = make(seed, B, N, Hq, Hkv, D, dtype)
    td = torch.tensor(docs, dtype=torch.int32, device="cuda")
    for b in blocks[:4]:  # single-block partials under the document mask
        op, lp = dfa.dfa_attn_block_fwd(tq, tk, tv, b, docs=td)
        torch.cuda.synchronize()
        xo, xl = oracle.block_partial(q, k, v, 1 / np.sqrt(D), *b[3:8], run=b[10], docs=docs)
        xa, _ = oracle.block_partial(q, k, np.abs(v), 1 / np.sqrt(D), *b[3:8], run=b[10], docs=docs)
        check_out(to_np(op), xo, to_np(lp), xl, dtype, f"block {b[:3]}", oabs=xa, n_keys=N)
    check_schedule(dfa, blocks, seed, N, B, Hq, Hkv, D, dtype, docs=docs)


def test_block_partials_bf16_with_empty_rows(dfa):
    """A striped block whose key shard comes after the query shard (shifted
    diagonal): local row 0 sees no key and must come out as (0, -inf)."""
    say("case: striped bf16 block partials N=512 P=4")
    N, P, D = 512, 4, 128
    (q, k, v, _), (tq, tk, tv, _) = make(3001, 1, N, 2, 2, D, "bf16")
    scale = 1 / np.sqrt(D)
    blocks = dfa.dfa_schedule_build(STR, N, P)
    for b in blocks[:8]:
        op, lp = dfa.dfa_attn_block_fwd(tq, tk, tv, b)
        torch.cuda.synchronize()
        xo, xl = oracle.block_partial(q, k, v, scale, *b[3:8])
        xa, _ = oracle.block_partial(q, k, np.abs(v), scale, *b[3:8])
        check_out(to_np(op), xo, to_np(lp), xl, "bf16", f"block {b[:3]}", oabs=xa, n_keys=N)
        if b[2] > b[0]:
            assert np.all(np.isneginf(to_np(lp)[:, :, 0]))


def test_merge_kernel_against_oracle(dfa):
    say("case: lse merge kernel")
    rng = np.random.default_rng(5)
    n, D = 1000, 128
    ao, po = rng.standard_normal((n, D)), rng.standard_normal((n, D))
    al, pl = rng.standard_normal(n) * 3, rng.standard_normal(n) * 3
    al[:10] = -np.inf
    pl[5:15] = -np.inf
    ta, tla = torch.tensor(ao, dtype=torch.float32, device="cuda"), torch.tensor(al, dtype=torch.float32, device="cuda")
    tp, tlp = torch.tensor(po, dtype=torch.float32, device="cuda"), torch.tensor(pl, dtype=torch.float32, device="cuda")
    # the oracle gets the same fp32 values
    ao32, al32 = ta.cpu().double().numpy(), tla.cpu().double().numpy()
    po32, pl32 = tp.cpu().double().numpy(), tlp.cpu().double().numpy()
    ro, rl = oracle.merge(np.stack([ao32, po32]), np.stack([al32, pl32]))
    dfa.dfa_lse_merge(ta, tla, tp, tlp)
    torch.cuda.synchronize()
    # rows 0-9: -inf accumulator takes the part; rows 5-9 both empty stay (0, -inf)
    check_out(to_np(ta), ro, to_np(tla), rl, "f32", "merge")


# score jumps: every query shares a component u and the keys carry a
# multiple of it that rises in steps along the sequence (plateaus of 20, 40,
# 60 and 80 in log2 units above the first keys), so a row's maximum score
# grows far beyond the rescale threshold at each step -- inside unmasked
# tiles as well as on the diagonal -- and its reference has to be raised
# mid-sequence.  Plateaus rather than single keys keep the softmax spread
# over many keys (no near-one-hot rows).  The outputs are held to the usual
# bounds.  For the bf16 gradients only the elementwise bound applies: the
# large shared components cancel exactly in dQ = scale sum_j dS_ij k_j (the
# dS of a row sum to zero) and in dK, so the true gradients are small
# against their terms; a float64 emulation of the kernels' bf16 roundings
# alone misses the mean bound by 100x on these inputs (dQ mean error 0.2
# rms, tests/test_tolerance.py), while the elementwise bound scales with the
# terms and holds.
# bf16 only: the fp32 path's gradient bound is relative to rms alone, which
# the same cancellation puts out of reach of any fp32 summation.
@pytest.mark.parametrize("dtype", ["bf16"])
@pytest.mark.parametrize("kind", [BAL, STR])
def test_rising_score_jumps(dfa, kind, dtype):
    from long_context_sequence_dfa_amd import inputs
    N, P, B, Hq, Hkv, D = 1024, 4, 1, 2, 1, 128
    say(f"case: score jumps {sr.KIND_NAMES[kind]} N={N} P={P} {dtype}")
    q, k, v, do = inputs.workload_tensors(3010, B, N, Hq, Hkv, D, dtype, 1 / np.sqrt(D), with_do=True)
    rnd = inputs.normal_tensor(3011, 0, (D,), "f32")
    u = (rnd / np.linalg.norm(rnd)).astype(np.float32)
    scale = 1 / np.sqrt(D)
    a = 2.0  # shared query component: a key carrying c*u scores about a*c*scale more
    q = q + a * u
    for n, (lo, hi) in enumerate(((150, 333), (333, 600), (600, 901), (901, N))):
        level = (n + 1) * 20.0 / np.log2(np.e)  # natural-log units
        k[:, lo:hi] = k[:, lo:hi] + (level / (a * scale)) * u
    exact = inputs.round_bf16 if dtype == "bf16" else (lambda x: np.asarray(x, np.float32))
    q, k = exact(q), exact(k)
    blocks = dfa.dfa_schedule_build(kind, N, P)
    check_schedule(dfa, blocks, 0, N, B, Hq, Hkv, D, dtype, arrays=(q, k, v, do), grad_mean=False)


def test_empty_block_list_and_tiny_sequences(dfa):
    say("case: empty block list, N=1, N=8 striped")
    (q, k, v, do), (tq, tk, tv, tdo) = make(3002, 1, 64, 2, 1, 64, "bf16")
    empty = np.zeros((0, 10), dtype=np.int64)
    o, lse = dfa.dfa_attn_fwd(tq, tk, tv, empty)
    dq, dk, dv = dfa.dfa_attn_bwd(tq, tk, tv, o, tdo, lse, empty)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)
    for kind, N, P in ((RING, 1, 1), (STR, 8, 4), (BAL, 8, 4), (STR, 4, 4)):
        (q, k, v, do), (tq, tk, tv, tdo) = make(3003, 1, N, 2, 1, 128, "bf16")
        blocks = dfa.dfa_schedule_build(kind, N, P)
        o, lse = dfa.dfa_attn_fwd(tq, tk, tv, blocks)
        dq, dk, dv = dfa.dfa_attn_bwd(tq, tk, tv, o, tdo, lse, blocks)
        torch.cuda.synchronize()
        scale = 1 / np.sqrt(128)
        ro, rl = oracle.attn_rows(q, k, v, scale)
        ra, _ = oracle.attn_rows(q, k, np.abs(v), scale)
        check_out(bhnd(to_np(o)), ro, to_np(lse), rl, "bf16", f"tiny {kind} {N} {P}", oabs=ra, n_keys=N)
        (rdq, rdk, rdv), (a1, a2, a3) = oracle.attn_grads(q, k, v, do, scale, with_abs=True)
        # the elementwise bound only: on 1-8 tokens the mean error over a few
        # hundred elements follows which roundings happen -- an emulation of
        # the kernels' roundings puts it on both sides of 2e-3 rms depending
        # on the (equally exact) softmax reference (tests/test_tolerance.py)
        check_grad(bhnd(to_np(dq)), rdq, a1, "bf16", "dq", check_mean=False)
        check_grad(bhnd(to_np(dk)), rdk, a2, "bf16", "dk", check_mean=False)
        check_grad(bhnd(to_np(dv)), rdv, a3, "bf16", "dv", check_mean=False)


def test_deterministic_forward_and_backward(dfa):
    """No atomics anywhere: two runs give identical bits."""
    say("case: determinism N=2048 balanced P=8 GQA")
    (q, k, v, do), (tq, tk, tv, tdo) = make(3004, 1, 2048, 8, 2, 128, "bf16")
    blocks = dfa.dfa_schedule_build(BAL, 2048, 8)
    o1, l1 = dfa.dfa_attn_fwd(tq, tk, tv, blocks)
    g1 = dfa.dfa_attn_bwd(tq, tk, tv, o1, tdo, l1, blocks)
    o2, l2 = dfa.dfa_attn_fwd(tq, tk, tv, blocks)
    g2 = dfa.dfa_attn_bwd(tq, tk, tv, o2, tdo, l2, blocks)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_strided_views(dfa):
    """Tensors that are views with non-packed strides ([B, H, N, d] storage
    seen as [B, N, H, d])."""
    say("case: strided views")
    N, H, D = 512, 2, 128
    (q, k, v, do), _ = make(3005, 1, N, H, H, D, "bf16")
    dev = torch.device("cuda")

    def strided(x):
        t = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).to(torch.bfloat16).to(dev)
        return t.permute(0, 2, 1, 3)  # logical [B, N, H, d], storage [B, H, N, d]

    tq, tk, tv, tdo = strided(q), strided(k), strided(v), strided(do)
    blocks = dfa.dfa_schedule_build(BAL, N, 2)
    o = torch.empty_like(tq)  # same strides as q
    o, lse = dfa.dfa_attn_fwd(tq, tk, tv, blocks, o=o)
    dq, dk, dv = dfa.dfa_attn_bwd(tq, tk, tv, o, tdo, lse, blocks,
                                  dq=torch.empty_like(tq), dk=torch.empty_like(tk), dv=torch.empty_like(tv))
    torch.cuda.synchronize()
    scale = 1 / np.sqrt(D)
    ro, rl = oracle.attn_rows(q, k, v, scale)
    ra, _ = oracle.attn_rows(q, k, np.abs(v), scale)
    check_out(bhnd(to_np(o)), ro, to_np(lse), rl, "bf16", "strided", oabs=ra, n_keys=N)
    (rdq, rdk, rdv), (a1, a2, a3) = oracle.attn_grads(q, k, v, do, scale, with_abs=True)
    check_grad(bhnd(to_np(dq)), rdq, a1, "bf16", "dq")
    check_grad(bhnd(to_np(dk)), rdk, a2, "bf16", "dk")
    check_grad(bhnd(to_np(dv)), rdv, a3, "bf16", "dv")


# every head of each full-size workload's head layout and schedule, at a
# length whose every row the oracle affords (N = 2048): name, kind, P,
# stripe, Hq, Hkv, inputs scaled by 1/sqrt(d), subset rank
ALL_HEADS = [
    ("llama7b-balanced-p8", BAL, 8, 1, 32, 32, True, None),
    ("llama7b-striped-p16-rank0", STR, 16, 1, 32, 32, False, 0),
    ("gqa-32-8-balanced-p32", BAL, 32, 1, 32, 8, False, None),   # chunks of 32 rows
    ("llama7b-striped64-p8", sr.STRIPED_BLOCK, 8, 64, 32, 32, True, None),
]


@pytest.mark.parametrize("case", ALL_HEADS, ids=[c[0] for c in ALL_HEADS])
def test_all_heads_at_workload_shapes(dfa, case):
    """Fused and stepwise forward and the backward on all 32 query heads
    (d = 128, bf16) of a workload's head layout and schedule, every row and
    key row the blocks touch against the oracle (the full-size tests sample
    heads and rows)."""
    from long_context_sequence_dfa_amd import inputs
    name, kind, P, stripe, Hq, Hkv, scaled, sub = case
    N, D = 2048, 128
    say(f"case: all heads {name} N={N}")
    if kind == sr.STRIPED_BLOCK:
        blocks = dfa.dfa_schedule_build_striped_blocks(N, P, stripe)
    else:
        blocks = dfa.dfa_schedule_build(kind, N, P)
    if sub is not None:
        blocks = blocks[blocks[:, 0] == sub]
    arrays = inputs.workload_tensors(5000 + P, 1, N, Hq, Hkv, D, "bf16", 1 / np.sqrt(D) if scaled else None,
                                     with_do=True)
    check_schedule(dfa, blocks, None, N, 1, Hq, Hkv, D, "bf16", arrays=arrays)


def random_cases(seed=7070, count=40):
    """Seeded random schedules: kind, ranks, length (a multiple of what the
    kind needs, ragged against the 64/256-row tiles), batch, heads, head_dim,
    dtype, a random non-empty set of whole ranks (each rank's blocks cover
    its rows completely) and sometimes packed documents."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        kind = int(rng.choice([RING, BAL, STR, sr.STRIPED_BLOCK]))
        P = int(rng.integers(1, 13))
        stripe = int(rng.choice([64, 128])) if kind == sr.STRIPED_BLOCK else 1
        unit = {BAL: 2 * P, sr.STRIPED_BLOCK: P * stripe}.get(kind, P)
        N = unit * int(rng.integers(max(1, 96 // unit), max(2, 1600 // unit) + 1))
        Hq, Hkv = [(1, 1), (2, 1), (4, 2), (3, 3), (4, 1)][int(rng.integers(0, 5))]
        B = int(rng.integers(1, 3))
        D = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.3 else "bf16"
        ranks = sorted(int(r) for r in rng.choice(P, size=int(rng.integers(1, P + 1)), replace=False))
        docs = None
        if rng.random() < 0.35:
            lo = int(rng.integers(1, 200))
            docs = (lo, lo + int(rng.integers(0, 600)))
        out.append(pytest.param((kind, N, P, stripe, B, Hq, Hkv, D, dtype, ranks, docs, 7000 + i),
                                id=f"r{i}-{sr.KIND_NAMES[kind]}-N{N}-P{P}-{dtype}"))
    return out


@pytest.mark.parametrize("case", random_cases())
def test_random_schedules(dfa, case):
    """Parity on seeded random schedules, rank sets, shapes and dtypes (fused
    and stepwise forward, backward, untouched rows zero)."""
    from long_context_sequence_dfa_amd import inputs
    kind, N, P, stripe, B, Hq, Hkv, D, dtype, ranks, doclens, seed = case
    docs = None if doclens is None else inputs.doc_bounds(seed, N, *doclens)
    say(f"case: random {sr.KIND_NAMES[kind]} N={N} P={P} stripe={stripe} B={B} Hq={Hq} Hkv={Hkv} D={D} "
        f"{dtype} ranks={ranks} docs={None if docs is None else len(docs) - 1}")
    if kind == sr.STRIPED_BLOCK:
        blocks = dfa.dfa_schedule_build_striped_blocks(N, P, stripe)
    else:
        blocks = dfa.dfa_schedule_build(kind, N, P)
    blocks = blocks[np.isin(blocks[:, 0], ranks)]
    check_schedule(dfa, blocks, seed, N, B, Hq, Hkv, D, dtype, docs=docs)
