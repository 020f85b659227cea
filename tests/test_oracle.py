"""Pins of the fp64 oracle against facts fixed outside it: a library routine
(torch's causal scaled-dot-product attention and autograd in float64), closed
forms, finite differences and invariants stated by the pages.

Each pin targets a plausible mistake: a wrong mask edge (j < i vs j <= i),
a dropped D term, a transposed operand, a wrong scale, a wrong head mapping
or a wrong merge weight would fail at least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import schedule_ref as sr

RNG = np.random.default_rng(1234)


def rand(*shape):
    return RNG.standard_normal(shape)


def sdpa_ref(q, k, v, scale):
    """torch causal attention in float64 on the CPU: o [B, Hq, N, d]."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)


@pytest.mark.parametrize("B,N,Hq,Hkv,d", [(1, 1, 1, 1, 4), (2, 17, 2, 1, 8), (1, 64, 4, 2, 16)])
def test_matches_torch_causal_sdpa(orc, B, N, Hq, Hkv, d):
    q, k, v = rand(B, N, Hq, d), rand(B, N, Hkv, d), rand(B, N, Hkv, d)
    scale = 1 / np.sqrt(d)
    o, lse = orc.attn_rows(q, k, v, scale)
    ref = sdpa_ref(q, k, v, scale).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # LSE against torch.logsumexp of the masked score matrix
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    s = tq @ tk.transpose(-1, -2) * scale
    s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,N,Hq,Hkv,d", [(1, 9, 1, 1, 4), (2, 20, 4, 2, 8)])
def test_gradients_match_torch_autograd(orc, B, N, Hq, Hkv, d):
    q, k, v, do = rand(B, N, Hq, d), rand(B, N, Hkv, d), rand(B, N, Hkv, d), rand(B, N, Hq, d)
    scale = 0.37
    dq, dk, dv = orc.attn_grads(q, k, v, do, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    g = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(g, 1),
        tv.permute(0, 2, 1, 3).repeat_interleave(g, 1), is_causal=True, scale=scale)
    (o * torch.from_numpy(do).permute(0, 2, 1, 3)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)


def test_zero_keys_give_prefix_mean(orc):
    # all scores 0: O_i = mean of v_0..v_i and LSE_i = ln(i+1) (inclusive diagonal)
    N, d = 23, 6
    q, k, v = rand(1, N, 1, d), np.zeros((1, N, 1, d)), rand(1, N, 1, d)
    o, lse = orc.attn_rows(q, k, v, 0.5)
    prefix = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], prefix, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=1e-13, rtol=0)


def test_constant_values_and_single_token(orc):
    N, d = 11, 5
    q, k = rand(1, N, 2, d), rand(1, N, 1, d)
    o, _ = orc.attn_rows(q, k, np.full((1, N, 1, d), 2.5), 0.3)
    np.testing.assert_allclose(o, 2.5, atol=1e-13, rtol=0)
    q1, k1, v1 = rand(1, 1, 1, d), rand(1, 1, 1, d), rand(1, 1, 1, d)
    o1, l1 = orc.attn_rows(q1, k1, v1, 0.3)
    np.testing.assert_allclose(o1[0, 0, 0], v1[0, 0, 0], atol=1e-15, rtol=0)
    assert abs(l1[0, 0, 0] - 0.3 * float(q1.ravel() @ k1.ravel())) < 1e-15


def test_dominant_logit_selects_its_value(orc):
    N, d = 10, 4
    q, v = np.zeros((1, N, 1, d)), rand(1, N, 1, d)
    q[0, :, 0, 0] = 1.0
    k = np.zeros((1, N, 1, d))
    k[0, 3, 0, 0] = 1.0
    o, _ = orc.attn_rows(q, k, v, 200.0)
    # rows 0..2 cannot see key 3; rows >= 3 put all weight on it
    np.testing.assert_allclose(o[0, 0, 3:], np.repeat(v[0, 3:4, 0], N - 3, axis=0), atol=1e-12)
    assert np.abs(o[0, 0, 2] - v[0, 0:3, 0].mean(0)).max() < 1e-12


def test_linear_in_v_and_rows_independent(orc):
    N, d = 15, 4
    q, k, v1, v2 = rand(1, N, 1, d), rand(1, N, 1, d), rand(1, N, 1, d), rand(1, N, 1, d)
    o1, _ = orc.attn_rows(q, k, v1, 0.5)
    o2, _ = orc.attn_rows(q, k, v2, 0.5)
    o3, _ = orc.attn_rows(q, k, 2 * v1 - 3 * v2, 0.5)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, atol=1e-12)
    sub, _ = orc.attn_rows(q, k, v1, 0.5, rows=[14, 0, 7])
    np.testing.assert_allclose(sub[0, 0], o1[0, 0, [14, 0, 7]], atol=0, rtol=0)


def test_gqa_head_mapping_equals_repeated_heads(orc):
    N, d = 12, 4
    q, k, v, do = rand(1, N, 4, d), rand(1, N, 2, d), rand(1, N, 2, d), rand(1, N, 4, d)
    o, lse = orc.attn_rows(q, k, v, 0.5)
    kr, vr = np.repeat(k, 2, axis=2), np.repeat(v, 2, axis=2)  # heads 0,1 -> kv 0; 2,3 -> kv 1
    o2, lse2 = orc.attn_rows(q, kr, vr, 0.5)
    np.testing.assert_allclose(o, o2, atol=0)
    np.testing.assert_allclose(lse, lse2, atol=0)
    dq, dk, dv = orc.attn_grads(q, k, v, do, 0.5)
    dq2, dk2, dv2 = orc.attn_grads(q, kr, vr, do, 0.5)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(1, 2, 2, N, d).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(1, 2, 2, N, d).sum(2), atol=1e-13)


@pytest.mark.parametrize("N", [8, 12])
def test_gradients_by_central_differences(orc, N):
    d, Hq, Hkv, scale, h = 4, 2, 1, 0.45, 1e-5
    q, k, v, do = rand(1, N, Hq, d), rand(1, N, Hkv, d), rand(1, N, Hkv, d), rand(1, N, Hq, d)
    dq, dk, dv = orc.attn_grads(q, k, v, do, scale)

    def loss(q_, k_, v_):
        o, _ = orc.attn_rows(q_, k_, v_, scale)
        return float((o * do.transpose(0, 2, 1, 3)).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{k_ + "_": a for k_, a in args_p.items()})
                        - loss(**{k_ + "_": a for k_, a in args_m.items()})) / (2 * h)
        ana = g.transpose(0, 2, 1, 3)
        err = np.abs(num - ana).max() / np.abs(ana).max()
        assert err < 1e-6, (name, err)


def test_gradient_invariants_and_row_stats(orc):
    N, d = 40, 8
    q, k, v, do = rand(2, N, 4, d), rand(2, N, 2, d), rand(2, N, 2, d), rand(2, N, 4, d)
    dq, dk, dv = orc.attn_grads(q, k, v, do, 0.35)
    # softmax is shift invariant in k: sum_j dK_j = 0 per (b, kv head)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    # sum_j dV_j = sum over the group's query heads of sum_i dO_i
    dsum = do.sum(axis=1).reshape(2, 2, 2, d).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=2), dsum, atol=1e-12)
    # D_i = sum_j P_ij dP_ij equals rowsum(dO_i * O_i) (two independent routes)
    lse, dd, _ = orc.grad_rows(q, k, v, do, 0.35)
    o, lse2 = orc.attn_rows(q, k, v, 0.35)
    np.testing.assert_allclose(dd, (o * do.transpose(0, 2, 1, 3)).sum(-1), atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


def test_error_magnitudes_bound_the_gradients(orc):
    N, d = 30, 8
    q, k, v, do = rand(1, N, 2, d), rand(1, N, 1, d), rand(1, N, 1, d), rand(1, N, 2, d)
    g, a = orc.attn_grads(q, k, v, do, 0.4, with_abs=True)
    for gi, ai in zip(g, a):
        assert np.all(ai >= np.abs(gi) - 1e-12)
    # dv_abs is dv of |dO|: exact identity of the definition
    _, dv_absdo = orc.attn_grads(q, k, v, np.abs(do), 0.4)[1:]
    np.testing.assert_allclose(a[2], dv_absdo, atol=1e-12)


@pytest.mark.parametrize("kind,N,P,stripe", [(sr.RING, 24, 4, 1), (sr.BALANCED, 24, 3, 1),
                                             (sr.STRIPED, 24, 4, 1), (sr.STRIPED, 24, 6, 1),
                                             (sr.BALANCED, 16, 8, 1), (sr.RING, 7, 7, 1),
                                             (sr.STRIPED_BLOCK, 24, 3, 2), (sr.STRIPED_BLOCK, 32, 2, 4),
                                             (sr.STRIPED_BLOCK, 30, 2, 5)])
def test_merged_block_partials_equal_full_attention(orc, kind, N, P, stripe):
    """The pages' exactness claim: merging every block of any schedule gives
    monolithic causal attention (also for stripe blocks, where a block's
    visibility is no single shifted diagonal)."""
    B, Hq, Hkv, d = 2, 2, 1, 4
    q, k, v = rand(B, N, Hq, d), rand(B, N, Hkv, d), rand(B, N, Hkv, d)
    scale = 0.6
    full_o, full_l = orc.attn_rows(q, k, v, scale)
    blocks = sr.enumerate_schedule(kind, N, P, stripe)
    merged_o = np.zeros_like(full_o)
    merged_l = np.full_like(full_l, -np.inf)
    for b in blocks:
        op, lp = orc.block_partial(q, k, v, scale, b[3], b[4], b[5], b[6], b[7], b[10])
        rows = sr.positions((b[3], b[5], b[7], b[10]))
        acc_o, acc_l = merged_o[:, :, rows], merged_l[:, :, rows]
        mo, ml = orc.merge(np.stack([acc_o, op]), np.stack([acc_l, lp]))
        merged_o[:, :, rows], merged_l[:, :, rows] = mo, ml
    np.testing.assert_allclose(merged_o, full_o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(merged_l, full_l, atol=1e-12, rtol=0)


def test_merge_identity_commutes_and_associates(orc):
    n, d = 7, 3
    parts_o, parts_l = rand(3, n, d), rand(3, n)
    parts_l[1, 2] = -np.inf
    a = orc.merge(parts_o, parts_l)
    b = orc.merge(parts_o[[2, 0, 1]], parts_l[[2, 0, 1]])
    ab = orc.merge(parts_o[:2], parts_l[:2])
    c = orc.merge(np.stack([ab[0], parts_o[2]]), np.stack([ab[1], parts_l[2]]))
    for x in (b, c):
        np.testing.assert_allclose(x[0], a[0], atol=1e-13)
        np.testing.assert_allclose(x[1], a[1], atol=1e-13)
    ident = orc.merge(np.stack([np.zeros((n, d)), parts_o[0]]),
                      np.stack([np.full(n, -np.inf), parts_l[0]]))
    np.testing.assert_allclose(ident[0], parts_o[0], atol=1e-15)
    both_empty = orc.merge(np.zeros((2, n, d)), np.full((2, n), -np.inf))
    assert np.all(both_empty[0] == 0) and np.all(np.isneginf(both_empty[1]))


def test_block_with_no_visible_key_row(orc):
    # striped shard of rank 0 against the keys of rank 3 (P = 4): local row 0
    # (position 0) sees nothing; row m sees keys 0..m-1 (shifted diagonal)
    N, P, d = 16, 4, 4
    q, k, v = rand(1, N, 1, d), rand(1, N, 1, d), rand(1, N, 1, d)
    o, l = orc.block_partial(q, k, v, 0.5, 0, 3, N // P, N // P, P)
    assert np.all(o[0, 0, 0] == 0) and np.isneginf(l[0, 0, 0])
    o1, l1 = orc.attn_rows(q[:, [4]], k[:, [3]], v[:, [3]], 0.5)  # row 1 sees only key 3
    np.testing.assert_allclose(o[0, 0, 1], o1[0, 0, 0], atol=1e-15)


# ---------------------------------------------------------------------------
# Packed documents (Striped Attention Guide, "Production Deployment and Best
# Practices", item 3): a query attends only to keys of its own document.


def random_bounds(rng, n, max_len):
    """Cumulative document boundaries 0 = b0 < b1 < ... = n, lengths 1..max_len."""
    b = [0]
    while b[-1] < n:
        b.append(min(n, b[-1] + int(rng.integers(1, max_len + 1))))
    return np.array(b)


DOC_CASES = [(np.array([0, 5, 6, 19, 31]), 31), (np.array([0, 1, 2, 3, 4, 5, 6]), 6),
             (np.array([0, 40]), 40)]


@pytest.mark.parametrize("bounds,N", DOC_CASES)
def test_documents_equal_separate_sequences(orc, bounds, N):
    """Document masking gives, document by document, plain causal attention of
    that document alone (its own slice of q, k, v, positions restarting at 0)."""
    B, Hq, Hkv, d = 2, 4, 2, 8
    q, k, v = rand(B, N, Hq, d), rand(B, N, Hkv, d), rand(B, N, Hkv, d)
    o, lse = orc.attn_rows(q, k, v, 0.4, docs=bounds)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        od, ld = orc.attn_rows(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], 0.4)
        np.testing.assert_allclose(o[:, :, lo:hi], od, atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[:, :, lo:hi], ld, atol=1e-13, rtol=0)


def doc_mask(bounds, N):
    """Boolean [N, N]: key j visible to query i (same document, j <= i)."""
    did = np.searchsorted(bounds, np.arange(N), side="right") - 1
    return (did[:, None] == did[None, :]) & np.tril(np.ones((N, N), dtype=bool))


def test_documents_match_torch_sdpa_and_autograd(orc):
    B, N, Hq, Hkv, d = 1, 37, 2, 1, 8
    bounds = random_bounds(np.random.default_rng(5), N, 9)
    q, k, v, do = rand(B, N, Hq, d), rand(B, N, Hkv, d), rand(B, N, Hkv, d), rand(B, N, Hq, d)
    scale = 0.45
    mask = torch.from_numpy(doc_mask(bounds, N))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o_ref = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, 1),
        tv.permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, 1), attn_mask=mask, scale=scale)
    (o_ref * torch.from_numpy(do).permute(0, 2, 1, 3)).sum().backward()
    o, _ = orc.attn_rows(q, k, v, scale, docs=bounds)
    np.testing.assert_allclose(o, o_ref.detach().numpy(), atol=1e-12, rtol=0)
    dq, dk, dv = orc.attn_grads(q, k, v, do, scale, docs=bounds)
    np.testing.assert_allclose(dq, tq.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11, rtol=0)


def test_documents_gradients_equal_separate_sequences(orc):
    B, N, Hq, Hkv, d = 1, 29, 2, 2, 4
    bounds = np.array([0, 3, 4, 17, 29])
    q, k, v, do = rand(B, N, Hq, d), rand(B, N, Hkv, d), rand(B, N, Hkv, d), rand(B, N, Hq, d)
    dq, dk, dv = orc.attn_grads(q, k, v, do, 0.5, docs=bounds)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        s = slice(lo, hi)
        gq, gk, gv = orc.attn_grads(q[:, s], k[:, s], v[:, s], do[:, s], 0.5)
        np.testing.assert_allclose(dq[:, :, s], gq, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dk[:, :, s], gk, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dv[:, :, s], gv, atol=1e-12, rtol=0)


def test_one_token_documents_closed_form(orc):
    """Every token its own document: each query sees only its own key, so
    O = v, LSE = scale q.k, dQ = dK = 0 (dP = D) and dV = dO summed over the
    query heads of the group."""
    B, N, Hq, Hkv, d = 1, 6, 4, 2, 4
    q, k, v, do = rand(B, N, Hq, d), rand(B, N, Hkv, d), rand(B, N, Hkv, d), rand(B, N, Hq, d)
    bounds = np.arange(N + 1)
    o, lse = orc.attn_rows(q, k, v, 0.3, docs=bounds)
    g = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], v[0, :, h // g], atol=1e-15)
        np.testing.assert_allclose(lse[0, h], 0.3 * np.sum(q[0, :, h] * k[0, :, h // g], -1), atol=1e-14)
    dq, dk, dv = orc.attn_grads(q, k, v, do, 0.3, docs=bounds)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    for hk in range(Hkv):
        np.testing.assert_allclose(dv[0, hk], do[0, :, hk * g:(hk + 1) * g].sum(1), atol=1e-14)


@pytest.mark.parametrize("kind,N,P,stripe", [(sr.RING, 24, 4, 1), (sr.BALANCED, 24, 3, 1),
                                             (sr.STRIPED, 24, 4, 1), (sr.STRIPED_BLOCK, 32, 2, 4)])
def test_documents_merged_block_partials_equal_full(orc, kind, N, P, stripe):
    B, Hq, Hkv, d = 1, 2, 1, 4
    q, k, v = rand(B, N, Hq, d), rand(B, N, Hkv, d), rand(B, N, Hkv, d)
    bounds = random_bounds(np.random.default_rng(N + P), N, 7)
    full_o, full_l = orc.attn_rows(q, k, v, 0.6, docs=bounds)
    merged_o = np.zeros_like(full_o)
    merged_l = np.full_like(full_l, -np.inf)
    for b in sr.enumerate_schedule(kind, N, P, stripe):
        op, lp = orc.block_partial(q, k, v, 0.6, b[3], b[4], b[5], b[6], b[7], b[10], docs=bounds)
        rows = sr.positions((b[3], b[5], b[7], b[10]))
        mo, ml = orc.merge(np.stack([merged_o[:, :, rows], op]), np.stack([merged_l[:, :, rows], lp]))
        merged_o[:, :, rows], merged_l[:, :, rows] = mo, ml
    np.testing.assert_allclose(merged_o, full_o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(merged_l, full_l, atol=1e-12, rtol=0)


def test_document_bounds_are_validated(orc):
    q = rand(1, 5, 1, 2)
    for bad in ([0, 3], [1, 5], [0, 3, 3, 5], [0, 4, 2, 5]):
        with pytest.raises(ValueError):
            orc.attn_rows(q, q, q, 1.0, docs=bad)


# ---------------------------------------------------------------------------
# Rotary position embedding at absolute positions (Striped Attention Guide,
# "Preserving Rotary Position Embeddings (RoPE)").


def test_rope_single_pair_closed_form(orc):
    """d = 2: one pair turning by pos radians (frequency base^0 = 1)."""
    x = rand(1, 7, 1, 2)
    y = orc.rope(x, base=10000.0)
    p = np.arange(7)
    np.testing.assert_allclose(y[0, :, 0, 0], x[0, :, 0, 0] * np.cos(p) - x[0, :, 0, 1] * np.sin(p), atol=1e-15)
    np.testing.assert_allclose(y[0, :, 0, 1], x[0, :, 0, 0] * np.sin(p) + x[0, :, 0, 1] * np.cos(p), atol=1e-15)


def test_rope_frequencies_and_offset(orc):
    """d = 4, base b: pair 1 turns by pos / sqrt(b); pos_offset shifts positions."""
    x = np.zeros((1, 3, 1, 4))
    x[..., 2] = 1.0  # unit vector in pair 1
    y = orc.rope(x, base=100.0, pos_offset=5)
    ang = (5 + np.arange(3)) / 10.0
    np.testing.assert_allclose(y[0, :, 0, 2], np.cos(ang), atol=1e-15)
    np.testing.assert_allclose(y[0, :, 0, 3], np.sin(ang), atol=1e-15)
    assert np.all(y[..., :2] == 0)


def test_rope_identity_norms_inverse_relative(orc):
    B, N, H, d = 2, 40, 3, 16
    x = rand(B, N, H, d)
    y = orc.rope(x)
    np.testing.assert_allclose(y[:, 0], x[:, 0], atol=0)  # position 0: no rotation
    pn = lambda a: np.sqrt(a[..., 0::2] ** 2 + a[..., 1::2] ** 2)
    np.testing.assert_allclose(pn(y), pn(x), atol=1e-13)   # each pair keeps its length
    np.testing.assert_allclose(orc.rope(y, inverse=True), x, atol=1e-13)
    # the score depends on the distance only: positions (i, j) and (i + s, j + s)
    q, k = rand(1, 1, 1, d), rand(1, 1, 1, d)
    for i, j, sft in ((9, 4, 17), (30, 30, 5), (3, 11, 1000)):
        a = np.sum(orc.rope(q, pos_offset=i) * orc.rope(k, pos_offset=j))
        b = np.sum(orc.rope(q, pos_offset=i + sft) * orc.rope(k, pos_offset=j + sft))
        assert abs(a - b) < 1e-11


def test_round_bf16_nearest_even(orc):
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5 - 2 ** -9, 3.0e38, 1e-40])
    r = orc.round_bf16(v)
    assert list(r[:3]) == [1.0, 1.0, 1.0 + 2 ** -6]
    assert r[3] == -2.5
    assert np.all(np.isfinite(r[:4]))
    t = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(r, t)
