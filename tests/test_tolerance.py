"""The bf16 gradient tolerance against the arithmetic the kernels do (CPU).

* The oracle's error magnitudes g_abs (dq_abs, dk_abs, dv_abs), which scale
  the elementwise gradient bound, equal an independent dense computation
  of their definition (tests/bf16_emulation.py) to 1e-12, and meet closed
  forms.  An inflated magnitude (a term counted twice, a wrong index) would
  loosen every gradient check; these pins catch it.
* A float64 emulation of exactly the kernels' bf16 roundings (probabilities
  into P.V, the stored output, P into dV, dS into dK and dQ, the stored
  gradients) shows:
  - the literal bound max |dg| <= 2e-2 rms(g) fails even for the exact
    gradient merely rounded to bf16 (gradient elements reach 15-100x rms);
  - the elementwise bound |dg| <= 2e-2 rms(g) + 2^-7 g_abs holds with margin,
    and so does the mean bound mean |dg| <= 2e-3 rms(g), at the parity
    tests' sizes (so the GPU tests keep both there);
  - 2^-7 and not 2^-8: bf16's unit roundoff is 2^-8, and a token-striped
    rank share (rank 0 of 16, N = 2048) has a dV element whose two emulated
    roundings (P into dV, the stored dV) reach 1.27 times 2^-8 g_abs;
  - on 1-8 tokens the mean statistic follows the rounding pattern: with the
    references the online softmax may keep it lands on both sides of the
    bound, so the tiny-sequence GPU test keeps the elementwise bound only;
  - on the score-jump inputs (large shared components that cancel in dQ)
    the mean bound fails under the emulated roundings alone, so the GPU test
    of those inputs keeps only the elementwise bound.
"""
import math

import numpy as np
import pytest

import oracle
from long_context_sequence_dfa_amd import inputs
from tests.bf16_emulation import dense_grads, dense_magnitudes, round_bf16
from tests.parity_util import sum_invariant_bounds

G_MEAN, G_MAX, G_REL = 2e-3, 2e-2, 2.0 ** -7


def rel_err(a, b):
    scale = np.abs(b).max()
    return float(np.abs(a - b).max() / scale) if scale > 0 else float(np.abs(a).max())


def stats(g, r, a):
    """(max/rms, mean/rms, elementwise bound ratio) of g against r."""
    rms = math.sqrt(float((r ** 2).mean()))
    e = np.abs(g - r)
    ratio = float((e / (G_MAX * rms + G_REL * a)).max())
    if rms == 0:
        return 0.0, 0.0, ratio
    return float(e.max() / rms), float(e.mean() / rms), ratio


@pytest.mark.parametrize("B,N,Hq,Hkv,d,seed", [(1, 1, 2, 1, 8, 1), (1, 13, 2, 2, 8, 2),
                                               (2, 64, 4, 2, 16, 3), (1, 200, 4, 1, 32, 4)])
def test_oracle_magnitudes_equal_the_dense_definition(B, N, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal(s) for s in ((B, N, Hq, d), (B, N, Hkv, d),
                                                    (B, N, Hkv, d), (B, N, Hq, d)))
    scale = 1 / math.sqrt(d)
    (dq, dk, dv), (aq, ak, av) = oracle.attn_grads(q, k, v, do, scale, with_abs=True)
    xq, xk, xv = dense_magnitudes(q, k, v, do, scale)
    for got, want in ((aq, xq), (ak, xk), (av, xv)):
        assert rel_err(got, want) <= 1e-12
    # gradients, measured against their magnitudes (one-token rows give
    # gradients that cancel to rounding residue)
    for got, want, a in zip((dq, dk, dv), dense_grads(q, k, v, do, scale), (xq, xk, xv)):
        assert np.abs(got - want).max() <= 1e-12 * a.max()
    # a magnitude bounds its own element (triangle inequality)
    for g, a in ((dq, aq), (dk, ak), (dv, av)):
        assert np.all(np.abs(g) <= a * (1 + 1e-12) + 1e-300)


def test_magnitude_closed_forms():
    rng = np.random.default_rng(9)
    d, scale = 8, 0.3
    # one token: P = 1, dP - D = 0, so dq_abs = dk_abs = scale A |k| (q) with
    # A = sum_c |dO_c v_c|, and dv_abs = |dO|
    q, k, v, do = (rng.standard_normal((1, 1, 1, d)) for _ in range(4))
    (dq, dk, dv), (aq, ak, av) = oracle.attn_grads(q, k, v, do, scale, with_abs=True)
    A = np.abs(do * v).sum()
    np.testing.assert_allclose(aq[0, 0, 0], scale * A * np.abs(k[0, 0, 0]), rtol=1e-14, atol=0)
    np.testing.assert_allclose(ak[0, 0, 0], scale * A * np.abs(q[0, 0, 0]), rtol=1e-14, atol=0)
    np.testing.assert_allclose(av[0, 0, 0], np.abs(do[0, 0, 0]), rtol=1e-14, atol=0)
    assert np.all(dq == 0) and np.all(dk == 0)
    # dO >= 0: every term of dV is non-negative, so dv_abs is dV itself
    N = 12
    q, k, v = (rng.standard_normal((1, N, 2, d)) for _ in range(3))
    do = np.abs(rng.standard_normal((1, N, 2, d)))
    (_, _, dv), (_, _, av) = oracle.attn_grads(q, k, v, do, scale, with_abs=True)
    np.testing.assert_allclose(av, dv, rtol=1e-13, atol=0)
    # dO = 0: no gradient and no error magnitude at all
    (_, _, _), (aq, ak, av) = oracle.attn_grads(q, k, v, np.zeros_like(do), scale, with_abs=True)
    assert not aq.any() and not ak.any() and not av.any()


def workload_inputs(N, Hq, Hkv, seed, scaled):
    D = 128
    return inputs.workload_tensors(seed, 1, N, Hq, Hkv, D, "bf16",
                                   1 / math.sqrt(D) if scaled else None, with_do=True)


@pytest.mark.parametrize("N,Hq,Hkv,seed,scaled", [(1024, 2, 1, 1003, True),
                                                  (1024, 2, 2, 1005, False),
                                                  (2048, 1, 1, 1003, True)])
def test_emulated_roundings_against_the_bounds(N, Hq, Hkv, seed, scaled):
    q, k, v, do = workload_inputs(N, Hq, Hkv, seed, scaled)
    scale = 1 / math.sqrt(128)
    exact = dense_grads(q, k, v, do, scale)
    emul = dense_grads(q, k, v, do, scale, emulate=True)
    mags = dense_magnitudes(q, k, v, do, scale)
    # at these sizes the mean does not depend on which (equally exact)
    # softmax reference the forward rounds against
    for off in (2.5, 5.75):
        for g, r, a in zip(dense_grads(q, k, v, do, scale, emulate=True, ref_offset=off), exact, mags):
            assert stats(g, r, a)[1] <= G_MEAN
    literal_fails = False
    for name, g, r, a in zip(("dq", "dk", "dv"), emul, exact, mags):
        mx, mean, ratio = stats(g, r, a)
        rmx = stats(round_bf16(r), r, a)[0]
        print(f"N={N} {name}: emulated max/rms {mx:.4f} mean/rms {mean:.5f} bound ratio {ratio:.3f}; "
              f"exact rounded to bf16: max/rms {rmx:.4f}")
        assert ratio <= 0.5, (name, ratio)      # the elementwise bound, with margin
        assert mean <= G_MEAN, (name, mean)     # the stated mean bound
        literal_fails |= rmx > G_MAX
    # the stated max bound is below the rounding of the outputs themselves
    assert literal_fails


# the GPU test's tiny sequences: (kind, N, P) with seed 3003, one batch entry,
# 2 query heads sharing one key/value head, d = 128
TINY = [(0, 1, 1), (2, 8, 4), (1, 8, 4), (2, 4, 4)]
TAU = 8.0  # the forward's rescale threshold (log2 units): references up to TAU below the max


@pytest.mark.parametrize("kind,N,P", TINY)
def test_tiny_sequences_mean_statistic_follows_the_rounding_pattern(kind, N, P):
    """On 1-8 tokens a gradient element is formed from a handful of rounded
    terms, so the mean error over the few hundred elements measures which
    roundings happened, not the arithmetic: the emulated roundings with the
    references the online softmax may keep (0 to TAU below the row maximum,
    all giving the same exact result) put dQ and dK's mean error on both
    sides of 2e-3 rms -- the GPU test keeps only the elementwise bound here,
    which every reference meets with margin."""
    q, k, v, do = inputs.workload_tensors(3003, 1, N, 2, 1, 128, "bf16", with_do=True)
    scale = 1 / math.sqrt(128)
    exact = dense_grads(q, k, v, do, scale)
    mags = dense_magnitudes(q, k, v, do, scale)
    if N == 1:
        # one visible key per row: dS = 0, so dq = dk = 0 exactly, and the
        # mean check has no rms to be relative to
        assert not exact[0].any() and not exact[1].any()
        return
    means = []
    for off in np.arange(0.0, TAU, 0.125):
        emul = dense_grads(q, k, v, do, scale, emulate=True, ref_offset=off)
        row = []
        for g, r, a in zip(emul, exact, mags):
            _, mean, ratio = stats(g, r, a)
            assert ratio <= 0.5
            row.append(mean)
        means.append(row)
    means = np.array(means)
    print(f"tiny N={N}: mean/rms over references, dq {means[:, 0].min():.5f}-{means[:, 0].max():.5f}, "
          f"dk {means[:, 1].min():.5f}-{means[:, 1].max():.5f}, dv {means[:, 2].min():.5f}-"
          f"{means[:, 2].max():.5f}")
    for col in (0, 1):  # dq, dk: below and above the bound, depending on the pattern
        assert means[:, col].min() < G_MEAN < means[:, col].max()


def score_jump_inputs():
    """The GPU score-jump test's inputs: queries share a component u, keys
    carry multiples of it in plateaus 20, 40, 60, 80 log2 units high."""
    N, D = 1024, 128
    q, k, v, do = inputs.workload_tensors(3010, 1, N, 2, 1, D, "bf16", 1 / np.sqrt(D), with_do=True)
    rnd = inputs.normal_tensor(3011, 0, (D,), "f32")
    u = (rnd / np.linalg.norm(rnd)).astype(np.float32)
    scale, a = 1 / np.sqrt(D), 2.0
    q = q + a * u
    for n, (lo, hi) in enumerate(((150, 333), (333, 600), (600, 901), (901, N))):
        level = (n + 1) * 20.0 / np.log2(np.e)
        k[:, lo:hi] = k[:, lo:hi] + (level / (a * scale)) * u
    return inputs.round_bf16(q), inputs.round_bf16(k), v, do


def test_score_jumps_fail_the_mean_bound_under_emulation():
    q, k, v, do = score_jump_inputs()
    scale = 1 / math.sqrt(128)
    exact = dense_grads(q, k, v, do, scale)
    emul = dense_grads(q, k, v, do, scale, emulate=True)
    mags = dense_magnitudes(q, k, v, do, scale)
    _, mean_dq, ratio_dq = stats(emul[0], exact[0], mags[0])
    print(f"score jumps dq: mean/rms {mean_dq:.4f} bound ratio {ratio_dq:.3f}")
    # the shared components cancel in dQ: the exact gradient is small against
    # its terms, so roundings the size of the terms dwarf its rms ...
    assert mean_dq > 10 * G_MEAN
    # ... while the elementwise bound, which scales with the terms, holds
    for g, r, a in zip(emul, exact, mags):
        assert stats(g, r, a)[2] <= 0.5


def test_sum_invariant_bounds_hold_under_emulation():
    """The whole-tensor invariants the full-size GPU tests check, with the
    input-only bounds they use (sum_invariant_bounds): the emulated roundings
    stay inside them, with margin."""
    for (N, Hq, Hkv, seed, scaled) in ((2048, 2, 1, 1003, True), (1024, 4, 1, 1005, False)):
        q, k, v, do = workload_inputs(N, Hq, Hkv, seed, scaled)
        scale = 1 / math.sqrt(128)
        _, dk, dv = dense_grads(q, k, v, do, scale, emulate=True)
        bk, bv = sum_invariant_bounds(q, k, v, do, scale)
        want_v = np.asarray(do, np.float64).sum(axis=1).reshape(1, Hkv, Hq // Hkv, -1).sum(axis=2)
        rk = float((np.abs(dk.sum(axis=2)) / bk).max())
        rv = float((np.abs(dv.sum(axis=2) - want_v) / bv).max())
        print(f"N={N}: sum dK error / bound {rk:.4f}, sum dV error / bound {rv:.4f}")
        assert rk <= 0.25 and rv <= 0.25


def test_unit_roundoff_of_bf16_sets_the_elementwise_bound():
    """bf16 keeps 8 significant bits: one rounding errs by up to 2^-8
    relative (checked on the rounding itself), so a gradient element made
    of rounded terms and stored in bf16 needs 2^-7 g_abs.  Rank 0's share of
    token striping over 16 ranks (N = 2048, its query rows only, head 31 of
    the all-heads GPU case) has a dV element whose emulated roundings exceed
    2^-8 g_abs by 27 % and stay within 2^-7 g_abs."""
    # just below the midpoint between 1 and the next bf16 value 1 + 2^-7
    x = np.array([1 + 2.0 ** -8 - 2.0 ** -20])
    assert round_bf16(x)[0] == 1.0 and abs(round_bf16(x)[0] - x[0]) / x[0] > 0.99 * 2.0 ** -8
    N, P, H, D = 2048, 16, 32, 128
    q, k, v, do = inputs.workload_tensors(5000 + P, 1, N, H, H, D, "bf16", None, with_do=True)
    head = [31]
    q, k, v = (np.asarray(t[:, :, head], np.float64) for t in (q, k, v))
    do = np.array(do[:, :, head], np.float64)
    share = np.zeros(N, bool)
    share[::P] = True
    do[:, ~share] = 0.0  # the loss covers rank 0's query rows only
    scale = 1 / math.sqrt(D)
    exact = dense_grads(q, k, v, do, scale)
    emul = dense_grads(q, k, v, do, scale, emulate=True)
    mags = dense_magnitudes(q, k, v, do, scale)
    r, a = exact[2], mags[2]
    rms = math.sqrt(float((r ** 2).mean()))
    e = np.abs(emul[2] - r)
    old = float((e / (G_MAX * rms + 2.0 ** -8 * a)).max())
    new = float((e / (G_MAX * rms + G_REL * a)).max())
    print(f"rank-0 share dV: emulated error / (2e-2 rms + 2^-8 g_abs) {old:.3f}, with 2^-7: {new:.3f}")
    assert old > 1.2 and new < 0.7


@pytest.mark.parametrize("N,Hq,Hkv,seed,scaled", [(1024, 2, 1, 1003, True), (2048, 2, 2, 1005, False)])
def test_output_elementwise_bound_under_emulation(N, Hq, Hkv, seed, scaled):
    """The forward output's elementwise bound of the GPU tests
    (parity_util.o_bound_ratio: (2^-7 + 2^-12 + gamma) sum_j P_ij |v_j|)
    holds for the emulated roundings (every probability entering P.V and
    the stored output rounded to bf16) with margin, and fails for an output
    off by a relative 2^-6 -- the check sees errors far below the absolute
    2e-2 bound when the inputs are scaled by 1/sqrt(d)."""
    from tests.parity_util import o_bound_ratio
    from tests.bf16_emulation import _mask
    q, k, v, _ = workload_inputs(N, Hq, Hkv, seed, scaled)
    scale = 1 / math.sqrt(128)
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    M = _mask(N)
    for h in range(Hq):
        hk = h // (Hq // Hkv)
        S = np.where(M, scale * q[0, :, h] @ k[0, :, hk].T, -np.inf)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        ell = E.sum(axis=1, keepdims=True)
        exact = (E @ v[0, :, hk]) / ell
        emul = round_bf16((round_bf16(E) @ v[0, :, hk]) / ell)
        oabs = (E @ np.abs(v[0, :, hk])) / ell
        ratio = o_bound_ratio(emul, exact, oabs, N)
        print(f"N={N} head {h}: emulated output bound ratio {ratio:.3f}, max |dO| {np.abs(emul - exact).max():.2e}")
        assert ratio <= 0.8
        assert o_bound_ratio(exact * (1 + 2.0 ** -6), exact, oabs, N) > 1.0
