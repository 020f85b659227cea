"""Shared helpers of the GPU parity tests: inputs, oracle calls and the
tolerances.

Tolerances (the stated accuracy targets, with one derived reading for bf16
gradients):
* fp32 path: |dO|, |dLSE| <= 1e-4; gradients elementwise
  |dg| <= 1e-4 rms(g) + (n + 2 d + 64) u g_abs, u = 2^-24, n the number of
  terms summed into the element (keys per row for dQ, rows times group heads
  per key for dK/dV): the textbook first-order bound of an n-term sequential
  fp32 sum, gamma_n sum |terms|, plus the error of the two d-term dot
  products (scores and dP) and of the exponential inside each term.
* bf16 path: O max |dO| <= 2e-2 and mean <= 2e-3; LSE max <= 1e-3.
* bf16 gradients: mean |dg| <= 2e-3 rms(g) as stated, and elementwise
  |dg| <= 2e-2 rms(g) + 2^-7 g_abs, where g_abs is the sum of the absolute
  values of the terms that make up the element (the oracle's magnitude
  output).  The stated max bound alone is below the bf16 rounding of the
  outputs themselves (gradient elements reach 30-100x rms).  bf16 keeps 8
  significant bits, so one rounding errs by at most u = 2^-8 relative;
  2^-7 g_abs is the first-order bound of one rounding of P or dS in every
  term (u g_abs) plus one of the output (u |g| <= u g_abs).
"""
import numpy as np

from oracle import schedule_ref as sr

import oracle

BF16_O_MAX, BF16_O_MEAN, BF16_LSE_MAX = 2e-2, 2e-3, 1e-3
F32_TOL = 1e-4
F32_U = 2.0 ** -24
G_MEAN, G_MAX, G_REL = 2e-3, 2e-2, 2.0 ** -7


def to_np(t):
    return t.float().cpu().numpy()


def bhnd(x):
    """[B, N, H, d] -> [B, H, N, d]"""
    return x.transpose(0, 2, 1, 3)


def check_out(go, ro, gl, rl, dtype, what="", oabs=None, n_keys=None):
    """go/ro [..., d] outputs, gl/rl LSE with matching leading dims.
    ``oabs`` (bf16): the output's error magnitudes sum_j P_ij |v_jc| (the
    oracle's output with |v| for v); then also elementwise
    |dO| <= (2^-7 + 2^-12 + (n + 2d + 64) 2^-24) oabs, n the key count: one
    bf16 rounding of every probability entering P.V plus one of the stored
    output (u = 2^-8 each), the fp32 score error inside the exponent
    (2^-12 covers d 2^-24 sum_c |q_c k_c| scale log2(e) for scores up to 30
    log2 units, which normal inputs of these shapes stay below) and the fp32
    sums -- a relative check that the absolute bounds cannot give when the
    inputs are scaled by 1/sqrt(d) and the outputs are small.  ``n_keys``: an
    upper bound of n (the sequence length)."""
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin), f"{what}: -inf rows differ"
    assert np.all(gl[~fin] == rl[~fin]), f"{what}: empty-row LSE"
    assert np.all(go[~fin] == 0), f"{what}: empty rows must be 0"
    eo = np.abs(go - ro)
    el = np.abs(gl[fin] - rl[fin]) if fin.any() else np.zeros(1)
    if dtype == "f32":
        assert eo.max() <= F32_TOL and el.max() <= F32_TOL, (what, eo.max(), el.max())
    else:
        assert eo.max() <= BF16_O_MAX, (what, "O max", eo.max())
        assert eo.mean() <= BF16_O_MEAN, (what, "O mean", eo.mean())
        assert el.max() <= BF16_LSE_MAX, (what, "LSE max", el.max())
        if oabs is not None:
            rel = o_bound_ratio(go, ro, oabs, n_keys)
            rms = float(np.sqrt((ro ** 2).mean()))
            print(f"{what}: O max|dO|/rms {eo.max() / rms if rms > 0 else 0.0:.4f}, "
                  f"elementwise bound ratio {rel:.3f}", flush=True)
            assert rel <= 1.0, (what, "O elementwise bound ratio", rel)
    return float(eo.max()), float(el.max())


def o_bound_ratio(go, ro, oabs, n_keys):
    """max of |go - ro| / ((2^-7 + 2^-12 + (n + 2d + 64) 2^-24) oabs); exact
    zeros where oabs is 0 (rows that see no key)."""
    e = np.abs(go - ro)
    bound = (G_REL + 2.0 ** -12 + (n_keys + 2 * ro.shape[-1] + 64) * F32_U) * oabs
    assert np.all(e[bound == 0] == 0)
    return float((e / np.where(bound > 0, bound, np.inf)).max())


def check_grad(g, r, rabs, dtype, what="", check_mean=True, n_terms=None):
    """bf16: mean and elementwise bounds; fp32: the elementwise bound with
    n_terms summed terms per element (module docstring)."""
    rms = float(np.sqrt((r ** 2).mean()))
    e = np.abs(g - r)
    if dtype == "f32":
        gamma = (n_terms + 2 * g.shape[-1] + 64) * F32_U
        bound = F32_TOL * rms + gamma * rabs
        ratio = e / np.where(bound > 0, bound, np.inf)
        assert np.all(e[bound == 0] == 0), (what, "nonzero error where every term is 0")
        assert ratio.max() <= 1.0, (what, "fp32 bound ratio", ratio.max(), "max/rms",
                                    e.max() / rms if rms > 0 else e.max())
        return float(ratio.max())
    if rms > 0 and check_mean:
        assert e.mean() <= G_MEAN * rms, (what, "mean/rms", e.mean() / rms)
    ratio = e / (G_MAX * rms + G_REL * rabs)
    assert ratio.max() <= 1.0, (what, "bound ratio", ratio.max(), "max/rms", e.max() / rms)
    return float(ratio.max())


def _run(b):
    return int(b[10]) if len(b) > 10 else 1


def rows_of(blocks):
    """Global query positions of a block list (runs as in dfa_block)."""
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate([sr.positions((b[3], b[5], b[7], _run(b))) for b in blocks]))


def kv_rows_of(blocks):
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate([sr.positions((b[4], b[6], b[7], _run(b))) for b in blocks]))


def sum_invariant_bounds(q, k, v, do, scale, rows=None):
    """Bounds on the rounding error of the whole-tensor sums sum_j dK_j (= 0)
    and sum_j dV_j (= sum_i dO_i over the rows and the group's heads), per
    batch entry, key/value head and column, from the inputs alone: the sums
    of the elementwise magnitudes times G_REL.  sum_j dv_abs_jc = sum_i |dO_ic|
    exactly (the probabilities of a row sum to 1); sum_j dk_abs_jc =
    scale sum_i |q_ic| sum_j P_ij (|dP_ij - D_i| + A_i) <= 3 scale V sum_i
    |q_ic| |dO_i|, V = max_j |v_j| (|dP_ij|, |D_i| and A_i are each at most
    |dO_i| V by Cauchy-Schwarz, O_i being an average of the v_j).  Returns
    (bound_dk, bound_dv), each [B, Hkv, d]."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if rows is not None:
        q, do = q[:, rows], do[:, rows]
    # float64 accumulation without float64 copies of full-size tensors
    vmax = np.sqrt(np.square(v, dtype=np.float64).sum(axis=3)).max(axis=1)       # [B, Hkv]
    sk = np.zeros((B, Hq, d))
    sv = np.zeros((B, Hq, d))
    for h in range(Hq):
        qh, dh = np.asarray(q[:, :, h], np.float64), np.asarray(do[:, :, h], np.float64)
        don = np.sqrt((dh ** 2).sum(axis=2, keepdims=True))                        # [B, n, 1]
        sk[:, h] = (np.abs(qh) * don).sum(axis=1)
        sv[:, h] = np.abs(dh).sum(axis=1)
    sk = sk.reshape(B, Hkv, g, d).sum(axis=2)
    sv = sv.reshape(B, Hkv, g, d).sum(axis=2)
    return G_REL * 3 * scale * vmax[:, :, None] * sk, G_REL * sv
