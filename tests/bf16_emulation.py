"""Test infrastructure: dense float64 attention gradients with the bf16
roundings the GPU kernels apply, and an independent dense computation of
the oracle's error magnitudes (g_abs).

Everything here is written from the definitions, with full N x N matrices
and explicit masks (no row streaming, nothing shared with the oracle or the
library), for small problems only.

Roundings emulated (each to bf16, nearest even, through fp32):
  forward  : every probability entering P.V (taken against the row maximum),
             and the output O;
  backward : D is formed from the bf16 output; P enters dV = P^T dO as bf16,
             dS = P (dP - D) enters dK = scale dS^T Q and dQ = scale dS K as
             bf16; the three gradients are stored as bf16.
Accumulations are exact (float64): the fp32 accumulation error of the
kernels is second order next to these roundings.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x):
    """float64 -> fp32 -> bf16 (nearest even), as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _mask(N):
    return np.tril(np.ones((N, N), dtype=bool))


def _heads(q, k):
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    return B, N, Hq, Hkv, d, Hq // Hkv


def dense_grads(q, k, v, do, scale, emulate=False, ref_offset=0.0):
    """Gradients of L = sum_i dO_i . O_i for causal attention over every row.

    q, do: [B, N, Hq, d]; k, v: [B, N, Hkv, d] (float64 holding bf16 values).
    Returns dq [B, Hq, N, d], dk, dv [B, Hkv, N, d]; with ``emulate`` the
    kernels' bf16 roundings (module docstring) are applied, otherwise the
    result is the exact float64 gradient.  ``ref_offset`` (log2 units, >= 0):
    the forward's probabilities are rounded as 2^(s c - m) with a reference
    m that many units below the row maximum -- the online softmax may keep an
    older reference up to its rescale threshold below the maximum, which
    changes which bf16 roundings happen but not the exact result."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, N, Hq, Hkv, d, group = _heads(q, k)
    M = _mask(N)
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    rnd = round_bf16 if emulate else (lambda x: x)
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            Q, K, V, dO = q[b, :, h], k[b, :, hk], v[b, :, hk], do[b, :, h]
            S = np.where(M, scale * Q @ K.T, -np.inf)
            mx = S.max(axis=1, keepdims=True)
            E = np.exp(S - mx + ref_offset * np.log(2.0))  # against the reference
            ell = E.sum(axis=1, keepdims=True)
            lse = mx - ref_offset * np.log(2.0) + np.log(ell)
            O = rnd((rnd(E) @ V) / ell)             # the forward's stored output
            P = np.exp(S - lse)                     # recomputed from the saved LSE
            D = (dO * O).sum(axis=1, keepdims=True)
            dP = dO @ V.T
            dS = np.where(M, P * (dP - D), 0.0)
            dv[b, hk] += rnd(P).T @ dO
            dk[b, hk] += scale * rnd(dS).T @ Q
            dq[b, h] = rnd(scale * rnd(dS) @ K)
    if emulate:
        dk, dv = round_bf16(dk), round_bf16(dv)
    return dq, dk, dv


def dense_magnitudes(q, k, v, do, scale):
    """The error magnitudes of each gradient element: the sum of the absolute
    values of the terms that form it, with the D term of dS counted through
    A_i = sum_c |dO_ic O_ic| (D_i is a sum of those products):
      dq_abs[i, c] = scale sum_j P_ij (|dP_ij - D_i| + A_i) |k_jc|
      dk_abs[j, c] = scale sum_i P_ij (|dP_ij - D_i| + A_i) |q_ic|   (over the group)
      dv_abs[j, c] = sum_i P_ij |dO_ic|                                (over the group)
    Dense float64; the same layouts as dense_grads."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, N, Hq, Hkv, d, group = _heads(q, k)
    M = _mask(N)
    aq = np.zeros((B, Hq, N, d))
    ak = np.zeros((B, Hkv, N, d))
    av = np.zeros((B, Hkv, N, d))
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            Q, K, V, dO = q[b, :, h], k[b, :, hk], v[b, :, hk], do[b, :, h]
            S = np.where(M, scale * Q @ K.T, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O = P @ V
            dP = dO @ V.T
            D = (P * dP).sum(axis=1, keepdims=True)
            A = np.abs(dO * O).sum(axis=1, keepdims=True)
            W = np.where(M, P * (np.abs(dP - D) + A), 0.0)
            aq[b, h] = scale * W @ np.abs(K)
            ak[b, hk] += scale * W.T @ np.abs(Q)
            av[b, hk] += P.T @ np.abs(dO)
    return aq, ak, av
