"""fp64 CPU oracle for blockwise exact causal attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``long_context_sequence_dfa_amd`` and the library never calls it.

* ``oracle.c`` (compiled here with gcc + OpenMP) holds the attention maths:
  full causal attention rows (O1), one block's partial result (O2), the merge
  of partials (O3) and the two halves of the gradient (O5).
  It also holds the rotary position embedding at absolute positions (O6).
* ``schedule_ref.py`` enumerates the virtual-rank schedules by brute force.

Every array argument is float64; inputs are the exact stored values of the
tensors the GPU reads, widened to double.  Layout: q, dO [B, N, Hq, d];
k, v [B, N, Hkv, d].
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc -O2 -fopenmp)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            i64, f64, p = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
            lib.orc_attn_rows.argtypes = [i64] * 5 + [f64] + [p] * 3 + [i64, p, i64, p, p, p, p]
            lib.orc_block_partial.argtypes = [i64] * 5 + [f64] + [p] * 3 + [i64] * 6 + [p, p, p]
            lib.orc_merge.argtypes = [i64, i64, i64, p, p, p, p]
            lib.orc_grad_rows.argtypes = [i64] * 5 + [f64] + [p] * 4 + [i64, p, i64, p] + [p] * 6
            lib.orc_grad_cols.argtypes = ([i64] * 5 + [f64] + [p] * 4 + [i64, p, p, p]
                                          + [i64, p, i64, p, p, p, p, p, p, p])
            lib.orc_rope.argtypes = [i64] * 4 + [p, p, i64, f64, ctypes.c_int]
            for f in ("orc_attn_rows", "orc_block_partial", "orc_merge", "orc_grad_rows",
                      "orc_grad_cols", "orc_num_threads", "orc_rope"):
                getattr(lib, f).restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64).reshape(-1))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _dims(q, k):
    B, N, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if (B, N, d) != (Bk, Nk, dk):
        raise ValueError("q and k shapes disagree")
    return B, N, Hq, Hkv, d


def doc_ids(bounds, n):
    """Document id of each of the n positions for packed documents given by
    their cumulative boundaries (0 = bounds[0] < bounds[1] < ... = n):
    positions [bounds[t], bounds[t+1]) form document t."""
    b = [int(x) for x in np.asarray(bounds).reshape(-1)]
    if len(b) < 2 or b[0] != 0 or b[-1] != n or any(b[t + 1] <= b[t] for t in range(len(b) - 1)):
        raise ValueError("document bounds must rise strictly from 0 to N")
    ids = np.empty(n, dtype=np.int64)
    for t in range(len(b) - 1):
        ids[b[t]:b[t + 1]] = t
    return ids


def _doc_arg(docs, n):
    """(keep-alive array, pointer) for an optional document-bounds argument."""
    if docs is None:
        return None, ctypes.c_void_p(0)
    ids = doc_ids(docs, n)
    return ids, _ptr(ids)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def attn_rows(q, k, v, scale, rows=None, heads=None, docs=None):
    """O1: causal attention for query rows ``rows`` (global positions) and
    query heads ``heads``; ``docs``: optional cumulative document boundaries
    (attention stays inside each document).  Returns o [B, n_heads, n_rows, d],
    lse [B, n_heads, n_rows]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, Hq, Hkv, d = _dims(q, k)
    keep, dp = _doc_arg(docs, N)
    rows = _i64(np.arange(N) if rows is None else rows)
    heads = _i64(np.arange(Hq) if heads is None else heads)
    o = np.zeros((B, heads.size, rows.size, d))
    lse = np.zeros((B, heads.size, rows.size))
    _check(_load().orc_attn_rows(B, N, Hq, Hkv, d, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                 rows.size, _ptr(rows), heads.size, _ptr(heads), _ptr(o), _ptr(lse),
                                 dp), "attn_rows")
    return o, lse


def block_partial(q, k, v, scale, q_start, kv_start, len_q, len_kv, stride, run=1, docs=None):
    """O2: one block's normalised partial.  Local row i of either piece sits at
    start + (i // run) * stride + i % run.  ``docs`` as in attn_rows.
    Returns o [B, Hq, len_q, d], lse [B, Hq, len_q]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, Hq, Hkv, d = _dims(q, k)
    keep, dp = _doc_arg(docs, N)
    o = np.zeros((B, Hq, len_q, d))
    lse = np.zeros((B, Hq, len_q))
    _check(_load().orc_block_partial(B, N, Hq, Hkv, d, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                     int(q_start), int(kv_start), int(len_q), int(len_kv),
                                     int(stride), int(run), _ptr(o), _ptr(lse), dp), "block_partial")
    return o, lse


def merge(o_parts, lse_parts):
    """O3: merge partials.  o_parts [n_parts, ..., d], lse_parts [n_parts, ...]
    (the same row layout in every part).  Returns (o, lse) without the part axis."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    n_parts = o_parts.shape[0]
    d = o_parts.shape[-1]
    row_shape = lse_parts.shape[1:]
    n_rows = int(np.prod(row_shape)) if len(row_shape) else 1
    if o_parts.shape[1:-1] != row_shape:
        raise ValueError("o_parts and lse_parts disagree")
    o = np.zeros(row_shape + (d,))
    lse = np.zeros(row_shape)
    _check(_load().orc_merge(n_parts, n_rows, d, _ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse)),
           "merge")
    return o, lse


def grad_rows(q, k, v, dout, scale, rows=None, heads=None, with_abs=False, docs=None):
    """O5 row half.  Returns lse, D [B, n_heads, n_rows] and dq [B, n_heads, n_rows, d];
    with ``with_abs`` also A [B, n_heads, n_rows] and dq_abs like dq (the
    rounding-error magnitudes tests use for tolerances).  ``docs`` as in attn_rows."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, N, Hq, Hkv, d = _dims(q, k)
    keep, dp = _doc_arg(docs, N)
    rows = _i64(np.arange(N) if rows is None else rows)
    heads = _i64(np.arange(Hq) if heads is None else heads)
    lse = np.zeros((B, heads.size, rows.size))
    dd = np.zeros((B, heads.size, rows.size))
    dq = np.zeros((B, heads.size, rows.size, d))
    aa = np.zeros((B, heads.size, rows.size)) if with_abs else None
    dq_abs = np.zeros((B, heads.size, rows.size, d)) if with_abs else None
    nul = ctypes.c_void_p(0)
    _check(_load().orc_grad_rows(B, N, Hq, Hkv, d, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(dout), rows.size, _ptr(rows), heads.size, _ptr(heads),
                                 _ptr(lse), _ptr(dd), _ptr(dq),
                                 _ptr(aa) if with_abs else nul,
                                 _ptr(dq_abs) if with_abs else nul, dp), "grad_rows")
    if with_abs:
        return lse, dd, dq, aa, dq_abs
    return lse, dd, dq


def grad_cols(q, k, v, dout, scale, rows, lse, dd, keys=None, kv_heads=None, aa=None, docs=None):
    """O5 column half.  ``lse`` and ``dd`` (and ``aa`` if given) are
    [B, Hq, n_rows] for the row set ``rows`` (every query head).  Returns
    dk, dv [B, n_kv_heads, n_keys, d], plus dk_abs, dv_abs when ``aa`` is given.
    ``docs`` as in attn_rows (and as given to grad_rows for lse, dd)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, N, Hq, Hkv, d = _dims(q, k)
    keep, dp = _doc_arg(docs, N)
    rows = _i64(rows)
    lse, dd = _f64(lse), _f64(dd)
    if lse.shape != (B, Hq, rows.size) or dd.shape != lse.shape:
        raise ValueError("lse/D must be [B, Hq, n_rows]")
    keys = _i64(np.arange(N) if keys is None else keys)
    kv_heads = _i64(np.arange(Hkv) if kv_heads is None else kv_heads)
    dk = np.zeros((B, kv_heads.size, keys.size, d))
    dv = np.zeros((B, kv_heads.size, keys.size, d))
    nul = ctypes.c_void_p(0)
    if aa is not None:
        aa = _f64(aa)
        if aa.shape != lse.shape:
            raise ValueError("aa must be [B, Hq, n_rows]")
        dk_abs, dv_abs = np.zeros_like(dk), np.zeros_like(dv)
    _check(_load().orc_grad_cols(B, N, Hq, Hkv, d, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(dout), rows.size, _ptr(rows), _ptr(lse), _ptr(dd),
                                 keys.size, _ptr(keys), kv_heads.size, _ptr(kv_heads),
                                 _ptr(dk), _ptr(dv),
                                 _ptr(aa) if aa is not None else nul,
                                 _ptr(dk_abs) if aa is not None else nul,
                                 _ptr(dv_abs) if aa is not None else nul, dp), "grad_cols")
    if aa is not None:
        return dk, dv, dk_abs, dv_abs
    return dk, dv


def attn_grads(q, k, v, dout, scale, rows=None, with_abs=False, docs=None):
    """Full O5 for the query row set ``rows`` (default: every row): the loss is
    sum over those rows of dO.O.  Returns dq [B, Hq, n_rows, d] and
    dk, dv [B, Hkv, N, d]; with ``with_abs`` a second tuple of the matching
    rounding-error magnitudes (dq_abs, dk_abs, dv_abs).  ``docs`` as in attn_rows."""
    q = _f64(q)
    B, N, Hq, d = q.shape
    rows = _i64(np.arange(N) if rows is None else rows)
    if not with_abs:
        lse, dd, dq = grad_rows(q, k, v, dout, scale, rows=rows, docs=docs)
        dk, dv = grad_cols(q, k, v, dout, scale, rows, lse, dd, docs=docs)
        return dq, dk, dv
    lse, dd, dq, aa, dq_abs = grad_rows(q, k, v, dout, scale, rows=rows, with_abs=True, docs=docs)
    dk, dv, dk_abs, dv_abs = grad_cols(q, k, v, dout, scale, rows, lse, dd, aa=aa, docs=docs)
    return (dq, dk, dv), (dq_abs, dk_abs, dv_abs)


def rope(x, base=10000.0, pos_offset=0, inverse=False):
    """O6: rotary position embedding of x [B, N, H, d] at positions
    pos_offset + token index (interleaved pairs, angle pos * base^(-2c/d));
    ``inverse`` rotates back.  Returns float64 [B, N, H, d]."""
    x = _f64(x)
    B, N, H, d = x.shape
    y = np.zeros_like(x)
    _check(_load().orc_rope(B, N, H, d, _ptr(x), _ptr(y), int(pos_offset), float(base),
                            1 if inverse else 0), "rope")
    return y


def round_bf16(x):
    """float64 -> nearest fp32 -> nearest-even bf16, returned as float64 (the
    storage rounding of a bf16 tensor written from an fp32 value)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)
