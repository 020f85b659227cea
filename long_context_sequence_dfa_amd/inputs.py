"""Seeded synthetic inputs shared by the GPU path's callers and the oracle.

This module holds no attention arithmetic: it only draws numbers.  Each
tensor is a stream of standard normals from a counter-based generator:

* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the 64-bit output for counter c of stream key s
  is mix(s + (c + 1) * 0x9E3779B97F4A7C15) with the published mix function;
* the stream key of a tensor is mix(seed * 16 + tensor_id);
* Box-Muller in fp64 turns outputs 2m and 2m+1 into normals 2m and 2m+1:
  u1 = (x_2m >> 11) * 2^-53, u2 = (x_2m+1 >> 11) * 2^-53,
  r = sqrt(-2 ln(1 - u1)), z_2m = r cos(2 pi u2), z_2m+1 = r sin(2 pi u2);
* the fp64 value is rounded to fp32; optionally multiplied (in fp32) by a
  scale; then, for bf16 tensors, rounded to bf16 (round to nearest even).

Values fill the tensor in its logical [batch, token, head, head_dim] order.
Tensor ids: Q = 0, K = 1, V = 2, dO = 3.  Seeds are 1000 + workload number.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}
_CHUNK = 1 << 22  # elements per worker chunk (even)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * M1
    z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        return _mix(np.array([seed * 16 + tensor_id], dtype=np.uint64))[0]


def _normals(key: np.uint64, start: int, count: int) -> np.ndarray:
    """fp64 normals for elements [start, start+count); start and count even."""
    pairs = np.arange(start // 2, (start + count) // 2, dtype=np.uint64)
    with np.errstate(over="ignore"):
        c1 = key + (pairs * np.uint64(2) + np.uint64(1)) * GAMMA
        c2 = key + (pairs * np.uint64(2) + np.uint64(2)) * GAMMA
        x1 = _mix(c1)
        x2 = _mix(c2)
    u1 = (x1 >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    u2 = (x2 >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    r = np.sqrt(-2.0 * np.log1p(-u1))
    th = 2.0 * np.pi * u2
    out = np.empty(count, dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def normal_tensor(seed: int, tensor_id: int, shape, dtype: str = "bf16", scale=None,
                  threads: int = 8) -> np.ndarray:
    """Seeded N(0,1) tensor of ``shape`` as fp32 values exactly representable
    in ``dtype`` ("bf16" or "f32").  ``scale`` multiplies in fp32 before the
    final rounding."""
    n = int(np.prod(shape))
    key = stream_key(seed, tensor_id)
    out = np.empty(n, dtype=np.float32)
    padded = n + (n & 1)

    def work(start):
        cnt = min(_CHUNK, padded - start)
        vals = _normals(key, start, cnt).astype(np.float32)
        if scale is not None:
            vals = vals * np.float32(scale)
        if dtype == "bf16":
            vals = round_bf16(vals)
        elif dtype != "f32":
            raise ValueError("dtype must be bf16 or f32")
        end = min(start + cnt, n)
        out[start:end] = vals[: end - start]

    starts = list(range(0, padded, _CHUNK))
    if len(starts) == 1 or threads <= 1:
        for s in starts:
            work(s)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, starts))
    return out.reshape(shape)


def to_torch(x: np.ndarray, dtype: str, device="cpu"):
    """fp32 numpy values -> torch tensor of bf16/fp32 (exact) on ``device``."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device)


def workload_tensors(seed: int, B: int, N: int, Hq: int, Hkv: int, D: int, dtype: str = "bf16",
                     qkv_scale=None, with_do: bool = False):
    """Q, K, V (and dO) of one workload as fp32 numpy arrays [B, N, H, D]."""
    q = normal_tensor(seed, 0, (B, N, Hq, D), dtype, qkv_scale)
    k = normal_tensor(seed, 1, (B, N, Hkv, D), dtype, qkv_scale)
    v = normal_tensor(seed, 2, (B, N, Hkv, D), dtype, qkv_scale)
    if not with_do:
        return q, k, v
    do = normal_tensor(seed, 3, (B, N, Hq, D), dtype)
    return q, k, v, do


DOC_STREAM_ID = 4  # stream key id of document lengths


def doc_bounds(seed: int, n: int, min_len: int, max_len: int) -> np.ndarray:
    """Cumulative boundaries of packed documents over n positions: document
    lengths drawn uniformly from [min_len, max_len] (splitmix64 output t of
    stream mix(seed * 16 + 4), length = min_len + output mod (max_len -
    min_len + 1)) until they cover n; the last document is cut at n.
    Returns int64 [0, b1, ..., n]."""
    if not (1 <= min_len <= max_len) or n < 1:
        raise ValueError("need 1 <= min_len <= max_len and n >= 1")
    key = stream_key(seed, DOC_STREAM_ID)
    span = np.uint64(max_len - min_len + 1)
    bounds, pos, t = [0], 0, 0
    while pos < n:
        with np.errstate(over="ignore"):
            x = _mix(np.array([key + np.uint64(t + 1) * GAMMA], dtype=np.uint64))[0]
        pos = min(n, pos + min_len + int(x % span))
        bounds.append(pos)
        t += 1
    return np.array(bounds, dtype=np.int64)
