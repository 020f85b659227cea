"""Thin ctypes binding over libdfa.so (the C ABI in include/dfa.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the ABI.  PyTorch supplies device memory and the stream.
Functions carry the C names.  There is no CPU fallback: if libdfa.so is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdfa.so")

DFA_OK, DFA_E_NULL, DFA_E_SHAPE, DFA_E_UNSUPPORTED = 0, -1, -2, -3
DFA_E_ALIGN, DFA_E_CAPACITY, DFA_E_WORKSPACE, DFA_E_HIP = -4, -5, -6, -7
DFA_SCHED_RING, DFA_SCHED_BALANCED, DFA_SCHED_STRIPED = 0, 1, 2
DFA_F32, DFA_BF16 = 0, 1
DFA_FWD_FUSED, DFA_FWD_STEPWISE = 0, 1
DFA_OP_FWD_FUSED, DFA_OP_FWD_STEPWISE, DFA_OP_BWD = 0, 1, 2

EXPORTED = ("dfa_schedule_build", "dfa_schedule_build_striped_blocks", "dfa_schedule_balance",
            "dfa_attn_block_fwd", "dfa_lse_merge",
            "dfa_attn_fwd", "dfa_attn_fwd_slots", "dfa_attn_bwd", "dfa_attn_bwd_ex",
            "dfa_attn_bwd_noalloc", "dfa_workspace_size",
            "dfa_rope", "dfa_status_string")
BLOCK_FIELDS = ("rank", "step", "kv_rank", "q_start", "kv_start", "len_q", "len_kv", "stride",
                "diag_offset", "pairs", "run")
NB = len(BLOCK_FIELDS)


class DfaBlock(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in BLOCK_FIELDS]


class DfaAttnDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("seqlen", ctypes.c_int64),
                ("q_strides", ctypes.c_int64 * 3), ("k_strides", ctypes.c_int64 * 3),
                ("v_strides", ctypes.c_int64 * 3), ("o_strides", ctypes.c_int64 * 3),
                ("doc_bounds", ctypes.c_void_p), ("n_docs", ctypes.c_int64)]


class DfaBalance(ctypes.Structure):
    _fields_ = [("total_pairs", ctypes.c_int64), ("busy_slots", ctypes.c_int64),
                ("bubble", ctypes.c_double), ("eta_blocks", ctypes.c_double)]


class DfaKernelMarks(ctypes.Structure):
    _fields_ = [("pre_begin", ctypes.c_void_p), ("dq_begin", ctypes.c_void_p),
                ("dk_begin", ctypes.c_void_p), ("dv_begin", ctypes.c_void_p),
                ("end", ctypes.c_void_p)]


class DfaSlotMarks(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("n_ranks", ctypes.c_int32)]


class DfaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_text(status)} (status {status})")


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libdfa.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"libdfa.so is not built ({LIB_PATH}); run "
                                   "`python -c 'import __graft_entry__ as g; g.build()'`")
            L = ctypes.CDLL(LIB_PATH)
            i32, i64, p, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
            L.dfa_schedule_build.argtypes = [i32, i64, i32, p, i64, ctypes.POINTER(i64)]
            L.dfa_schedule_build_striped_blocks.argtypes = [i64, i32, i64, p, i64, ctypes.POINTER(i64)]
            L.dfa_schedule_balance.argtypes = [p, i64, i32, p, p, p]
            L.dfa_attn_block_fwd.argtypes = [p, p, p, p, p, p, p, p]
            L.dfa_lse_merge.argtypes = [i64, i32, p, p, p, p, p]
            L.dfa_attn_fwd.argtypes = [p, p, i64, i32, p, p, p, p, p, p, sz, p]
            L.dfa_attn_fwd_slots.argtypes = [p, p, i64, p, p, p, p, p, p, sz, p, p]
            L.dfa_attn_bwd.argtypes = [p, p, i64, p, p, p, p, p, p, p, p, p, p, sz, p]
            L.dfa_attn_bwd_ex.argtypes = [p, p, i64, p, p, p, p, p, p, p, p, p, p, sz, p, p]
            L.dfa_attn_bwd_noalloc.argtypes = [p, p, i64, p, p, p, p, p, p, p, p, p, p]
            L.dfa_workspace_size.argtypes = [p, p, i64, i32, ctypes.POINTER(sz)]
            L.dfa_rope.argtypes = [i32, i32, i64, i32, i32, p, p, p, p, i64, ctypes.c_double, i32, p]
            L.dfa_status_string.argtypes = [i32]
            L.dfa_status_string.restype = ctypes.c_char_p
            for f in EXPORTED[:-1]:
                getattr(L, f).restype = i32
            _lib = L
    return _lib


def status_text(status: int) -> str:
    return lib().dfa_status_string(int(status)).decode()


def dfa_status_string(status: int) -> str:
    return status_text(status)


def _check(st: int, what: str) -> None:
    if st != DFA_OK:
        raise DfaError(st, what)


# ---------------------------------------------------------------- schedules
def dfa_schedule_build(kind: int, seqlen: int, n_ranks: int) -> np.ndarray:
    """Blocks of a schedule as an int64 array [n_blocks, 11] (dfa_block fields)."""
    L = lib()
    n = ctypes.c_int64(0)
    _check(L.dfa_schedule_build(int(kind), int(seqlen), int(n_ranks), None, 0, ctypes.byref(n)),
           "dfa_schedule_build")
    out = np.zeros((n.value, NB), dtype=np.int64)
    _check(L.dfa_schedule_build(int(kind), int(seqlen), int(n_ranks),
                                out.ctypes.data_as(ctypes.c_void_p), n.value, ctypes.byref(n)),
           "dfa_schedule_build")
    return out


def dfa_schedule_build_striped_blocks(seqlen: int, n_ranks: int, stripe: int) -> np.ndarray:
    """The striped schedule with stripe blocks of ``stripe`` tokens, [n_blocks, 11]."""
    L = lib()
    n = ctypes.c_int64(0)
    _check(L.dfa_schedule_build_striped_blocks(int(seqlen), int(n_ranks), int(stripe), None, 0,
                                               ctypes.byref(n)), "dfa_schedule_build_striped_blocks")
    out = np.zeros((n.value, NB), dtype=np.int64)
    _check(L.dfa_schedule_build_striped_blocks(int(seqlen), int(n_ranks), int(stripe),
                                               out.ctypes.data_as(ctypes.c_void_p), n.value,
                                               ctypes.byref(n)), "dfa_schedule_build_striped_blocks")
    return out


def _blocks_arg(blocks) -> np.ndarray:
    """[n, 11] int64 dfa_block rows; rows without the trailing run field (10
    columns) get run = 1."""
    a = np.asarray(blocks, dtype=np.int64)
    if a.ndim == 1:
        a = a.reshape(1, -1)
    if a.shape[-1] == NB - 1:
        a = np.concatenate([a.reshape(-1, NB - 1), np.ones((a.size // (NB - 1), 1), np.int64)], axis=1)
    return np.ascontiguousarray(a.reshape(-1, NB))


def dfa_schedule_balance(blocks, n_ranks: int) -> dict:
    arr = _blocks_arg(blocks)
    rp = np.zeros(n_ranks, dtype=np.int64)
    sm = np.zeros(n_ranks, dtype=np.int64)
    bal = DfaBalance()
    _check(lib().dfa_schedule_balance(arr.ctypes.data_as(ctypes.c_void_p), arr.shape[0],
                                      int(n_ranks), rp.ctypes.data_as(ctypes.c_void_p),
                                      sm.ctypes.data_as(ctypes.c_void_p), ctypes.byref(bal)),
           "dfa_schedule_balance")
    return {"rank_pairs": rp, "step_max": sm, "total_pairs": bal.total_pairs,
            "busy_slots": bal.busy_slots, "bubble": bal.bubble, "eta_blocks": bal.eta_blocks}


# ---------------------------------------------------------------- descriptors
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DFA_BF16
    if t.dtype == torch.float32:
        return DFA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_desc(q, k, v, o=None, scale=None, docs=None) -> DfaAttnDesc:
    """Descriptor for tensors laid out [batch, token, head, head_dim].
    ``docs``: optional int32 device tensor of cumulative document boundaries
    (0 = docs[0] < ... < docs[-1] = N) for packed documents; the caller keeps
    it alive until the work has run."""
    B, N, Hq, D = q.shape
    d = DfaAttnDesc()
    if docs is not None:
        import torch
        if docs.dtype != torch.int32 or docs.dim() != 1 or not docs.is_contiguous() or docs.numel() < 2:
            raise ValueError("docs must be a contiguous 1-D int32 tensor of >= 2 boundaries")
        if docs.device != q.device:
            raise ValueError("docs must be on the tensors' device")
        d.doc_bounds = docs.data_ptr()
        d.n_docs = docs.numel() - 1
    d.dtype = _dtype_code(q)
    d.batch, d.heads_q, d.heads_kv, d.head_dim = B, Hq, k.shape[2], D
    d.seqlen = N
    d.softmax_scale = float(1.0 / math.sqrt(D) if scale is None else scale)
    for name, t in (("q_strides", q), ("k_strides", k), ("v_strides", v),
                    ("o_strides", q if o is None else o)):
        st = t.stride()
        if st[3] != 1:
            raise ValueError("head_dim must be contiguous")
        getattr(d, name)[:] = [st[0], st[1], st[2]]
    return d


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dfa_workspace_size(desc: DfaAttnDesc, blocks, op: int) -> int:
    arr = _blocks_arg(blocks)
    n = ctypes.c_size_t(0)
    _check(lib().dfa_workspace_size(ctypes.byref(desc), arr.ctypes.data_as(ctypes.c_void_p),
                                    arr.shape[0], int(op), ctypes.byref(n)), "dfa_workspace_size")
    return int(n.value)


def _workspace(desc, blocks, op, device, workspace):
    import torch
    need = dfa_workspace_size(desc, blocks, op)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel()


# ---------------------------------------------------------------- kernels
def dfa_attn_block_fwd(q, k, v, block, o_part=None, lse_part=None, scale=None, stream=None,
                       docs=None):
    """One block's normalised partial: o_part fp32 [B, Hq, len_q, d], lse_part fp32 [B, Hq, len_q]."""
    import torch
    blk = DfaBlock(*[int(x) for x in _blocks_arg(block)[0]])
    desc = make_desc(q, k, v, scale=scale, docs=docs)
    B, _, Hq, D = q.shape
    if o_part is None:
        o_part = torch.empty((B, Hq, blk.len_q, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, blk.len_q), dtype=torch.float32, device=q.device)
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("partials must be contiguous")
    _check(lib().dfa_attn_block_fwd(ctypes.byref(desc), ctypes.byref(blk), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(o_part), _ptr(lse_part), _stream(stream)),
           "dfa_attn_block_fwd")
    return o_part, lse_part


def dfa_lse_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    """In place (o_acc, lse_acc) <- merge with (o_part, lse_part); rows x head_dim fp32."""
    D = o_acc.shape[-1]
    n_rows = lse_acc.numel()
    for t in (o_acc, lse_acc, o_part, lse_part):
        if not t.is_contiguous():
            raise ValueError("merge operands must be contiguous")
    if o_acc.numel() != n_rows * D or o_part.numel() != n_rows * D or lse_part.numel() != n_rows:
        raise ValueError("merge operand sizes disagree")
    _check(lib().dfa_lse_merge(n_rows, D, _ptr(o_acc), _ptr(lse_acc), _ptr(o_part),
                               _ptr(lse_part), _stream(stream)), "dfa_lse_merge")
    return o_acc, lse_acc


def dfa_rope(x, y=None, pos_offset=0, base=10000.0, inverse=False, stream=None):
    """Rotary position embedding of x [B, N, H, d] (bf16 or fp32) at absolute
    positions pos_offset + token index; ``inverse`` turns back.  Writes y
    (default: a new tensor like x; pass y=x to rotate in place)."""
    import torch
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("x must be [B, N, H, d] with d contiguous")
    y = torch.empty_like(x) if y is None else y
    if y.shape != x.shape or y.dtype != x.dtype or y.stride(3) != 1:
        raise ValueError("y must match x")
    B, N, H, D = x.shape
    xs = (ctypes.c_int64 * 3)(*x.stride()[:3])
    ys = (ctypes.c_int64 * 3)(*y.stride()[:3])
    _check(lib().dfa_rope(_dtype_code(x), B, N, H, D, xs, _ptr(x), ys, _ptr(y), int(pos_offset),
                          float(base), 1 if inverse else 0, _stream(stream)), "dfa_rope")
    return y


def dfa_attn_fwd(q, k, v, blocks, mode=DFA_FWD_FUSED, o=None, lse=None, workspace=None,
                 scale=None, stream=None, docs=None):
    """Forward over a block list.  Returns (o [B, N, Hq, d], lse fp32 [B, Hq, N])."""
    import torch
    B, N, Hq, D = q.shape
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    desc = make_desc(q, k, v, o, scale, docs)
    arr = _blocks_arg(blocks)
    op = DFA_OP_FWD_FUSED if mode == DFA_FWD_FUSED else DFA_OP_FWD_STEPWISE
    ws, nbytes = _workspace(desc, arr, op, q.device, workspace)
    _check(lib().dfa_attn_fwd(ctypes.byref(desc), arr.ctypes.data_as(ctypes.c_void_p),
                              arr.shape[0], int(mode), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                              _ptr(lse), _ptr(ws), nbytes, _stream(stream)), "dfa_attn_fwd")
    return o, lse


def dfa_attn_fwd_slots(q, k, v, blocks, events, n_ranks, o=None, lse=None, workspace=None,
                       scale=None, stream=None, docs=None):
    """The stepwise forward launched one (rank, step) slot at a time in (step,
    rank) order; ``events`` holds n_ranks^2 + 1 hipEvent_t handles (ints or
    c_void_p): events[s * n_ranks + r] is recorded before slot (r, s) and the
    last one at the end.  Returns (o, lse)."""
    import torch
    B, N, Hq, D = q.shape
    if len(events) != n_ranks * n_ranks + 1:
        raise ValueError("need n_ranks^2 + 1 events")
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    desc = make_desc(q, k, v, o, scale, docs)
    arr = _blocks_arg(blocks)
    ws, nbytes = _workspace(desc, arr, DFA_OP_FWD_STEPWISE, q.device, workspace)
    ev = (ctypes.c_void_p * len(events))(*[e.value if isinstance(e, ctypes.c_void_p) else e
                                           for e in events])
    marks = DfaSlotMarks(ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)), int(n_ranks))
    _check(lib().dfa_attn_fwd_slots(ctypes.byref(desc), arr.ctypes.data_as(ctypes.c_void_p),
                                    arr.shape[0], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                    _ptr(ws), nbytes, ctypes.byref(marks), _stream(stream)),
           "dfa_attn_fwd_slots")
    return o, lse


def dfa_attn_bwd(q, k, v, o, d_o, lse, blocks, dq=None, dk=None, dv=None, workspace=None,
                 scale=None, stream=None, marks=None, docs=None):
    """Gradients (dq, dk, dv) of the forward over the same block list.
    ``marks``: optional DfaKernelMarks of hipEvent_t handles (dfa_attn_bwd_ex)."""
    import torch
    if d_o.stride() != o.stride():
        raise ValueError("d_o must have o's strides")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("gradients must have their primal's strides")
    desc = make_desc(q, k, v, o, scale, docs)
    arr = _blocks_arg(blocks)
    ws, nbytes = _workspace(desc, arr, DFA_OP_BWD, q.device, workspace)
    args = (ctypes.byref(desc), arr.ctypes.data_as(ctypes.c_void_p), arr.shape[0], _ptr(q),
            _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(ws), nbytes)
    if marks is None:
        _check(lib().dfa_attn_bwd(*args, _stream(stream)), "dfa_attn_bwd")
    else:
        _check(lib().dfa_attn_bwd_ex(*args, ctypes.byref(marks), _stream(stream)), "dfa_attn_bwd_ex")
    return dq, dk, dv


def dfa_attn_bwd_noalloc(q, k, v, o, d_o, lse, blocks, dq, dk, dv, scale=None, stream=None,
                         docs=None):
    """dfa_attn_bwd without a workspace: the library's fixed per-GPU scratch
    is used and nothing is allocated (the caller passes dq, dk, dv)."""
    if d_o.stride() != o.stride():
        raise ValueError("d_o must have o's strides")
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("gradients must have their primal's strides")
    desc = make_desc(q, k, v, o, scale, docs)
    arr = _blocks_arg(blocks)
    _check(lib().dfa_attn_bwd_noalloc(ctypes.byref(desc), arr.ctypes.data_as(ctypes.c_void_p),
                                      arr.shape[0], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o),
                                      _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)),
           "dfa_attn_bwd_noalloc")
    return dq, dk, dv
