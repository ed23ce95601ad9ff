"""MC-Sparse hot path on MI355X: Python binding of libmcs.so.

Every function marshals torch tensors (device memory, current HIP stream) into
the C ABI declared in include/mcs.h; all arithmetic runs in the library's HIP
kernels.  There is no fallback: a missing or failing library raises McsError.

Tensor conventions (see include/mcs.h): q, k, v, outputs and residuals are
[H, N, D] float32 or bfloat16 CUDA tensors; perm is int32 [H, N] (slot ->
token); idx is int32 [H, G, kpad] (ascending kept keys, -1 padded),
G = ceil(N / 64); lse is float32 [H, N].
"""
from __future__ import annotations

import ctypes
import math

from . import _abi
from ._abi import (MCS_BF16, MCS_COPY_D2D, MCS_COPY_D2H, MCS_COPY_H2D, MCS_F32, MCS_OP_ANCHOR,  # noqa: F401
                   MCS_OP_BLOCK_SELECT, MCS_OP_GROUP, MCS_OP_SELECT, McsDims, McsError)

GROUP = 64
POWER_ITERS = 32


def _torch():
    import torch
    return torch


def kpad_for(topk: int) -> int:
    return ((topk + 31) // 32) * 32


def make_dims(q, topk: int = 1, kpad: int | None = None, scale: float | None = None,
              power_iters: int = POWER_ITERS) -> McsDims:
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [H, N, D]")
    h, n, d = q.shape
    if q.dtype == torch.bfloat16:
        dt = MCS_BF16
    elif q.dtype == torch.float32:
        dt = MCS_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return McsDims(heads=h, n=n, head_dim=d, group=GROUP, topk=topk,
                   kpad=kpad_for(topk) if kpad is None else kpad, dtype=dt,
                   power_iters=power_iters, scale=(1.0 / math.sqrt(d)) if scale is None else scale)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _check_same(ref, *ts):
    for t in ts:
        if t is not None and (t.device != ref.device or t.shape != ref.shape or t.dtype != ref.dtype):
            raise ValueError("q, k, v (and outputs) must share device, shape and dtype")


# The C ABI receives bare pointers and cannot know buffer sizes: every tensor is
# checked here, before any library call, so that a wrong dtype, shape or device
# raises ValueError instead of reading or writing past an allocation.

def _check_tensor(t, name, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _groups(n):
    return -(-n // GROUP)


def _check_perm(perm, q):
    _check_tensor(perm, "perm", _torch().int32, q.shape[:2], q.device)


def _check_idx(idx, q, topk, name="idx"):
    """int32 [H, ceil(N/64), kpad], kpad >= topk and a multiple of 32; returns kpad."""
    torch = _torch()
    if not isinstance(idx, torch.Tensor) or idx.dim() != 3:
        raise ValueError(f"{name} must be an int32 [H, G, kpad] tensor")
    kpad = idx.shape[2]
    if kpad < topk or kpad % 32:
        raise ValueError(f"{name}: kpad {kpad} must be >= topk ({topk}) and a multiple of 32")
    _check_tensor(idx, name, torch.int32, (q.shape[0], _groups(q.shape[1]), kpad), q.device)
    return kpad


def _check_lse(lse, q, name="lse"):
    if lse is not None:
        _check_tensor(lse, name, _torch().float32, q.shape[:2], q.device)


def _check_like(t, q, name):
    if t is not None:
        _check_tensor(t, name, q.dtype, q.shape, q.device)


def _check_ws(ws, device):
    torch = _torch()
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")


def _check_gpu(q):
    if not q.is_cuda:
        raise ValueError(f"tensors must be on a GPU device, got {q.device}")


def mcs_workspace_bytes(dims: McsDims, op: int, heads_per_pass: int = 0) -> int:
    lib = _abi.load()
    out = ctypes.c_size_t(0)
    _abi.check(lib.mcs_workspace_bytes(ctypes.byref(dims), op, heads_per_pass, ctypes.byref(out)))
    return out.value


def _workspace(dims, op, device, ws, heads_per_pass):
    torch = _torch()
    need = mcs_workspace_bytes(dims, op, heads_per_pass)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    _check_ws(ws, device)
    return ws


def mcs_group(q, power_iters: int = POWER_ITERS, ws=None, perm=None):
    """PDDP grouping: returns perm int32 [H, N]."""
    torch = _torch()
    lib = _abi.load()
    d = make_dims(q, power_iters=power_iters)
    if perm is None:
        perm = torch.empty(q.shape[:2], dtype=torch.int32, device=q.device)
    _check_perm(perm, q)
    _check_gpu(q)
    ws = _workspace(d, MCS_OP_GROUP, q.device, ws, 0)
    _abi.check(lib.mcs_group(ctypes.byref(d), _ptr(q), _ptr(perm), _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device)))
    return perm


def mcs_select(q, k, perm, topk: int, lse=None, ws=None, heads_per_pass: int = 0, idx=None):
    """Two-pass exact top-K: returns idx int32 [H, G, kpad]."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k)
    d = make_dims(q, topk=topk)
    g = -(-q.shape[1] // GROUP)
    if idx is None:
        idx = torch.empty((q.shape[0], g, d.kpad), dtype=torch.int32, device=q.device)
    d.kpad = _check_idx(idx, q, topk)
    _check_perm(perm, q)
    _check_lse(lse, q)
    _check_gpu(q)
    ws = _workspace(d, MCS_OP_SELECT, q.device, ws, heads_per_pass)
    _abi.check(lib.mcs_select(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(perm), _ptr(lse), _ptr(idx), _ptr(ws),
                              ws.numel(), _stream(q.device)))
    return idx


def mcs_select_noalloc(q, k, perm, topk: int, lse=None, idx=None):
    """mcs_select without a workspace: the library's static device scratch holds the
    selection's intermediates (no device allocation inside the call when idx is given)."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k)
    d = make_dims(q, topk=topk)
    if idx is None:
        idx = torch.empty((q.shape[0], _groups(q.shape[1]), d.kpad), dtype=torch.int32, device=q.device)
    d.kpad = _check_idx(idx, q, topk)
    _check_perm(perm, q)
    _check_lse(lse, q)
    _check_gpu(q)
    _abi.check(lib.mcs_select_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(perm), _ptr(lse), _ptr(idx),
                                      _stream(q.device)))
    return idx


def mcs_dense_attn(q, k, v, want_lse: bool = False, o=None):
    """Dense attention: returns (o, lse or None)."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k, v)
    d = make_dims(q)
    if o is None:
        o = torch.empty_like(q)
    _check_like(o, q, "o")
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if want_lse else None
    _check_gpu(q)
    _abi.check(lib.mcs_dense_attn(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  _stream(q.device)))
    return o, lse


def mcs_sparse_attn(q, k, v, perm, idx, topk: int, resid_add=None, o=None):
    """Gather-sparse attention (+ optional residual): returns o [H, N, D]."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k, v, resid_add)
    d = make_dims(q, topk=topk, kpad=_check_idx(idx, q, topk))
    _check_perm(perm, q)
    if o is None:
        o = torch.empty_like(q)
    _check_like(o, q, "o")
    _check_gpu(q)
    _abi.check(lib.mcs_sparse_attn(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(idx),
                                   _ptr(resid_add), _ptr(o), _stream(q.device)))
    return o


def mcs_anchor(q, k, v, topk: int, power_iters: int = POWER_ITERS, want_lse: bool = False, ws=None,
               heads_per_pass: int = 0, out=None):
    """Anchor step: returns dict(perm, idx, resid, o_dense, lse)."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k, v)
    d = make_dims(q, topk=topk, power_iters=power_iters)
    h, n, _ = q.shape
    g = -(-n // GROUP)
    if out is None:
        out = dict(perm=torch.empty((h, n), dtype=torch.int32, device=q.device),
                   idx=torch.empty((h, g, d.kpad), dtype=torch.int32, device=q.device),
                   resid=torch.empty_like(q), o_dense=torch.empty_like(q),
                   lse=torch.empty((h, n), dtype=torch.float32, device=q.device) if want_lse else None)
    for key in ("perm", "idx", "resid", "o_dense"):
        if out.get(key) is None:
            raise ValueError(f"out[{key!r}] is required")
    _check_perm(out["perm"], q)
    d.kpad = _check_idx(out["idx"], q, topk, "out['idx']")
    _check_like(out["resid"], q, "out['resid']")
    _check_like(out["o_dense"], q, "out['o_dense']")
    _check_lse(out.get("lse"), q, "out['lse']")
    _check_gpu(q)
    ws = _workspace(d, MCS_OP_ANCHOR, q.device, ws, heads_per_pass)
    _abi.check(lib.mcs_anchor(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(out["perm"]), _ptr(out["idx"]),
                              _ptr(out["resid"]), _ptr(out["o_dense"]), _ptr(out.get("lse")), _ptr(ws),
                              ws.numel(), _stream(q.device)))
    return out


def mcs_residual(q, k, v, perm, idx, topk: int, o_dense, resid=None):
    """Residual of a supplied selection: o_dense - sparse attention(perm, idx), [H, N, D]."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k, v, o_dense)
    if o_dense is None:
        raise ValueError("o_dense is required")
    d = make_dims(q, topk=topk, kpad=_check_idx(idx, q, topk))
    _check_perm(perm, q)
    if resid is None:
        resid = torch.empty_like(q)
    _check_like(resid, q, "resid")
    if resid.data_ptr() == o_dense.data_ptr():
        raise ValueError("resid may not alias o_dense")
    _check_gpu(q)
    _abi.check(lib.mcs_residual(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(idx), _ptr(o_dense),
                                _ptr(resid), _stream(q.device)))
    return resid


def mcs_reuse(q, k, v, perm, idx, resid, topk: int, o=None):
    """Reuse step: sparse attention with cached perm/idx plus the cached residual."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k, v, resid)
    if resid is None:
        raise ValueError("resid is required")
    d = make_dims(q, topk=topk, kpad=_check_idx(idx, q, topk))
    _check_perm(perm, q)
    if o is None:
        o = torch.empty_like(q)
    _check_like(o, q, "o")
    _check_gpu(q)
    _abi.check(lib.mcs_reuse(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(idx), _ptr(resid),
                             _ptr(o), _stream(q.device)))
    return o


def mcs_block_select(q, k, topk: int, ws=None, idx=None):
    """Vanilla block sparsity (mean-pooled 64-token blocks): returns idx int32 [H, N/64, kpad] of the
    topk/64 best-scoring key blocks per query block, expanded ascending (use with an identity perm)."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k)
    d = make_dims(q, topk=topk)
    h, n, _ = q.shape
    if idx is None:
        idx = torch.empty((h, -(-n // GROUP), d.kpad), dtype=torch.int32, device=q.device)
    d.kpad = _check_idx(idx, q, topk)
    _check_gpu(q)
    ws = _workspace(d, MCS_OP_BLOCK_SELECT, q.device, ws, 0)
    _abi.check(lib.mcs_block_select(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(idx), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(q.device)))
    return idx


def mcs_sparse_lse(q, k, perm, idx, topk: int, lse=None):
    """Logsumexp of each query's logits over its group's kept keys: float32 [H, N] (token order)."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k)
    d = make_dims(q, topk=topk, kpad=_check_idx(idx, q, topk))
    _check_perm(perm, q)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    _check_lse(lse, q)
    _check_gpu(q)
    _abi.check(lib.mcs_sparse_lse(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(perm), _ptr(idx), _ptr(lse),
                                  _stream(q.device)))
    return lse


def bits_words(n: int) -> int:
    """Words per row of a key bitmap: ceil(n / 32)."""
    return (n + 31) // 32


def _check_rows(t, n, g, shape=None, device=None):
    """One row per (head, group): g must be ceil(n / 64); int32 storage."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 3:
        raise ValueError("key lists and bitmaps are int32 [H, G, width]")
    if g != -(-n // GROUP):
        raise ValueError(f"{g} groups do not match n={n} (expected {-(-n // GROUP)})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"shape {tuple(t.shape)} differs from {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"tensor on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError("key lists and bitmaps must be contiguous")


def _check_list_width(kpad, topk):
    if kpad < topk or kpad % 32:
        raise ValueError(f"kpad {kpad} must be >= topk ({topk}) and a multiple of 32")


def mcs_idx_to_bits(idx, n: int, topk: int, bits=None):
    """Kept-key lists int32 [H, G, kpad] -> key bitmaps uint32 (stored as int32) [H, G, ceil(n/32)]."""
    torch = _torch()
    lib = _abi.load()
    _check_rows(idx, n, idx.shape[1] if idx.dim() == 3 else -1)
    h, g, kpad = idx.shape
    _check_list_width(kpad, topk)
    d = McsDims(heads=h, n=n, head_dim=128, group=GROUP, topk=topk, kpad=kpad, dtype=MCS_BF16,
                power_iters=POWER_ITERS, scale=1.0)
    if bits is None:
        bits = torch.empty((h, g, bits_words(n)), dtype=torch.int32, device=idx.device)
    _check_rows(bits, n, g, (h, g, bits_words(n)), idx.device)
    _check_gpu(idx)
    _abi.check(lib.mcs_idx_to_bits(ctypes.byref(d), _ptr(idx), _ptr(bits), _stream(idx.device)))
    return bits


def mcs_bits_to_idx(bits, n: int, topk: int, idx=None, kpad: int | None = None):
    """Key bitmaps [H, G, ceil(n/32)] -> kept-key lists int32 [H, G, kpad] (ascending, -1 padded)."""
    torch = _torch()
    lib = _abi.load()
    _check_rows(bits, n, bits.shape[1] if bits.dim() == 3 else -1)
    h, g, _ = bits.shape
    _check_rows(bits, n, g, (h, g, bits_words(n)))
    if idx is not None:
        _check_rows(idx, n, idx.shape[1] if idx.dim() == 3 else -1)
        kpad = idx.shape[2]
    elif kpad is None:
        kpad = kpad_for(topk)
    _check_list_width(kpad, topk)
    d = McsDims(heads=h, n=n, head_dim=128, group=GROUP, topk=topk, kpad=kpad, dtype=MCS_BF16,
                power_iters=POWER_ITERS, scale=1.0)
    if idx is None:
        idx = torch.empty((h, g, kpad), dtype=torch.int32, device=bits.device)
    _check_rows(idx, n, g, (h, g, kpad), bits.device)
    _check_gpu(bits)
    _abi.check(lib.mcs_bits_to_idx(ctypes.byref(d), _ptr(bits), _ptr(idx), _stream(bits.device)))
    return idx


def pairs_of(n: int) -> int:
    """Pairs of neighbouring groups per head: ceil(G / 2), G = ceil(n / 64)."""
    return (-(-n // GROUP) + 1) // 2


def mcs_pair_plan(idx, n: int, topk: int, pidx=None, ncommon=None):
    """Kept-key lists [H, G, kpad] -> (pidx [H, G, kpad], ncommon int32 [H, ceil(G/2)]): both rows of
    each pair of groups (2p, 2p+1) list their common keys first (a multiple of 128 of them)."""
    torch = _torch()
    lib = _abi.load()
    _check_rows(idx, n, idx.shape[1] if idx.dim() == 3 else -1)
    h, g, kpad = idx.shape
    _check_list_width(kpad, topk)
    d = McsDims(heads=h, n=n, head_dim=128, group=GROUP, topk=topk, kpad=kpad, dtype=MCS_BF16,
                power_iters=POWER_ITERS, scale=1.0)
    if pidx is None:
        pidx = torch.empty_like(idx)
    _check_rows(pidx, n, g, idx.shape, idx.device)
    if ncommon is None:
        ncommon = torch.empty((h, pairs_of(n)), dtype=torch.int32, device=idx.device)
    _check_tensor(ncommon, "ncommon", torch.int32, (h, pairs_of(n)), idx.device)
    _check_gpu(idx)
    _abi.check(lib.mcs_pair_plan(ctypes.byref(d), _ptr(idx), _ptr(pidx), _ptr(ncommon), _stream(idx.device)))
    return pidx, ncommon


def mcs_sparse_attn_pairs(q, k, v, perm, pidx, ncommon, topk: int, resid_add=None, o=None):
    """Gather-sparse attention on pair-planned lists (+ optional residual): returns o [H, N, D]."""
    torch = _torch()
    lib = _abi.load()
    _check_same(q, k, v, resid_add)
    d = make_dims(q, topk=topk, kpad=_check_idx(pidx, q, topk, "pidx"))
    h, n, _ = q.shape
    _check_perm(perm, q)
    _check_tensor(ncommon, "ncommon", torch.int32, (h, pairs_of(n)), q.device)
    if o is None:
        o = torch.empty_like(q)
    _check_like(o, q, "o")
    _check_gpu(q)
    _abi.check(lib.mcs_sparse_attn_pairs(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(pidx),
                                         _ptr(ncommon), _ptr(resid_add), _ptr(o), _stream(q.device)))
    return o


def mcs_copy_async(dst, src, kind: int, stream=None, event=None):
    """Enqueue a byte copy of src into dst on `stream` (default: current) and record `event`."""
    torch = _torch()
    lib = _abi.load()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src sizes differ")
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("copies need contiguous tensors")
    want = {MCS_COPY_H2D: (False, True), MCS_COPY_D2H: (True, False), MCS_COPY_D2D: (True, True)}
    if kind not in want:
        raise ValueError(f"unknown copy kind {kind}")
    if (src.is_cuda, dst.is_cuda) != want[kind]:
        raise ValueError(f"copy kind {kind} does not match src on {src.device} and dst on {dst.device}")
    dev = src.device if src.is_cuda else dst.device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    ev = ctypes.c_void_p(event.cuda_event) if event is not None else None
    _abi.check(lib.mcs_copy_async(_ptr(dst), _ptr(src), nbytes, kind, ctypes.c_void_p(s.cuda_stream), ev))
