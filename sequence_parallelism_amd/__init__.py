"""Python binding of the ring-attention library (libra.so, C ABI in include/ra.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libra.so. PyTorch provides device memory and the current stream. The binding
fails loudly when the library is missing; there is no fallback of any kind.

Function names mirror the C entry points: ra_forward, ra_plan,
ra_forward_planned, ra_forward_steps, ra_backward, ra_lse_merge, ra_classify,
ulysses_permute, ulysses_permute_strided, usp_forward, cp_reorder,
cp_reorder_docs, ra_local_length, ra_workspace_size, ra_backward_workspace_size,
ra_doc_workspace_size, usp_workspace_size, ra_status_string.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra.so")

RA_OK = 0
RA_ERR_NULL, RA_ERR_SHAPE, RA_ERR_DIVISIBILITY, RA_ERR_HEADS = 1, 2, 3, 4
RA_ERR_CU_SEQLENS, RA_ERR_RANK, RA_ERR_UNSUPPORTED, RA_ERR_WORKSPACE, RA_ERR_HIP = 5, 6, 7, 8, 9
RA_BF16, RA_F32 = 0, 1
PARTITIONS = {"contiguous": 0, "zigzag": 1, "striped": 2, "doc_zigzag": 3}

# Symbols declared in include/ra.h.
EXPORTS = ("ra_workspace_size", "ra_forward", "ra_plan", "ra_forward_planned", "ra_forward_steps",
           "ra_backward_workspace_size", "ra_backward", "ra_lse_merge", "ra_classify",
           "ulysses_permute", "ulysses_permute_strided", "usp_workspace_size", "usp_forward",
           "cp_reorder", "cp_reorder_docs", "ra_local_length", "ra_doc_workspace_size",
           "ra_status_string", "ra_abi_version")


class RAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({ra_status_string(status)})")


class ra_shape(ctypes.Structure):
    _fields_ = [("s_total", ctypes.c_int64), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libra.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it first (python -m sequence_parallelism_amd.build "
                          f"or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    shp = ctypes.POINTER(ra_shape)
    lib.ra_workspace_size.argtypes = [shp, i32, i32]
    lib.ra_workspace_size.restype = sz
    lib.ra_forward.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, shp, vp, vp, vp, sz, vp]
    lib.ra_forward.restype = ctypes.c_int
    lib.ra_plan.argtypes = [shp, vp, i32, i32, i32, i32, vp, sz, vp]
    lib.ra_plan.restype = ctypes.c_int
    lib.ra_forward_planned.argtypes = [vp, vp, vp, i32, i32, i32, i32, shp, vp, vp, vp, sz, vp]
    lib.ra_forward_planned.restype = ctypes.c_int
    lib.ra_forward_steps.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, shp, vp, vp, vp, sz, vp]
    lib.ra_forward_steps.restype = ctypes.c_int
    lib.ra_backward_workspace_size.argtypes = [shp, i32, i32]
    lib.ra_backward_workspace_size.restype = sz
    lib.ra_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, shp, vp, vp, vp, vp, sz, vp]
    lib.ra_backward.restype = ctypes.c_int
    lib.ra_lse_merge.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.ra_lse_merge.restype = ctypes.c_int
    lib.ra_classify.argtypes = [shp, vp, i32, i32, i32, i32, i32, i32, vp, vp, sz, vp]
    lib.ra_classify.restype = ctypes.c_int
    lib.ulysses_permute.argtypes = [vp, vp, i32, i64, i32, i32, i32, i32, vp]
    lib.ulysses_permute.restype = ctypes.c_int
    lib.ulysses_permute_strided.argtypes = [vp, vp, i32, i64, i32, i32, i32, i32, i64, vp]
    lib.ulysses_permute_strided.restype = ctypes.c_int
    lib.usp_workspace_size.argtypes = [shp, i32, i32, i32]
    lib.usp_workspace_size.restype = sz
    lib.usp_forward.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, shp, vp, vp, vp, sz, vp]
    lib.usp_forward.restype = ctypes.c_int
    lib.ra_local_length.argtypes = [i64, i32, i32, vp, i32]
    lib.ra_local_length.restype = i64
    lib.ra_doc_workspace_size.argtypes = [i64, i32, vp, i32]
    lib.ra_doc_workspace_size.restype = sz
    lib.cp_reorder_docs.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, i32, i32, vp, sz, vp]
    lib.cp_reorder_docs.restype = ctypes.c_int
    lib.cp_reorder.argtypes = [vp, vp, i64, i32, i32, i32, i32, i32, i32, vp]
    lib.cp_reorder.restype = ctypes.c_int
    lib.ra_status_string.argtypes = [ctypes.c_int]
    lib.ra_status_string.restype = ctypes.c_char_p
    lib.ra_abi_version.argtypes = []
    lib.ra_abi_version.restype = i32
    _lib = lib
    return lib


def ra_status_string(status: int) -> str:
    return load_library().ra_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != RA_OK:
        raise RAError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.bfloat16:
        return RA_BF16
    if dt == torch.float32:
        return RA_F32
    raise ValueError(f"unsupported dtype {dt}")


def _part(partition) -> int:
    return PARTITIONS[partition] if isinstance(partition, str) else int(partition)


def _cu_array(cu_seqlens):
    """Host int32 array for cu_seqlens (or None)."""
    if cu_seqlens is None:
        return None, 0, None
    arr = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                                          dtype=np.int32))
    return arr, len(arr) - 1, arr.ctypes.data


def make_shape(s_total: int, hq: int, hkv: int, d: int, causal: bool = True, softmax_scale: float = 0.0,
               in_dtype: int = RA_BF16, out_dtype: int = RA_BF16) -> ra_shape:
    return ra_shape(int(s_total), int(hq), int(hkv), int(d), int(bool(causal)), float(softmax_scale),
                    int(in_dtype), int(out_dtype))


def ra_workspace_size(shape: ra_shape, cp_size: int, n_docs: int = 0) -> int:
    return int(load_library().ra_workspace_size(ctypes.byref(shape), int(cp_size), int(n_docs)))


def _global_len(partition, cp, s_l, cu_seqlens, s_total):
    """S: given, or the last cu_seqlens entry (doc_zigzag), or cp * S_l."""
    if s_total is not None:
        return int(s_total)
    if _part(partition) == PARTITIONS["doc_zigzag"]:
        if cu_seqlens is None:
            raise ValueError("doc_zigzag needs cu_seqlens or s_total")
        return int(np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens)[-1])
    return cp * s_l


def _attn_common(q, k, v, cp_size, causal, softmax_scale, out_dtype, partition="contiguous", cu_seqlens=None,
                 s_total=None):
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [S_l, hq, d]; k, v must be [cp, S_l, hkv, d]")
    s_l, hq, d = q.shape
    cp, s_l2, hkv, d2 = k.shape
    if cp != cp_size or s_l2 != s_l or d2 != d:
        raise ValueError("q / k / v shapes disagree")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    in_code = _dtype_code(q.dtype)
    if out_dtype is None:
        out_dtype = q.dtype
    S = _global_len(partition, cp, s_l, cu_seqlens, s_total)
    shape = make_shape(S, hq, hkv, d, causal, softmax_scale, in_code, _dtype_code(out_dtype))
    return shape, s_l, hq, d, out_dtype


def _workspace(shape, cp_size, n_docs, device, workspace):
    import torch
    need = ra_workspace_size(shape, cp_size, n_docs)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def ra_forward(q, k, v, cu_seqlens=None, cp_size: int = 1, rank: int = 0, partition="contiguous", *,
               causal: bool = True, softmax_scale: float = 0.0, out_dtype=None, out=None, lse=None,
               workspace=None, stream=None, s_total=None):
    """One rank's ring attention. q [S_l,hq,d]; k, v [cp,S_l,hkv,d] (rank-major chunks).
    Returns (out [S_l,hq,d], lse fp32 [hq,S_l])."""
    import torch
    shape, s_l, hq, d, out_dtype = _attn_common(q, k, v, cp_size, causal, softmax_scale, out_dtype, partition,
                                                cu_seqlens, s_total)
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    if out is None:
        out = torch.empty((s_l, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((hq, s_l), dtype=torch.float32, device=q.device)
    ws, ws_bytes = _workspace(shape, cp_size, n_docs, q.device, workspace)
    st = load_library().ra_forward(_ptr(q), _ptr(k), _ptr(v), cu_ptr, n_docs, int(cp_size), int(rank),
                                   _part(partition), ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(ws),
                                   ws_bytes, _stream(stream))
    _check(st, "ra_forward")
    return out, lse


class Plan:
    """A work list built by ra_plan in a workspace tensor, for ra_forward_planned."""

    def __init__(self, shape, n_docs, cp_size, rank, partition, workspace, ws_bytes):
        self.shape, self.n_docs, self.cp_size, self.rank = shape, n_docs, cp_size, rank
        self.partition, self.workspace, self.ws_bytes = partition, workspace, ws_bytes


def ra_plan(s_total: int, hq: int, hkv: int, d: int, cu_seqlens=None, cp_size: int = 1, rank: int = 0,
            partition="contiguous", *, causal: bool = True, softmax_scale: float = 0.0, in_dtype=None,
            out_dtype=None, device="cuda", workspace=None, stream=None) -> Plan:
    """Uploads cu_seqlens and builds the work list; returns a Plan for ra_forward_planned."""
    import torch
    in_dtype = torch.bfloat16 if in_dtype is None else in_dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    shape = make_shape(s_total, hq, hkv, d, causal, softmax_scale, _dtype_code(in_dtype), _dtype_code(out_dtype))
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    ws, ws_bytes = _workspace(shape, cp_size, n_docs, device, workspace)
    st = load_library().ra_plan(ctypes.byref(shape), cu_ptr, n_docs, int(cp_size), int(rank), _part(partition),
                                _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "ra_plan")
    return Plan(shape, n_docs, int(cp_size), int(rank), _part(partition), ws, ws_bytes)


def ra_forward_planned(q, k, v, plan: Plan, *, out=None, lse=None, stream=None):
    """The attention kernel alone, on a Plan from ra_plan with the same shape."""
    import torch
    s_l, hq, d = q.shape
    out_dtype = torch.bfloat16 if plan.shape.out_dtype == RA_BF16 else torch.float32
    if out is None:
        out = torch.empty((s_l, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((hq, s_l), dtype=torch.float32, device=q.device)
    st = load_library().ra_forward_planned(_ptr(q), _ptr(k), _ptr(v), plan.n_docs, plan.cp_size, plan.rank,
                                           plan.partition, ctypes.byref(plan.shape), _ptr(out), _ptr(lse),
                                           _ptr(plan.workspace), plan.ws_bytes, _stream(stream))
    _check(st, "ra_forward_planned")
    return out, lse


def ra_forward_steps(q, k, v, cu_seqlens=None, cp_size: int = 1, rank: int = 0, partition="contiguous", *,
                     causal: bool = True, softmax_scale: float = 0.0, o_steps=None, lse_steps=None,
                     workspace=None, stream=None, s_total=None):
    """Per-step normalised partials: (o_steps fp32 [cp,S_l,hq,d], lse_steps fp32 [cp,hq,S_l])."""
    import torch
    shape, s_l, hq, d, _ = _attn_common(q, k, v, cp_size, causal, softmax_scale, torch.float32, partition,
                                        cu_seqlens, s_total)
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    if o_steps is None:
        o_steps = torch.empty((cp_size, s_l, hq, d), dtype=torch.float32, device=q.device)
    if lse_steps is None:
        lse_steps = torch.empty((cp_size, hq, s_l), dtype=torch.float32, device=q.device)
    ws, ws_bytes = _workspace(shape, cp_size, n_docs, q.device, workspace)
    st = load_library().ra_forward_steps(_ptr(q), _ptr(k), _ptr(v), cu_ptr, n_docs, int(cp_size), int(rank),
                                         _part(partition), ctypes.byref(shape), _ptr(o_steps), _ptr(lse_steps),
                                         _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "ra_forward_steps")
    return o_steps, lse_steps


def ra_backward_workspace_size(shape: ra_shape, cp_size: int, n_docs: int = 0) -> int:
    return int(load_library().ra_backward_workspace_size(ctypes.byref(shape), int(cp_size), int(n_docs)))


def ra_backward(q, k, v, out, lse, dout, cu_seqlens=None, cp_size: int = 1, rank: int = 0, partition="contiguous",
                *, causal: bool = True, softmax_scale: float = 0.0, dq=None, dk=None, dv=None, workspace=None,
                stream=None, s_total=None):
    """Gradients of one rank's ring attention. q, dout [S_l,hq,d] (input dtype); k, v
    [cp,S_l,hkv,d]; out [S_l,hq,d] and lse fp32 [hq,S_l] from the forward. Returns
    (dq fp32 [S_l,hq,d], dk fp32 [cp,S_l,hkv,d], dv fp32 [cp,S_l,hkv,d]): dk / dv hold
    this rank's contribution to every chunk's gradient."""
    import torch
    shape, s_l, hq, d, _ = _attn_common(q, k, v, cp_size, causal, softmax_scale, out.dtype, partition, cu_seqlens,
                                        s_total)
    if dout.shape != q.shape or dout.dtype != q.dtype or out.shape != q.shape or lse.shape != (hq, s_l):
        raise ValueError("out / dout must be [S_l,hq,d] (dout in q's dtype), lse [hq,S_l]")
    for t in (out, lse, dout):
        if not t.is_contiguous():
            raise ValueError("out, lse, dout must be contiguous")
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    hkv = k.shape[2]
    if dq is None:
        dq = torch.empty((s_l, hq, d), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty((cp_size, s_l, hkv, d), dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty((cp_size, s_l, hkv, d), dtype=torch.float32, device=q.device)
    need = ra_backward_workspace_size(shape, cp_size, n_docs)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load_library().ra_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), cu_ptr, n_docs,
                                    int(cp_size), int(rank), _part(partition), ctypes.byref(shape), _ptr(dq),
                                    _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "ra_backward")
    return dq, dk, dv


def ra_lse_merge(o_a, lse_a, o_b, lse_b, o_out=None, lse_out=None, stream=None):
    """fp32 merge of two partials; o [rows,h,d], lse [h,rows]."""
    import torch
    rows, h, d = o_a.shape
    if o_out is None:
        o_out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    st = load_library().ra_lse_merge(rows, h, d, _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out),
                                     _ptr(lse_out), _stream(stream))
    _check(st, "ra_lse_merge")
    return o_out, lse_out


def ra_local_length(s_total: int, cp_size: int, partition, cu_seqlens=None) -> int:
    """Tokens (slots) one rank holds; -1 for invalid arguments."""
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    return int(load_library().ra_local_length(int(s_total), int(cp_size), _part(partition), cu_ptr, n_docs))


def ra_doc_workspace_size(s_total: int, cp_size: int, cu_seqlens=None) -> int:
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    return int(load_library().ra_doc_workspace_size(int(s_total), int(cp_size), cu_ptr, n_docs))


def cp_reorder_docs(x, cp_size: int, cu_seqlens=None, inverse: bool = False, out=None, s_total=None,
                    workspace=None, stream=None):
    """Per-document zigzag reorder. Forward: [S, h, d] -> [cp, S_l, h, d] (padding zero);
    inverse: [cp, S_l, h, d] -> [S, h, d] (pass s_total when cu_seqlens is None)."""
    import torch
    if not x.is_contiguous():
        raise ValueError("input must be contiguous")
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    if not inverse:
        s, h, d = x.shape
    else:
        _, _, h, d = x.shape
        s = int(cu_arr[-1]) if cu_arr is not None else int(s_total)
    sl = ra_local_length(s, cp_size, "doc_zigzag", cu_seqlens)
    if out is None:
        shape_out = (s, h, d) if inverse else (cp_size, sl, h, d)
        out = torch.empty(shape_out, dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(256, ra_doc_workspace_size(s, cp_size, cu_seqlens)), dtype=torch.uint8,
                                device=x.device)
    st = load_library().cp_reorder_docs(_ptr(x), _ptr(out), int(s), int(h), int(d), x.element_size(), int(cp_size),
                                        cu_ptr, n_docs, int(bool(inverse)), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "cp_reorder_docs")
    return out


def ra_classify(s_total: int, cp_size: int, rank: int, partition, bm: int, bn: int, cu_seqlens=None,
                causal: bool = True, device="cuda", stream=None):
    """Tile classes int8 [cp, ceil(S_l/bm), ceil(S_l/bn)]: 0 skip, 1 partial, 2 full."""
    import torch
    shape = make_shape(s_total, 1, 1, 64, causal)
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    s_l = ra_local_length(s_total, cp_size, partition, cu_seqlens)
    if s_l < 0:
        s_l = s_total // cp_size  # invalid arguments: the call below reports the status
    cls = torch.empty((cp_size, -(-s_l // bm), -(-s_l // bn)), dtype=torch.int8, device=device)
    need = ra_doc_workspace_size(s_total, cp_size, cu_seqlens) if _part(partition) == PARTITIONS["doc_zigzag"] else 0
    ws = torch.empty(max(256, 4 * (n_docs + 1), need), dtype=torch.uint8, device=device)
    st = load_library().ra_classify(ctypes.byref(shape), cu_ptr, n_docs, int(cp_size), int(rank), _part(partition),
                                    int(bm), int(bn), _ptr(cls), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "ra_classify")
    return cls


def ulysses_permute(x, n: int, inverse: bool = False, out=None, stream=None):
    """Forward: [n, s_l, h, d] -> [n, n*s_l, h/n, d]; inverse: the reverse."""
    import torch
    if not x.is_contiguous():
        raise ValueError("input must be contiguous")
    if not inverse:
        nn, s_l, h, d = x.shape
        shape_out = (nn, nn * s_l, h // max(1, n), d)
    else:
        nn, s, hn, d = x.shape
        s_l, h = s // max(1, n), hn * n
        shape_out = (nn, s_l, h, d)
    if nn != n:
        raise ValueError("leading dimension must equal n")
    if out is None:
        out = torch.empty(shape_out, dtype=x.dtype, device=x.device)
    st = load_library().ulysses_permute(_ptr(x), _ptr(out), int(n), int(s_l), int(h), int(d), x.element_size(),
                                        int(bool(inverse)), _stream(stream))
    _check(st, "ulysses_permute")
    return out


def ulysses_permute_strided(x, n: int, out, block_stride: int, inverse: bool = False, h: Optional[int] = None,
                            stream=None):
    """ulysses_permute with the head-split side's n blocks block_stride bytes apart.
    Forward: x [n, s_l, h, d] -> blocks of out; inverse: blocks of x -> out [n, s_l, h, d].
    `out` (forward) or `x` (inverse) is the base tensor of the strided side; for the
    inverse pass the full head count h."""
    if not inverse:
        nn, s_l, hh, d = x.shape
    else:
        nn, s_l, hh, d = out.shape
    if nn != n:
        raise ValueError("leading dimension must equal n")
    st = load_library().ulysses_permute_strided(_ptr(x), _ptr(out), int(n), int(s_l), int(hh), int(d),
                                                x.element_size(), int(bool(inverse)), int(block_stride),
                                                _stream(stream))
    _check(st, "ulysses_permute_strided")
    return out


def usp_workspace_size(shape: ra_shape, ulysses: int, ring: int, n_docs: int = 0) -> int:
    return int(load_library().usp_workspace_size(ctypes.byref(shape), int(ulysses), int(ring), int(n_docs)))


def usp_forward(q, k, v, cu_seqlens=None, ulysses: int = 1, ring: int = 1, partition="contiguous", *,
                causal: bool = True, softmax_scale: float = 0.0, out_dtype=None, out=None, lse=None, workspace=None,
                stream=None):
    """Ulysses x Ring grid on one GPU. q [ring, ulysses, S/(ring ulysses), hq, d]; k, v the same with hkv.
    Returns (out [ring, ulysses, S/(ring ulysses), hq, d], lse fp32 [ulysses, ring, hq/ulysses, S/ring])."""
    import torch
    if q.dim() != 5 or k.dim() != 5 or v.shape != k.shape:
        raise ValueError("q, k, v must be [ring, ulysses, S/(ring ulysses), heads, d]")
    R, U, sh, hq, d = q.shape
    hkv = k.shape[3]
    if (R, U, sh) != tuple(k.shape[:3]) or R != ring or U != ulysses or k.shape[4] != d:
        raise ValueError("q / k / v shapes disagree with the grid")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    S = R * U * sh
    shape = make_shape(S, hq, hkv, d, causal, softmax_scale, _dtype_code(q.dtype), _dtype_code(out_dtype))
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    if out is None:
        out = torch.empty((R, U, sh, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((U, R, hq // max(1, U), S // R), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(256, usp_workspace_size(shape, U, R, n_docs)), dtype=torch.uint8,
                                device=q.device)
    st = load_library().usp_forward(_ptr(q), _ptr(k), _ptr(v), cu_ptr, n_docs, int(U), int(R), _part(partition),
                                    ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "usp_forward")
    return out, lse


def cp_reorder(x, cp_size: int, partition, inverse: bool = False, out=None, stream=None):
    """Forward: [S, h, d] -> [cp, S/cp, h, d]; inverse: the reverse."""
    import torch
    if not x.is_contiguous():
        raise ValueError("input must be contiguous")
    if not inverse:
        s, h, d = x.shape
        shape_out = (cp_size, s // cp_size, h, d)
    else:
        cp, s_l, h, d = x.shape
        s = cp * s_l
        shape_out = (s, h, d)
    if out is None:
        out = torch.empty(shape_out, dtype=x.dtype, device=x.device)
    st = load_library().cp_reorder(_ptr(x), _ptr(out), int(s), int(h), int(d), x.element_size(), int(cp_size),
                                   _part(partition), int(bool(inverse)), _stream(stream))
    _check(st, "cp_reorder")
    return out
