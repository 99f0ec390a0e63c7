"""Python binding of the ring-attention library (libra.so, C ABI in include/ra.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libra.so. PyTorch provides device memory and the current stream. The binding
fails loudly when the library is missing; there is no fallback of any kind.

Function names mirror the C entry points: ra_forward, ra_forward_noalloc, ra_plan,
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
RA_ERR_SCRATCH = 10
NOALLOC_SCRATCH_BYTES = 16 << 20  # RA_NOALLOC_SCRATCH_BYTES of include/ra.h
RA_BF16, RA_F32 = 0, 1
PARTITIONS = {"contiguous": 0, "zigzag": 1, "striped": 2, "doc_zigzag": 3}
RA_PART_DOC_ZIGZAG = PARTITIONS["doc_zigzag"]

# Symbols declared in include/ra.h.
EXPORTS = ("ra_workspace_size", "ra_forward", "ra_forward_noalloc", "ra_plan", "ra_forward_planned",
           "ra_forward_planned_docs", "ra_forward_steps",
           "ra_backward_workspace_size", "ra_backward", "ra_lse_merge", "ra_classify",
           "ulysses_permute", "ulysses_permute_strided", "usp_workspace_size", "usp_forward",
           "cp_reorder", "cp_reorder_docs", "ra_local_length", "ra_doc_workspace_size",
           "ra_status_string", "ra_abi_version", "ra_probe_mfma")


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
    lib.ra_forward_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, shp, vp, vp, vp]
    lib.ra_forward_noalloc.restype = ctypes.c_int
    lib.ra_plan.argtypes = [shp, vp, i32, i32, i32, i32, vp, sz, vp]
    lib.ra_plan.restype = ctypes.c_int
    lib.ra_forward_planned.argtypes = [vp, vp, vp, i32, i32, i32, i32, shp, vp, vp, vp, sz, vp]
    lib.ra_forward_planned.restype = ctypes.c_int
    lib.ra_forward_planned_docs.argtypes = [vp, vp, vp, vp, i32, i32, i32, shp, vp, vp, vp, sz, vp]
    lib.ra_forward_planned_docs.restype = ctypes.c_int
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
    lib.ra_probe_mfma.argtypes = [i32, i32, i32, vp, vp]
    lib.ra_probe_mfma.restype = ctypes.c_int
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


def _torch_stream(stream):
    """The torch stream object of `stream` (None: the current stream; a raw
    hipStream_t handle is wrapped as an external stream)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    if int(stream) == 0:
        return torch.cuda.default_stream()
    return torch.cuda.ExternalStream(int(stream))


class _On:
    """Runs the body with `stream` as the current stream, so that the caching
    allocator associates every temporary (workspace, default outputs) with the
    stream the kernels run on: a temporary freed when the call returns is then
    reused only by work ordered after those kernels."""

    def __init__(self, stream):
        import torch
        self.s = _torch_stream(stream)
        self.ctx = torch.cuda.stream(self.s)

    def __enter__(self):
        self.ctx.__enter__()
        return self.s.cuda_stream

    def __exit__(self, *exc):
        return self.ctx.__exit__(*exc)


def _need(t, name: str, shape, dtype=None, contiguous: bool = True):
    """Raises ValueError unless tensor t has exactly `shape` (and `dtype`) and is contiguous."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(int(s) for s in shape):
        raise ValueError(f"{name} must have shape {tuple(int(s) for s in shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_bytes(t, name: str, nbytes: int):
    """Raises ValueError unless t is a contiguous tensor of at least nbytes bytes."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, {nbytes} needed")


def _same_gpu(*named):
    """Raises ValueError unless every given tensor sits on one GPU device."""
    ts = [(n, t) for n, t in named if t is not None]
    dev = ts[0][1].device
    if dev.type != "cuda":
        raise ValueError(f"{ts[0][0]} is on {dev}: every tensor must be on a GPU")
    for n, t in ts[1:]:
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, {ts[0][0]} on {dev}: tensors must share one GPU")
    return dev


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.bfloat16:
        return RA_BF16
    if dt == torch.float32:
        return RA_F32
    raise ValueError(f"unsupported dtype {dt}")


def _torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == RA_BF16 else torch.float32


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
    """Checks q [S_l,hq,d] and k, v [cp,S_l,hkv,d] against each other; returns the shape."""
    if q is None or k is None or v is None:
        raise ValueError("q, k and v are required")
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [S_l, hq, d]; k, v must be [cp, S_l, hkv, d]")
    s_l, hq, d = q.shape
    cp, s_l2, hkv, d2 = k.shape
    if cp != cp_size or s_l2 != s_l or d2 != d:
        raise ValueError(f"k has shape {tuple(k.shape)}; expected [{cp_size}, {s_l}, hkv, {d}]")
    _need(q, "q", q.shape)
    in_dtype = q.dtype
    _dtype_code(in_dtype)
    _need(k, "k", k.shape, in_dtype)
    _need(v, "v", k.shape, in_dtype)
    if out_dtype is None:
        out_dtype = q.dtype
    S = _global_len(partition, cp, s_l, cu_seqlens, s_total)
    if _part(partition) == PARTITIONS["doc_zigzag"]:
        want = ra_local_length(S, cp_size, partition, cu_seqlens)
        if want != s_l:
            raise ValueError(f"doc_zigzag: this S and cu_seqlens give S_l = {want}, the tensors hold {s_l}")
    elif S != cp * s_l:
        raise ValueError(f"s_total {S} is not cp * S_l = {cp * s_l}")
    shape = make_shape(S, hq, hkv, d, causal, softmax_scale, _dtype_code(in_dtype), _dtype_code(out_dtype))
    return shape, s_l, hq, d, out_dtype


def _check_ws(workspace, need: int):
    """Checks a caller's workspace against `need` bytes (None: one is allocated later)."""
    if workspace is not None:
        _need_bytes(workspace, "workspace", need)


def _workspace(need, device, workspace):
    """The caller's (checked) workspace, or a new one on the current stream."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def ra_forward(q, k, v, cu_seqlens=None, cp_size: int = 1, rank: int = 0, partition="contiguous", *,
               causal: bool = True, softmax_scale: float = 0.0, out_dtype=None, out=None, lse=None,
               workspace=None, stream=None, s_total=None):
    """One rank's ring attention. q [S_l,hq,d]; k, v [cp,S_l,hkv,d] (rank-major chunks).
    The output dtype is out_dtype, else out's dtype when out is given, else q's.
    Returns (out [S_l,hq,d], lse fp32 [hq,S_l])."""
    import torch
    if out_dtype is None and out is not None:
        out_dtype = out.dtype
    shape, s_l, hq, d, out_dtype = _attn_common(q, k, v, cp_size, causal, softmax_scale, out_dtype, partition,
                                                cu_seqlens, s_total)
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    if out is not None:
        _need(out, "out", (s_l, hq, d), out_dtype)
    if lse is not None:
        _need(lse, "lse", (hq, s_l), torch.float32)
    need = ra_workspace_size(shape, cp_size, n_docs)
    _check_ws(workspace, need)
    dev = _same_gpu(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("workspace", workspace))
    with _On(stream) as st:
        if out is None:
            out = torch.empty((s_l, hq, d), dtype=out_dtype, device=dev)
        if lse is None:
            lse = torch.empty((hq, s_l), dtype=torch.float32, device=dev)
        ws, ws_bytes = _workspace(need, dev, workspace)
        status = load_library().ra_forward(_ptr(q), _ptr(k), _ptr(v), cu_ptr, n_docs, int(cp_size), int(rank),
                                           _part(partition), ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(ws),
                                           ws_bytes, st)
    _check(status, "ra_forward")
    return out, lse


def ra_forward_noalloc(q, k, v, cu_seqlens=None, cp_size: int = 1, rank: int = 0, partition="contiguous", *,
                       out, lse, causal: bool = True, softmax_scale: float = 0.0, stream=None, s_total=None):
    """ra_forward without any allocation, for callers that cannot allocate: the
    caller passes out [S_l,hq,d] and lse fp32 [hq,S_l]; the plan lives in the
    library's fixed per-GPU scratch (NOALLOC_SCRATCH_BYTES). Calls that overlap on
    one GPU race. Returns (out, lse)."""
    import torch
    if out is None or lse is None:
        raise ValueError("ra_forward_noalloc allocates nothing: pass out and lse")
    shape, s_l, hq, d, out_dtype = _attn_common(q, k, v, cp_size, causal, softmax_scale, out.dtype, partition,
                                                cu_seqlens, s_total)
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    _need(out, "out", (s_l, hq, d), out_dtype)
    _need(lse, "lse", (hq, s_l), torch.float32)
    _same_gpu(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse))
    st = _torch_stream(stream).cuda_stream
    status = load_library().ra_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), cu_ptr, n_docs, int(cp_size), int(rank),
                                               _part(partition), ctypes.byref(shape), _ptr(out), _ptr(lse), st)
    _check(status, "ra_forward_noalloc")
    return out, lse


def ra_probe_mfma(iters: int, workgroups: int, waves: int = 8, sink=None, stream=None):
    """Calibration (include/ra_probe.h): `workgroups` x `waves` waves each run `iters`
    x 4 independent bf16 MFMAs from registers. Returns the sink tensor; executed
    FLOPs = workgroups * waves * iters * 4 * 32768."""
    import torch
    with _On(stream) as st:
        if sink is None:
            sink = torch.empty(int(workgroups) * int(waves) * 64, dtype=torch.float32, device="cuda")
        status = load_library().ra_probe_mfma(int(iters), int(workgroups), int(waves), _ptr(sink), st)
    _check(status, "ra_probe_mfma")
    return sink


class Plan:
    """A work list built by ra_plan in a workspace tensor, for ra_forward_planned.
    s_local is the rank's local length; cu (a host int32 array, or None) the
    documents a per-document zigzag plan was made for."""

    def __init__(self, shape, n_docs, cp_size, rank, partition, workspace, ws_bytes, s_local, cu=None, stream=None):
        self.shape, self.n_docs, self.cp_size, self.rank = shape, n_docs, cp_size, rank
        self.partition, self.workspace, self.ws_bytes = partition, workspace, ws_bytes
        self.s_local, self.cu, self.stream = s_local, cu, stream


def ra_plan(s_total: int, hq: int, hkv: int, d: int, cu_seqlens=None, cp_size: int = 1, rank: int = 0,
            partition="contiguous", *, causal: bool = True, softmax_scale: float = 0.0, in_dtype=None,
            out_dtype=None, device="cuda", workspace=None, stream=None) -> Plan:
    """Uploads cu_seqlens and builds the work list; returns a Plan for ra_forward_planned.
    The plan must be used on the stream it was built on (or after a synchronisation)."""
    import torch
    in_dtype = torch.bfloat16 if in_dtype is None else in_dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    shape = make_shape(s_total, hq, hkv, d, causal, softmax_scale, _dtype_code(in_dtype), _dtype_code(out_dtype))
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    need = ra_workspace_size(shape, cp_size, n_docs)
    _check_ws(workspace, need)
    dev = torch.device(device) if workspace is None else _same_gpu(("workspace", workspace))
    if dev.type != "cuda":
        raise ValueError(f"device {dev}: the plan lives on a GPU")
    on = _On(stream)
    with on as st:
        ws, ws_bytes = _workspace(need, dev, workspace)
        status = load_library().ra_plan(ctypes.byref(shape), cu_ptr, n_docs, int(cp_size), int(rank),
                                        _part(partition), _ptr(ws), ws_bytes, st)
    _check(status, "ra_plan")
    part = _part(partition)
    s_l = ra_local_length(s_total, cp_size, partition, cu_seqlens)
    return Plan(shape, n_docs, int(cp_size), int(rank), part, ws, ws_bytes, s_l,
                cu_arr if part == RA_PART_DOC_ZIGZAG else None, on.s)


def ra_forward_planned(q, k, v, plan: Plan, *, out=None, lse=None, stream=None):
    """The attention kernel alone, on a Plan from ra_plan. q, k, v (and out, lse when
    given) must match the plan's shape: q [S_l, hq, d], k, v [cp, S_l, hkv, d] with
    S_l = plan.s_local (S/cp, or the per-document zigzag length)."""
    import torch
    sh = plan.shape
    s_l = plan.s_local
    in_dtype, out_dtype = _torch_dtype(sh.in_dtype), _torch_dtype(sh.out_dtype)
    _need(q, "q", (s_l, sh.hq, sh.d), in_dtype)
    _need(k, "k", (plan.cp_size, s_l, sh.hkv, sh.d), in_dtype)
    _need(v, "v", (plan.cp_size, s_l, sh.hkv, sh.d), in_dtype)
    if out is not None:
        _need(out, "out", (s_l, sh.hq, sh.d), out_dtype)
    if lse is not None:
        _need(lse, "lse", (sh.hq, s_l), torch.float32)
    dev = _same_gpu(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("plan workspace", plan.workspace))
    on = _On(stream)
    if plan.stream is not None and on.s != plan.stream:
        # the workspace may come from the allocator on the plan's stream: keep it
        # from being handed out again before this launch has read it
        plan.workspace.record_stream(on.s)
    with on as st:
        if out is None:
            out = torch.empty((s_l, sh.hq, sh.d), dtype=out_dtype, device=dev)
        if lse is None:
            lse = torch.empty((sh.hq, s_l), dtype=torch.float32, device=dev)
        if plan.partition == RA_PART_DOC_ZIGZAG:
            cu_ptr = plan.cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if plan.cu is not None else None
            status = load_library().ra_forward_planned_docs(_ptr(q), _ptr(k), _ptr(v), cu_ptr, plan.n_docs,
                                                            plan.cp_size, plan.rank, ctypes.byref(sh), _ptr(out),
                                                            _ptr(lse), _ptr(plan.workspace), plan.ws_bytes, st)
        else:
            status = load_library().ra_forward_planned(_ptr(q), _ptr(k), _ptr(v), plan.n_docs, plan.cp_size,
                                                       plan.rank, plan.partition, ctypes.byref(sh), _ptr(out),
                                                       _ptr(lse), _ptr(plan.workspace), plan.ws_bytes, st)
    _check(status, "ra_forward_planned")
    return out, lse


def ra_forward_steps(q, k, v, cu_seqlens=None, cp_size: int = 1, rank: int = 0, partition="contiguous", *,
                     causal: bool = True, softmax_scale: float = 0.0, o_steps=None, lse_steps=None,
                     workspace=None, stream=None, s_total=None):
    """Per-step normalised partials: (o_steps fp32 [cp,S_l,hq,d], lse_steps fp32 [cp,hq,S_l])."""
    import torch
    shape, s_l, hq, d, _ = _attn_common(q, k, v, cp_size, causal, softmax_scale, torch.float32, partition,
                                        cu_seqlens, s_total)
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    if o_steps is not None:
        _need(o_steps, "o_steps", (cp_size, s_l, hq, d), torch.float32)
    if lse_steps is not None:
        _need(lse_steps, "lse_steps", (cp_size, hq, s_l), torch.float32)
    need = ra_workspace_size(shape, cp_size, n_docs)
    _check_ws(workspace, need)
    dev = _same_gpu(("q", q), ("k", k), ("v", v), ("o_steps", o_steps), ("lse_steps", lse_steps),
                    ("workspace", workspace))
    with _On(stream) as st:
        if o_steps is None:
            o_steps = torch.empty((cp_size, s_l, hq, d), dtype=torch.float32, device=dev)
        if lse_steps is None:
            lse_steps = torch.empty((cp_size, hq, s_l), dtype=torch.float32, device=dev)
        ws, ws_bytes = _workspace(need, dev, workspace)
        status = load_library().ra_forward_steps(_ptr(q), _ptr(k), _ptr(v), cu_ptr, n_docs, int(cp_size), int(rank),
                                                 _part(partition), ctypes.byref(shape), _ptr(o_steps),
                                                 _ptr(lse_steps), _ptr(ws), ws_bytes, st)
    _check(status, "ra_forward_steps")
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
    if out is None:
        raise ValueError("out is required")
    shape, s_l, hq, d, _ = _attn_common(q, k, v, cp_size, causal, softmax_scale, out.dtype, partition, cu_seqlens,
                                        s_total)
    _need(out, "out", q.shape)
    _need(lse, "lse", (hq, s_l), torch.float32)
    _need(dout, "dout", q.shape, q.dtype)
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    hkv = k.shape[2]
    for name, t, shp in (("dq", dq, (s_l, hq, d)), ("dk", dk, (cp_size, s_l, hkv, d)),
                         ("dv", dv, (cp_size, s_l, hkv, d))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    need = ra_backward_workspace_size(shape, cp_size, n_docs)
    _check_ws(workspace, need)
    dev = _same_gpu(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv), ("workspace", workspace))
    with _On(stream) as st:
        if dq is None:
            dq = torch.empty((s_l, hq, d), dtype=torch.float32, device=dev)
        if dk is None:
            dk = torch.empty((cp_size, s_l, hkv, d), dtype=torch.float32, device=dev)
        if dv is None:
            dv = torch.empty((cp_size, s_l, hkv, d), dtype=torch.float32, device=dev)
        ws, ws_bytes = _workspace(need, dev, workspace)
        status = load_library().ra_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), cu_ptr,
                                            n_docs, int(cp_size), int(rank), _part(partition), ctypes.byref(shape),
                                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes, st)
    _check(status, "ra_backward")
    return dq, dk, dv


def ra_lse_merge(o_a, lse_a, o_b, lse_b, o_out=None, lse_out=None, stream=None):
    """fp32 merge of two partials; o [rows,h,d], lse [h,rows]. o_out / lse_out may be
    o_a or o_b / lse_a or lse_b (in place)."""
    import torch
    if o_a is None or o_a.dim() != 3:
        raise ValueError("o_a must be [rows, h, d]")
    rows, h, d = o_a.shape
    _need(o_a, "o_a", (rows, h, d), torch.float32)
    _need(o_b, "o_b", (rows, h, d), torch.float32)
    _need(lse_a, "lse_a", (h, rows), torch.float32)
    _need(lse_b, "lse_b", (h, rows), torch.float32)
    if o_out is not None:
        _need(o_out, "o_out", (rows, h, d), torch.float32)
    if lse_out is not None:
        _need(lse_out, "lse_out", (h, rows), torch.float32)
    dev = _same_gpu(("o_a", o_a), ("lse_a", lse_a), ("o_b", o_b), ("lse_b", lse_b), ("o_out", o_out),
                    ("lse_out", lse_out))
    with _On(stream) as st:
        if o_out is None:
            o_out = torch.empty_like(o_a)
        if lse_out is None:
            lse_out = torch.empty_like(lse_a)
        status = load_library().ra_lse_merge(rows, h, d, _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b),
                                             _ptr(o_out), _ptr(lse_out), st)
    _check(status, "ra_lse_merge")
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
    if x is None or x.dim() != (4 if inverse else 3):
        raise ValueError("input must be [S, h, d] (forward) or [cp, S_l, h, d] (inverse)")
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    if not inverse:
        s, h, d = x.shape
    else:
        _, _, h, d = x.shape
        if cu_arr is None and s_total is None:
            raise ValueError("the inverse needs cu_seqlens or s_total")
        s = int(cu_arr[-1]) if cu_arr is not None else int(s_total)
    sl = ra_local_length(s, cp_size, "doc_zigzag", cu_seqlens)
    if sl < 0:
        raise ValueError(f"doc_zigzag: S={s}, cp={cp_size} and cu_seqlens give no valid layout")
    shape_in = (cp_size, sl, h, d) if inverse else (s, h, d)
    shape_out = (s, h, d) if inverse else (cp_size, sl, h, d)
    _need(x, "input", shape_in)
    if out is not None:
        _need(out, "out", shape_out, x.dtype)
    need = ra_doc_workspace_size(s, cp_size, cu_seqlens)
    _check_ws(workspace, need)
    dev = _same_gpu(("input", x), ("out", out), ("workspace", workspace))
    with _On(stream) as st:
        if out is None:
            out = torch.empty(shape_out, dtype=x.dtype, device=dev)
        ws, ws_bytes = _workspace(need, dev, workspace)
        status = load_library().cp_reorder_docs(_ptr(x), _ptr(out), int(s), int(h), int(d), x.element_size(),
                                                int(cp_size), cu_ptr, n_docs, int(bool(inverse)), _ptr(ws), ws_bytes,
                                                st)
    _check(status, "cp_reorder_docs")
    return out


def ra_classify(s_total: int, cp_size: int, rank: int, partition, bm: int, bn: int, cu_seqlens=None,
                causal: bool = True, device="cuda", stream=None):
    """Tile classes int8 [cp, ceil(S_l/bm), ceil(S_l/bn)]: 0 skip, 1 partial, 2 full."""
    import torch
    shape = make_shape(s_total, 1, 1, 64, causal)
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    s_l = ra_local_length(s_total, cp_size, partition, cu_seqlens)
    if s_l < 0:
        s_l = s_total // max(1, cp_size)  # invalid arguments: the call below reports the status
    if bm < 1 or bn < 1:
        raise ValueError("bm and bn must be positive")
    dev = torch.device(device)
    if dev.type != "cuda":
        raise ValueError(f"device {dev}: classification runs on a GPU")
    need = ra_doc_workspace_size(s_total, cp_size, cu_seqlens) if _part(partition) == PARTITIONS["doc_zigzag"] else 0
    with _On(stream) as st:
        cls = torch.empty((cp_size, -(-s_l // bm), -(-s_l // bn)), dtype=torch.int8, device=dev)
        ws = torch.empty(max(256, 4 * (n_docs + 1), need), dtype=torch.uint8, device=dev)
        status = load_library().ra_classify(ctypes.byref(shape), cu_ptr, n_docs, int(cp_size), int(rank),
                                            _part(partition), int(bm), int(bn), _ptr(cls), _ptr(ws), ws.numel(), st)
    _check(status, "ra_classify")
    return cls


def ulysses_permute(x, n: int, inverse: bool = False, out=None, stream=None):
    """Forward: [n, s_l, h, d] -> [n, n*s_l, h/n, d]; inverse: the reverse."""
    import torch
    if x is None or x.dim() != 4:
        raise ValueError("input must be 4-d: [n, s_l, h, d] (forward) or [n, n*s_l, h/n, d] (inverse)")
    if not inverse:
        nn, s_l, h, d = x.shape
        if n < 1 or h % n:
            raise ValueError(f"the head count {h} must divide by n = {n}")
        shape_out = (nn, nn * s_l, h // n, d)
    else:
        nn, s, hn, d = x.shape
        if n < 1 or s % n:
            raise ValueError(f"the token count {s} must divide by n = {n}")
        s_l, h = s // n, hn * n
        shape_out = (nn, s_l, h, d)
    if nn != n:
        raise ValueError("leading dimension must equal n")
    _need(x, "input", x.shape)
    if out is not None:
        _need(out, "out", shape_out, x.dtype)
    dev = _same_gpu(("input", x), ("out", out))
    with _On(stream) as st:
        if out is None:
            out = torch.empty(shape_out, dtype=x.dtype, device=dev)
        status = load_library().ulysses_permute(_ptr(x), _ptr(out), int(n), int(s_l), int(h), int(d),
                                                x.element_size(), int(bool(inverse)), st)
    _check(status, "ulysses_permute")
    return out


def ulysses_permute_strided(x, n: int, out, block_stride: int, inverse: bool = False, h: Optional[int] = None,
                            stream=None):
    """ulysses_permute with the head-split side's n blocks block_stride bytes apart.
    Forward: x [n, s_l, h, d] -> blocks of out; inverse: blocks of x -> out [n, s_l, h, d].
    `out` (forward) or `x` (inverse) is the base tensor of the strided side, and must
    hold the n blocks: (n - 1) block_stride bytes plus one block."""
    if x is None or out is None:
        raise ValueError("x and out are required")
    packed = out if inverse else x
    if packed.dim() != 4:
        raise ValueError("the packed side must be [n, s_l, h, d]")
    nn, s_l, hh, d = packed.shape
    if nn != n:
        raise ValueError("leading dimension must equal n")
    if n < 1 or hh % n:
        raise ValueError(f"the head count {hh} must divide by n = {n}")
    strided = x if inverse else out
    if strided.dtype != packed.dtype:
        raise ValueError("x and out must share a dtype")
    _need(packed, "out" if inverse else "x", packed.shape)
    block = n * s_l * (hh // n) * d * packed.element_size()
    if block_stride < block:
        raise ValueError(f"block_stride {block_stride} is smaller than one block ({block} bytes)")
    _need_bytes(strided, "x" if inverse else "out", (n - 1) * int(block_stride) + block)
    _same_gpu(("x", x), ("out", out))
    with _On(stream) as st:
        status = load_library().ulysses_permute_strided(_ptr(x), _ptr(out), int(n), int(s_l), int(hh), int(d),
                                                        packed.element_size(), int(bool(inverse)),
                                                        int(block_stride), st)
    _check(status, "ulysses_permute_strided")
    return out


def usp_workspace_size(shape: ra_shape, ulysses: int, ring: int, n_docs: int = 0) -> int:
    return int(load_library().usp_workspace_size(ctypes.byref(shape), int(ulysses), int(ring), int(n_docs)))


def usp_forward(q, k, v, cu_seqlens=None, ulysses: int = 1, ring: int = 1, partition="contiguous", *,
                causal: bool = True, softmax_scale: float = 0.0, out_dtype=None, out=None, lse=None, workspace=None,
                stream=None):
    """Ulysses x Ring grid on one GPU. q [ring, ulysses, S/(ring ulysses), hq, d]; k, v the same with hkv.
    Returns (out [ring, ulysses, S/(ring ulysses), hq, d], lse fp32 [ulysses, ring, hq/ulysses, S/ring])."""
    import torch
    if q is None or k is None or v is None or q.dim() != 5 or k.dim() != 5:
        raise ValueError("q, k, v must be [ring, ulysses, S/(ring ulysses), heads, d]")
    R, U, sh, hq, d = q.shape
    hkv = k.shape[3]
    if (R, U, sh) != tuple(k.shape[:3]) or R != ring or U != ulysses or k.shape[4] != d:
        raise ValueError("q / k / v shapes disagree with the grid")
    if hq % U or hkv % U:
        raise ValueError(f"the head counts {hq}, {hkv} must divide by ulysses = {U}")
    _dtype_code(q.dtype)
    _need(q, "q", q.shape)
    _need(k, "k", k.shape, q.dtype)
    _need(v, "v", k.shape, q.dtype)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else q.dtype
    S = R * U * sh
    shape = make_shape(S, hq, hkv, d, causal, softmax_scale, _dtype_code(q.dtype), _dtype_code(out_dtype))
    cu_arr, n_docs, cu_ptr = _cu_array(cu_seqlens)
    if out is not None:
        _need(out, "out", (R, U, sh, hq, d), out_dtype)
    if lse is not None:
        _need(lse, "lse", (U, R, hq // U, S // R), torch.float32)
    need = usp_workspace_size(shape, U, R, n_docs)
    _check_ws(workspace, need)
    dev = _same_gpu(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("workspace", workspace))
    with _On(stream) as st:
        if out is None:
            out = torch.empty((R, U, sh, hq, d), dtype=out_dtype, device=dev)
        if lse is None:
            lse = torch.empty((U, R, hq // U, S // R), dtype=torch.float32, device=dev)
        ws, ws_bytes = _workspace(need, dev, workspace)
        status = load_library().usp_forward(_ptr(q), _ptr(k), _ptr(v), cu_ptr, n_docs, int(U), int(R),
                                            _part(partition), ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(ws),
                                            ws_bytes, st)
    _check(status, "usp_forward")
    return out, lse


def cp_reorder(x, cp_size: int, partition, inverse: bool = False, out=None, stream=None):
    """Forward: [S, h, d] -> [cp, S/cp, h, d]; inverse: the reverse."""
    import torch
    if x is None or x.dim() != (4 if inverse else 3):
        raise ValueError("input must be [S, h, d] (forward) or [cp, S/cp, h, d] (inverse)")
    if not inverse:
        s, h, d = x.shape
        if cp_size < 1 or s % cp_size:
            raise ValueError(f"S = {s} must divide by cp = {cp_size}")
        shape_out = (cp_size, s // cp_size, h, d)
    else:
        cp, s_l, h, d = x.shape
        if cp != cp_size:
            raise ValueError(f"leading dimension {cp} must equal cp = {cp_size}")
        s = cp * s_l
        shape_out = (s, h, d)
    _need(x, "input", x.shape)
    if out is not None:
        _need(out, "out", shape_out, x.dtype)
    dev = _same_gpu(("input", x), ("out", out))
    with _On(stream) as st:
        if out is None:
            out = torch.empty(shape_out, dtype=x.dtype, device=dev)
        status = load_library().cp_reorder(_ptr(x), _ptr(out), int(s), int(h), int(d), x.element_size(),
                                           int(cp_size), _part(partition), int(bool(inverse)), st)
    _check(status, "cp_reorder")
    return out
