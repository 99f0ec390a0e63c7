"""The C-ABI library loads, exports every symbol include/ra.h declares, and its
host-side validation returns the documented error codes (CPU only: no call
here reaches a HIP launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sequence_parallelism_amd as ra
import synth
from oracle.partition import local_length as oracle_local_length

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p(0x100000)           # stand-in device pointer: never dereferenced by validation
P2 = ctypes.c_void_p(0x7f0000000000)    # far from P: no overlap


def _lib():
    return ra.load_library()


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(\w+)\s*\(", src, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    names = _declared_functions()
    assert names == set(ra.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name
    assert lib.ra_abi_version() == 3


def test_status_strings():
    for code in range(11):
        assert ra.ra_status_string(code) != "unknown status"
    assert ra.ra_status_string(99) == "unknown status"


def shape(**kw):
    base = dict(s_total=32768, hq=32, hkv=32, d=128, causal=True, softmax_scale=0.0,
                in_dtype=ra.RA_BF16, out_dtype=ra.RA_BF16)
    base.update(kw)
    return ra.ra_shape(int(base["s_total"]), int(base["hq"]), int(base["hkv"]), int(base["d"]),
                       int(base["causal"]), float(base["softmax_scale"]), int(base["in_dtype"]),
                       int(base["out_dtype"]))


def fwd(sh, cu=None, n_docs=0, cp=4, rank=0, part=1, ws=P, ws_bytes=1 << 40, q=P, out=P):
    arr = None
    if cu is not None:
        arr = (ctypes.c_int32 * len(cu))(*cu)
    return _lib().ra_forward(q, P, P, arr, n_docs, cp, rank, part, ctypes.byref(sh), out, P, ws, ws_bytes, None)


def test_forward_validation_codes():
    assert fwd(shape(), q=None) == ra.RA_ERR_NULL
    assert fwd(shape(), out=None) == ra.RA_ERR_NULL
    assert _lib().ra_forward(P, P, P, None, 0, 4, 0, 1, None, P, P, P, 1 << 40, None) == ra.RA_ERR_NULL
    assert fwd(shape(s_total=0)) == ra.RA_ERR_SHAPE
    assert fwd(shape(hq=0)) == ra.RA_ERR_SHAPE
    assert fwd(shape(causal=2)) == ra.RA_ERR_SHAPE
    assert fwd(shape(softmax_scale=-1.0)) == ra.RA_ERR_SHAPE
    assert fwd(shape(softmax_scale=float("nan"))) == ra.RA_ERR_SHAPE
    assert fwd(shape(), cp=0) == ra.RA_ERR_SHAPE
    assert fwd(shape(), cp=65) == ra.RA_ERR_SHAPE
    assert fwd(shape(), part=4) == ra.RA_ERR_UNSUPPORTED
    assert fwd(shape(), rank=4) == ra.RA_ERR_RANK
    assert fwd(shape(), rank=-1) == ra.RA_ERR_RANK
    assert fwd(shape(hq=32, hkv=6)) == ra.RA_ERR_HEADS
    assert fwd(shape(d=96)) == ra.RA_ERR_UNSUPPORTED
    assert fwd(shape(in_dtype=7)) == ra.RA_ERR_UNSUPPORTED
    assert fwd(shape(in_dtype=ra.RA_F32, out_dtype=ra.RA_BF16)) == ra.RA_ERR_UNSUPPORTED
    # divisibility: zigzag needs S % 2cp, contiguous / striped need S % cp
    assert fwd(shape(s_total=4 * 1001), part=1) == ra.RA_ERR_DIVISIBILITY
    assert fwd(shape(s_total=4 * 1001), part=0, ws=None, ws_bytes=0) == ra.RA_ERR_WORKSPACE
    assert fwd(shape(s_total=4001), part=2) == ra.RA_ERR_DIVISIBILITY
    # workspace
    sh = shape()
    need = ra.ra_workspace_size(sh, 4, 0)
    assert need > 0
    assert fwd(sh, ws=None) == ra.RA_ERR_WORKSPACE
    assert fwd(sh, ws_bytes=256) == ra.RA_ERR_WORKSPACE
    # the per-step entry point checks its workspace too
    assert _lib().ra_forward_steps(P, P, P, None, 0, 4, 0, 1, ctypes.byref(sh), P, P, P, 1024, None) \
        == ra.RA_ERR_WORKSPACE


def test_cu_seqlens_validation():
    sh = shape(s_total=64, hq=2, hkv=2)
    good = [0, 10, 64]
    assert fwd(sh, cu=[1, 10, 64], n_docs=2, ws_bytes=0) == ra.RA_ERR_CU_SEQLENS
    assert fwd(sh, cu=[0, 10, 63], n_docs=2) == ra.RA_ERR_CU_SEQLENS
    assert fwd(sh, cu=[0, 10, 10, 64], n_docs=3) == ra.RA_ERR_CU_SEQLENS
    assert fwd(sh, cu=[0, 20, 10, 64], n_docs=3) == ra.RA_ERR_CU_SEQLENS
    assert fwd(sh, cu=good, n_docs=0) == ra.RA_ERR_CU_SEQLENS
    # a valid cu_seqlens with too little workspace fails on the workspace, not the documents
    assert fwd(sh, cu=good, n_docs=2, ws_bytes=16) == ra.RA_ERR_WORKSPACE


def test_workspace_size_grows_with_documents_and_is_zero_for_bad_shapes():
    sh = shape()
    a = ra.ra_workspace_size(sh, 4, 0)
    b = ra.ra_workspace_size(sh, 4, 100)
    assert b > a
    assert ra.ra_workspace_size(shape(s_total=0), 4, 0) == 0
    assert ra.ra_workspace_size(sh, 0, 0) == 0
    assert _lib().ra_workspace_size(None, 4, 0) == 0


def test_forward_steps_and_merge_validation():
    lib = _lib()
    sh = shape()
    assert lib.ra_forward_steps(P, P, P, None, 0, 4, 0, 1, ctypes.byref(sh), None, P, P, 1 << 40, None) \
        == ra.RA_ERR_NULL
    assert lib.ra_forward_steps(P, P, P, None, 0, 4, 9, 1, ctypes.byref(sh), P, P, P, 1 << 40, None) \
        == ra.RA_ERR_RANK
    assert lib.ra_lse_merge(-1, 4, 128, P, P, P, P, P, P, None) == ra.RA_ERR_SHAPE
    assert lib.ra_lse_merge(10, 0, 128, P, P, P, P, P, P, None) == ra.RA_ERR_SHAPE
    assert lib.ra_lse_merge(10, 4, 128, None, P, P, P, P, P, None) == ra.RA_ERR_NULL
    assert lib.ra_lse_merge(0, 4, 128, None, None, None, None, None, None, None) == ra.RA_OK
    # the launch grids are bounded: more than 2^37 elements per tensor is refused
    assert lib.ra_lse_merge((1 << 37) // 128 + 1, 1, 128, P, P, P, P, P, P, None) == ra.RA_ERR_SHAPE


def test_classify_validation():
    lib = _lib()
    sh = shape(s_total=4096)
    assert lib.ra_classify(ctypes.byref(sh), None, 0, 4, 0, 1, 128, 128, None, P, 0, None) == ra.RA_ERR_NULL
    assert lib.ra_classify(ctypes.byref(sh), None, 0, 4, 4, 1, 128, 128, P, P, 0, None) == ra.RA_ERR_RANK
    assert lib.ra_classify(ctypes.byref(sh), None, 0, 4, 0, 1, 0, 128, P, P, 0, None) == ra.RA_ERR_SHAPE
    assert lib.ra_classify(ctypes.byref(shape(s_total=4100)), None, 0, 4, 0, 1, 64, 64, P, P, 0, None) \
        == ra.RA_ERR_DIVISIBILITY
    cu = (ctypes.c_int32 * 3)(0, 100, 4096)
    assert lib.ra_classify(ctypes.byref(sh), cu, 2, 4, 0, 1, 64, 64, P, None, 0, None) == ra.RA_ERR_WORKSPACE
    # more than 2^36 tile classes (one launch thread each) is refused
    big = shape(s_total=1 << 20)
    assert lib.ra_classify(ctypes.byref(big), None, 0, 1, 0, 0, 1, 8, P, P, 0, None) == ra.RA_ERR_SHAPE
    bad = (ctypes.c_int32 * 3)(0, 5000, 4096)
    assert lib.ra_classify(ctypes.byref(sh), bad, 2, 4, 0, 1, 64, 64, P, P, 64, None) == ra.RA_ERR_CU_SEQLENS


def test_permute_validation():
    lib = _lib()
    # Ulysses: n must divide the head count (sequence_parallel_size must divide num_attention_heads)
    assert lib.ulysses_permute(P, P2, 4, 1024, 30, 128, 2, 0, None) == ra.RA_ERR_HEADS
    assert lib.ulysses_permute(None, P2, 4, 1024, 32, 128, 2, 0, None) == ra.RA_ERR_NULL
    assert lib.ulysses_permute(P, P2, 0, 1024, 32, 128, 2, 0, None) == ra.RA_ERR_SHAPE
    assert lib.ulysses_permute(P, P2, 4, 1024, 32, 128, 3, 0, None) == ra.RA_ERR_UNSUPPORTED
    assert lib.ulysses_permute(P, P, 4, 1024, 32, 128, 2, 0, None) == ra.RA_ERR_SHAPE  # in == out
    assert lib.cp_reorder(P, P2, 1000, 32, 128, 2, 8, 1, 0, None) == ra.RA_ERR_DIVISIBILITY
    assert lib.cp_reorder(P, P2, 1000, 32, 128, 2, 3, 2, 0, None) == ra.RA_ERR_DIVISIBILITY
    assert lib.cp_reorder(P, P2, 1024, 32, 128, 2, 4, 5, 0, None) == ra.RA_ERR_UNSUPPORTED
    assert lib.cp_reorder(P, P2, 1024, 32, 128, 2, 4, 1, 2, None) == ra.RA_ERR_SHAPE
    assert lib.cp_reorder(None, P2, 1024, 32, 128, 2, 4, 1, 0, None) == ra.RA_ERR_NULL


def bwd(sh, cu=None, n_docs=0, cp=4, rank=0, part=1, ws=P, ws_bytes=1 << 40, q=P, out=P, lse=P, dout=P, dq=P,
        dk=P, dv=P):
    arr = None
    if cu is not None:
        arr = (ctypes.c_int32 * len(cu))(*cu)
    return _lib().ra_backward(q, P, P, out, lse, dout, arr, n_docs, cp, rank, part, ctypes.byref(sh), dq, dk, dv,
                              ws, ws_bytes, None)


def test_backward_validation_codes():
    for kw in ("q", "out", "lse", "dout", "dq", "dk", "dv"):
        assert bwd(shape(), **{kw: None}) == ra.RA_ERR_NULL, kw
    assert _lib().ra_backward(P, P, P, P, P, P, None, 0, 4, 0, 1, None, P, P, P, P, 1 << 40, None) == ra.RA_ERR_NULL
    assert bwd(shape(s_total=0)) == ra.RA_ERR_SHAPE
    assert bwd(shape(), rank=4) == ra.RA_ERR_RANK
    assert bwd(shape(hq=32, hkv=5)) == ra.RA_ERR_HEADS
    assert bwd(shape(d=80)) == ra.RA_ERR_UNSUPPORTED
    assert bwd(shape(), part=7) == ra.RA_ERR_UNSUPPORTED
    assert bwd(shape(s_total=4 * 1001), part=1) == ra.RA_ERR_DIVISIBILITY
    assert bwd(shape(s_total=64, hq=2, hkv=2), cu=[0, 70, 64], n_docs=2) == ra.RA_ERR_CU_SEQLENS
    # fp32 gradients of one rank's rows must stay below 2^31 bytes (bf16 inputs pass the forward's bound)
    big = shape(s_total=4 * 65536, hq=64, hkv=64, d=128)
    assert bwd(big) == ra.RA_ERR_SHAPE
    sh = shape()
    need = ra.ra_backward_workspace_size(sh, 4, 0)
    assert need > ra.ra_workspace_size(sh, 4, 0)
    assert bwd(sh, ws=None) == ra.RA_ERR_WORKSPACE
    assert bwd(sh, ws_bytes=1024) == ra.RA_ERR_WORKSPACE
    assert ra.ra_backward_workspace_size(shape(s_total=0), 4, 0) == 0
    assert _lib().ra_backward_workspace_size(None, 4, 0) == 0
    assert ra.ra_backward_workspace_size(sh, 4, 50) > need


def test_ulysses_strided_and_usp_validation():
    lib = _lib()
    blk = 4 * 1024 * 8 * 128 * 2  # n s_local (h/n) d elem for n=4, s_local=1024, h=32, d=128, bf16
    assert lib.ulysses_permute_strided(P, P2, 4, 1024, 32, 128, 2, 0, blk - 2, None) == ra.RA_ERR_SHAPE  # < block
    assert lib.ulysses_permute_strided(P, P2, 4, 1024, 32, 128, 2, 0, blk + 2, None) == ra.RA_ERR_SHAPE  # not runs
    assert lib.ulysses_permute_strided(P, P2, 4, 1024, 30, 128, 2, 0, blk, None) == ra.RA_ERR_HEADS
    assert lib.ulysses_permute_strided(None, P2, 4, 1024, 32, 128, 2, 0, blk, None) == ra.RA_ERR_NULL
    # the strided span (3 * 2 blk + blk) of the output would reach the input
    near = ctypes.c_void_p(0x100000 + 7 * blk - 16)
    assert lib.ulysses_permute_strided(near, P, 4, 1024, 32, 128, 2, 0, 2 * blk, None) == ra.RA_ERR_SHAPE
    sh = shape(s_total=65536, hq=32, hkv=8)

    def usp(sh, U=4, R=2, part=1, ws=P, ws_bytes=1 << 40, cu=None, n_docs=0, q=P):
        arr = None if cu is None else (ctypes.c_int32 * len(cu))(*cu)
        return lib.usp_forward(q, P, P, arr, n_docs, U, R, part, ctypes.byref(sh), P, P, ws, ws_bytes, None)

    assert usp(sh, q=None) == ra.RA_ERR_NULL
    assert usp(sh, U=16) == ra.RA_ERR_HEADS        # 8 KV heads cannot split 16 ways
    assert usp(sh, U=3) == ra.RA_ERR_HEADS
    assert usp(shape(s_total=4 * 1001, hq=4, hkv=4), U=4, R=2, part=0) == ra.RA_ERR_DIVISIBILITY  # 2002 % 4 != 0
    assert usp(sh, R=0) == ra.RA_ERR_SHAPE
    assert usp(sh, U=0) == ra.RA_ERR_SHAPE
    need = ra.usp_workspace_size(sh, 4, 2, 0)
    assert need > 0
    assert usp(sh, ws_bytes=need - 1) == ra.RA_ERR_WORKSPACE
    assert ra.usp_workspace_size(sh, 3, 2, 0) == 0


def test_doc_zigzag_validation_and_lengths():
    lib = _lib()
    cu = [0, 100, 101, 333, 512]
    arr = (ctypes.c_int32 * len(cu))(*cu)
    # local length: the largest rank's pieces, each padded to whole 256-slot granules
    for S, cp, c in ((512, 4, cu), (510, 4, None), (131072, 8, None), (2600, 3, [0, 1000, 1001, 2600]),
                     (131072, 8, list(synth.loguniform_cu_seqlens(0, 131072, 512, 32768)))):
        assert ra.ra_local_length(S, cp, "doc_zigzag", c) == oracle_local_length(
            "doc_zigzag", S, cp, None if c is None else np.asarray(c)), (S, cp)
    assert ra.ra_local_length(512, 4, "zigzag", cu) == 128
    assert ra.ra_local_length(510, 4, "zigzag") == -1          # not divisible by 2cp
    assert ra.ra_local_length(510, 4, "doc_zigzag") == 256     # pieces [0, 256) and [256, 510) on two ranks
    assert ra.ra_local_length(131072, 8, "doc_zigzag") == 16384  # one document: the zigzag split
    assert ra.ra_local_length(512, 4, "doc_zigzag", [0, 600, 512]) == -1
    assert ra.ra_doc_workspace_size(512, 4, cu) > 0
    # a doc-zigzag plan is sized by its documents and runs through ra_forward_planned_docs;
    # ra_forward_planned (no cu_seqlens) and the Ulysses x Ring grid do not take doc-zigzag
    sh = shape(s_total=512, hq=2, hkv=2)
    need = ra.ra_workspace_size(sh, 4, 4)
    assert lib.ra_plan(ctypes.byref(sh), arr, 4, 4, 0, 3, P, 64, None) == ra.RA_ERR_WORKSPACE
    assert lib.ra_plan(ctypes.byref(sh), bad_cu := (ctypes.c_int32 * 3)(0, 600, 512), 2, 4, 0, 3, P, need, None) \
        == ra.RA_ERR_CU_SEQLENS
    assert lib.ra_forward_planned(P, P, P, 4, 4, 0, 3, ctypes.byref(sh), P, P, P, 1 << 40, None) \
        == ra.RA_ERR_UNSUPPORTED
    assert lib.ra_forward_planned_docs(None, P, P, arr, 4, 4, 0, ctypes.byref(sh), P, P, P, need, None) \
        == ra.RA_ERR_NULL
    assert lib.ra_forward_planned_docs(P, P, P, bad_cu, 2, 4, 0, ctypes.byref(sh), P, P, P, need, None) \
        == ra.RA_ERR_CU_SEQLENS
    assert lib.ra_forward_planned_docs(P, P, P, arr, 4, 4, 4, ctypes.byref(sh), P, P, P, need, None) \
        == ra.RA_ERR_RANK
    assert lib.ra_forward_planned_docs(P, P, P, arr, 4, 4, 0, ctypes.byref(sh), P, P, P, 64, None) \
        == ra.RA_ERR_WORKSPACE
    assert lib.usp_forward(P, P, P, arr, 4, 2, 2, 3, ctypes.byref(sh), P, P, P, 1 << 40, None) \
        == ra.RA_ERR_UNSUPPORTED
    assert lib.cp_reorder(P, P2, 512, 2, 128, 2, 4, 3, 0, None) == ra.RA_ERR_UNSUPPORTED
    # doc-zigzag classification: tiles of 16..128 only, and the document tables' workspace
    assert lib.ra_classify(ctypes.byref(sh), arr, 4, 4, 0, 3, 96, 64, P, P, 1 << 20, None) == ra.RA_ERR_UNSUPPORTED
    assert lib.ra_classify(ctypes.byref(sh), arr, 4, 4, 0, 3, 64, 64, P, P, 64, None) == ra.RA_ERR_WORKSPACE
    # reorder: tensors, documents and workspace
    assert lib.cp_reorder_docs(None, P2, 512, 2, 128, 2, 4, arr, 4, 0, P, 1 << 20, None) == ra.RA_ERR_NULL
    bad = (ctypes.c_int32 * 3)(0, 600, 512)
    assert lib.cp_reorder_docs(P, P2, 512, 2, 128, 2, 4, bad, 2, 0, P, 1 << 20, None) == ra.RA_ERR_CU_SEQLENS
    assert lib.cp_reorder_docs(P, P2, 512, 2, 128, 2, 4, arr, 4, 0, P, 64, None) == ra.RA_ERR_WORKSPACE
    # the forward's workspace size covers the doc-zigzag layout
    assert fwd(sh, cu=cu, n_docs=4, part=3, ws_bytes=ra.ra_workspace_size(sh, 4, 4) - 1, q=None) == ra.RA_ERR_NULL


def test_noalloc_validation_codes():
    lib = _lib()
    sh = shape()

    def na(sh, q=P, out=P, cp=4, rank=0, part=1):
        return lib.ra_forward_noalloc(q, P, P, None, 0, cp, rank, part, ctypes.byref(sh), out, P, None)

    assert na(sh, q=None) == ra.RA_ERR_NULL
    assert na(sh, out=None) == ra.RA_ERR_NULL
    assert na(sh, rank=4) == ra.RA_ERR_RANK
    assert na(shape(d=96)) == ra.RA_ERR_UNSUPPORTED
    assert na(shape(s_total=4 * 1001)) == ra.RA_ERR_DIVISIBILITY
    # 2^20 tokens on one rank: a 256 MiB plan, above the fixed scratch (refused before any launch)
    assert na(shape(s_total=1 << 20, hq=1, hkv=1, d=64), cp=1, part=0) == ra.RA_ERR_SCRATCH
    # the largest workload shapes fit: 131072 tokens on one rank, 8 x 16384 under doc-zigzag bounds
    big = shape(s_total=131072, hq=8, hkv=8, d=128)
    assert ra.ra_workspace_size(big, 1, 0) <= ra.NOALLOC_SCRATCH_BYTES
    assert ra.ra_workspace_size(shape(s_total=131072), 8, 32) <= ra.NOALLOC_SCRATCH_BYTES


def test_probe_validation_codes():
    lib = _lib()
    assert lib.ra_probe_mfma(10, 4, 8, None, None) == ra.RA_ERR_NULL
    assert lib.ra_probe_mfma(0, 4, 8, P, None) == ra.RA_ERR_SHAPE
    assert lib.ra_probe_mfma(10, 0, 8, P, None) == ra.RA_ERR_SHAPE
    assert lib.ra_probe_mfma(10, 4, 6, P, None) == ra.RA_ERR_SHAPE
