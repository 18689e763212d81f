"""Thin ctypes binding of libmi355_attn.so.

The functions carry the C ABI's names and do argument marshalling only:
tensor pointers, shapes and the current HIP stream go to the library, every
step of the computation runs in its kernels.  torch supplies device memory
and streams.  There is no fallback: a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmi355_attn.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "mi355_attn.h")

ATTN_OK = 0


class attn_shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("groups", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


class attn_varlen_shape(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("groups", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


class gla_shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


class smla_shape(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int32),
        ("kv_tokens", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("dim_qk", ctypes.c_int32),
        ("dim_v", ctypes.c_int32),
    ]


_lib = None


def library():
    """Load the shared library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m attention_backward_fwd_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.attn_strerror.restype = ctypes.c_char_p
        lib.attn_strerror.argtypes = [ctypes.c_int]
        lib.attn_fwd.restype = ctypes.c_int
        lib.attn_fwd.argtypes = [P, P, P, P, P, attn_shape, ctypes.c_float, ctypes.c_int, P]
        lib.attn_bwd_preprocess.restype = ctypes.c_int
        lib.attn_bwd_preprocess.argtypes = [P, P, P, P, attn_shape, P]
        lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_bwd_workspace_bytes.argtypes = [attn_shape, ctypes.c_int, ctypes.c_int]
        lib.attn_bwd.restype = ctypes.c_int
        lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, attn_shape, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_int, P]
        lib.attn_bwd_postprocess.restype = ctypes.c_int
        lib.attn_bwd_dq_sum.restype = ctypes.c_int
        lib.attn_bwd_dq_sum.argtypes = [P, ctypes.c_size_t, P, attn_shape, ctypes.c_int, P]
        lib.attn_bwd_noalloc.restype = ctypes.c_int
        lib.attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, attn_shape, ctypes.c_float, ctypes.c_int, P]
        lib.attn_bwd_postprocess.argtypes = [P, P, ctypes.c_size_t, P, P, P, attn_shape, P]
        lib.attn_merge.restype = ctypes.c_int
        lib.attn_merge.argtypes = [P, P, ctypes.c_int, P, P, attn_shape, P]
        lib.attn_fwd_varlen.restype = ctypes.c_int
        lib.attn_fwd_varlen.argtypes = [P, P, P, P, P, P, P, attn_varlen_shape, ctypes.c_float, ctypes.c_int, P]
        lib.attn_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_bwd_varlen_workspace_bytes.argtypes = [attn_varlen_shape, ctypes.c_int, ctypes.c_int]
        lib.attn_bwd_varlen.restype = ctypes.c_int
        lib.attn_bwd_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, P, attn_varlen_shape,
                                        ctypes.c_float, ctypes.c_int, ctypes.c_int, P]
        lib.attn_bwd_varlen_postprocess.restype = ctypes.c_int
        lib.attn_bwd_varlen_postprocess.argtypes = [P, P, ctypes.c_size_t, P, P, P, attn_varlen_shape, P]
        lib.gla_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gla_chunk_bwd_workspace_bytes.argtypes = [gla_shape]
        lib.gla_chunk_bwd.restype = ctypes.c_int
        lib.gla_chunk_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, gla_shape, ctypes.c_float, P]
        lib.attn_sparse_mla_fwd.restype = ctypes.c_int
        lib.attn_sparse_mla_fwd.argtypes = [P, P, P, P, P, smla_shape, ctypes.c_float, P]
        lib.attn_sparse_mla_bwd_preprocess.restype = ctypes.c_int
        lib.attn_sparse_mla_bwd_preprocess.argtypes = [P, P, P, P, smla_shape, P]
        lib.attn_sparse_mla_bwd.restype = ctypes.c_int
        lib.attn_sparse_mla_bwd.argtypes = [P, P, P, P, P, P, P, P, smla_shape, ctypes.c_float, P]
        lib.attn_sparse_mla_bwd_postprocess.restype = ctypes.c_int
        lib.attn_sparse_mla_bwd_postprocess.argtypes = [P, P, smla_shape, P]
        lib.attn_sparse_mla_bwd_split_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_sparse_mla_bwd_split_workspace_bytes.argtypes = [smla_shape]
        lib.attn_sparse_mla_bwd_split.restype = ctypes.c_int
        lib.attn_sparse_mla_bwd_split.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_size_t, smla_shape,
                                                  ctypes.c_float, P]
        _lib = lib
    return _lib


def header_functions():
    """Names of the functions include/mi355_attn.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:attn|gla)_[a-z_]+)\s*\(", text)))


class AttnError(RuntimeError):
    def __init__(self, status, where):
        msg = library().attn_strerror(status).decode()
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


def _check(status, where):
    if status != ATTN_OK:
        raise AttnError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_shape(batch, seqlen, heads_q, groups, head_dim):
    return attn_shape(batch, seqlen, heads_q, groups, head_dim)


def shape_of(q, k):
    """attn_shape from BSHD q [B,S,Hq,D] and k [B,S,Hkv,D]."""
    b, s, hq, d = q.shape
    hkv = k.shape[2]
    if hkv < 1 or hq % hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return attn_shape(b, s, hq, hq // hkv, d)


# ------------------------------------------------------------ the C ABI calls

def attn_fwd(q, k, v, o, lse, shape, softmax_scale, causal, stream=None):
    _check(library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), shape, float(softmax_scale),
                              int(causal), _stream(stream)), "attn_fwd")


def attn_bwd_preprocess(o, dout, delta, dq_accum, shape, stream=None):
    _check(library().attn_bwd_preprocess(_ptr(o), _ptr(dout), _ptr(delta), _ptr(dq_accum), shape,
                                         _stream(stream)), "attn_bwd_preprocess")


def attn_bwd_workspace_bytes(shape, causal, use_atomic):
    return int(library().attn_bwd_workspace_bytes(shape, int(causal), int(use_atomic)))


def attn_bwd(q, k, v, dout, lse, delta, dq_accum, dk, dv, workspace, shape, softmax_scale, causal,
             use_atomic, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq_accum),
                              _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, shape, float(softmax_scale),
                              int(causal), int(use_atomic), _stream(stream)), "attn_bwd")


def attn_bwd_dq_sum(workspace, dq_accum, shape, causal, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().attn_bwd_dq_sum(_ptr(workspace), ws_bytes, _ptr(dq_accum), shape, int(causal),
                                     _stream(stream)), "attn_bwd_dq_sum")


def attn_bwd_noalloc(q, k, v, dout, lse, delta, dq_accum, dk, dv, shape, softmax_scale, causal, stream=None):
    _check(library().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                                      _ptr(dq_accum), _ptr(dk), _ptr(dv), shape, float(softmax_scale),
                                      int(causal), _stream(stream)), "attn_bwd_noalloc")


def attn_bwd_postprocess(dq_accum, workspace, dq, dk, dv, shape, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().attn_bwd_postprocess(_ptr(dq_accum), _ptr(workspace), ws_bytes, _ptr(dq), _ptr(dk),
                                          _ptr(dv), shape, _stream(stream)), "attn_bwd_postprocess")


def attn_merge(o_parts, lse_parts, n_parts, o, lse, shape, stream=None):
    _check(library().attn_merge(_ptr(o_parts), _ptr(lse_parts), int(n_parts), _ptr(o), _ptr(lse), shape,
                                _stream(stream)), "attn_merge")


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, shape, softmax_scale, causal, stream=None):
    _check(library().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                                     _ptr(cu_seqlens_k), shape, float(softmax_scale), int(causal), _stream(stream)),
           "attn_fwd_varlen")


def attn_bwd_varlen_workspace_bytes(shape, causal, use_atomic):
    return int(library().attn_bwd_varlen_workspace_bytes(shape, int(causal), int(use_atomic)))


def attn_bwd_varlen(q, k, v, dout, lse, delta, dq_accum, dk, dv, workspace, cu_seqlens_q, cu_seqlens_k, shape,
                    softmax_scale, causal, use_atomic, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                                     _ptr(dq_accum), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                                     _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), shape, float(softmax_scale),
                                     int(causal), int(use_atomic), _stream(stream)), "attn_bwd_varlen")


def attn_bwd_varlen_postprocess(dq_accum, workspace, dq, dk, dv, shape, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().attn_bwd_varlen_postprocess(_ptr(dq_accum), _ptr(workspace), ws_bytes, _ptr(dq), _ptr(dk),
                                                 _ptr(dv), shape, _stream(stream)), "attn_bwd_varlen_postprocess")


def attn_sparse_mla_fwd(q, kv, indices, o, lse, shape, softmax_scale, stream=None):
    _check(library().attn_sparse_mla_fwd(_ptr(q), _ptr(kv), _ptr(indices), _ptr(o), _ptr(lse), shape,
                                         float(softmax_scale), _stream(stream)), "attn_sparse_mla_fwd")


def attn_sparse_mla_bwd_preprocess(o, dout, delta, dkv_accum, shape, stream=None):
    _check(library().attn_sparse_mla_bwd_preprocess(_ptr(o), _ptr(dout), _ptr(delta), _ptr(dkv_accum), shape,
                                                    _stream(stream)), "attn_sparse_mla_bwd_preprocess")


def attn_sparse_mla_bwd(q, kv, dout, indices, lse, delta, dq, dkv_accum, shape, softmax_scale, stream=None):
    _check(library().attn_sparse_mla_bwd(_ptr(q), _ptr(kv), _ptr(dout), _ptr(indices), _ptr(lse), _ptr(delta),
                                         _ptr(dq), _ptr(dkv_accum), shape, float(softmax_scale), _stream(stream)),
           "attn_sparse_mla_bwd")


def attn_sparse_mla_bwd_postprocess(dkv_accum, dkv, shape, stream=None):
    _check(library().attn_sparse_mla_bwd_postprocess(_ptr(dkv_accum), _ptr(dkv), shape, _stream(stream)),
           "attn_sparse_mla_bwd_postprocess")


def attn_sparse_mla_bwd_split_workspace_bytes(shape):
    return int(library().attn_sparse_mla_bwd_split_workspace_bytes(shape))


def attn_sparse_mla_bwd_split(q, kv, dout, indices, lse, delta, dq, dkv, workspace, shape, softmax_scale,
                              stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().attn_sparse_mla_bwd_split(_ptr(q), _ptr(kv), _ptr(dout), _ptr(indices), _ptr(lse), _ptr(delta),
                                               _ptr(dq), _ptr(dkv), _ptr(workspace), ws_bytes, shape,
                                               float(softmax_scale), _stream(stream)),
           "attn_sparse_mla_bwd_split")


def gla_chunk_bwd_workspace_bytes(shape):
    return int(library().gla_chunk_bwd_workspace_bytes(shape))


def gla_chunk_bwd(q, k, v, g, dout, dq, dk, dv, dg, workspace, shape, scale, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().gla_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _ptr(dg), _ptr(workspace), ws_bytes, shape, float(scale), _stream(stream)),
           "gla_chunk_bwd")


# ------------------------------------------------------------ conveniences

def _require_gpu_inputs(*ts):
    for t in ts:
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("inputs must be contiguous bf16 tensors on the GPU")


def forward(q, k, v, causal, scale, stream=None):
    """O, LSE = attention(q, k, v); allocates the outputs with torch."""
    _require_gpu_inputs(q, k, v)
    shape = shape_of(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, o, lse, shape, scale, causal, stream)
    return o, lse


class BwdBuffers:
    """Outputs and scratch of one backward problem, allocated once."""

    def __init__(self, q, k, causal, use_atomic):
        self.shape = shape_of(q, k)
        dev = q.device
        b, s, hq, d = q.shape
        self.delta = torch.empty((b, hq, s), dtype=torch.float32, device=dev)
        self.dq_accum = torch.empty((b, hq, s, d), dtype=torch.float32, device=dev)  # head-major
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(k)
        self.dv = torch.empty_like(k)
        nbytes = attn_bwd_workspace_bytes(self.shape, causal, use_atomic)
        self.workspace = torch.empty(max(nbytes, 0) // 4, dtype=torch.float32, device=dev) if nbytes else None


def backward(q, k, v, o, lse, do, causal, scale, use_atomic=True, buffers=None, stream=None):
    """dQ, dK, dV via preprocess -> bwd (-> sum) -> postprocess."""
    _require_gpu_inputs(q, k, v, o, do)
    bb = buffers or BwdBuffers(q, k, causal, use_atomic)
    sh = bb.shape
    attn_bwd_preprocess(o, do, bb.delta, bb.dq_accum if use_atomic else None, sh, stream)
    attn_bwd(q, k, v, do, lse, bb.delta, bb.dq_accum, bb.dk, bb.dv, bb.workspace, sh, scale, causal, use_atomic,
             stream)
    attn_bwd_postprocess(bb.dq_accum, bb.workspace, bb.dq, bb.dk, bb.dv, sh, stream)
    return bb.dq, bb.dk, bb.dv


def merge(o_parts, lse_parts, stream=None):
    """O, LSE merged over the parts: o_parts [P,B,S,Hq,D] bf16, lse_parts
    [P,B,Hq,S] fp32 (contiguous, on the GPU)."""
    _require_gpu_inputs(o_parts)
    if not lse_parts.is_cuda or lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous():
        raise ValueError("lse_parts must be a contiguous fp32 GPU tensor")
    n, b, s, hq, d = o_parts.shape
    if lse_parts.shape != (n, b, hq, s):
        raise ValueError("lse_parts must be [P, B, Hq, S] matching o_parts")
    shape = attn_shape(b, s, hq, 1, d)
    o = torch.empty((b, s, hq, d), dtype=torch.bfloat16, device=o_parts.device)
    lse = torch.empty((b, hq, s), dtype=torch.float32, device=o_parts.device)
    attn_merge(o_parts, lse_parts, n, o, lse, shape, stream)
    return o, lse


def varlen_shape_of(q, k, n_seqs, max_seqlen_q, max_seqlen_k=None):
    """attn_varlen_shape from packed q [Tq,Hq,D] and k [Tk,Hkv,D]."""
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    if hkv < 1 or hq % hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    mk = max_seqlen_q if max_seqlen_k is None else max_seqlen_k
    return attn_varlen_shape(n_seqs, tq, tk, max_seqlen_q, mk, hq, hq // hkv, d)


def _require_cu(cu):
    if not cu.is_cuda or cu.dtype != torch.int32 or not cu.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor on the GPU")


def forward_varlen(q, k, v, cu_seqlens_q, max_seqlen_q, causal, scale, cu_seqlens_k=None, max_seqlen_k=None,
                   stream=None):
    """Packed sequences: O [Tq,Hq,D], LSE [Hq,Tq]; allocates the outputs.
    Keys default to the query offsets and bound."""
    _require_gpu_inputs(q, k, v)
    cu_k = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
    _require_cu(cu_seqlens_q)
    _require_cu(cu_k)
    shape = varlen_shape_of(q, k, cu_seqlens_q.numel() - 1, max_seqlen_q, max_seqlen_k)
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_k, shape, scale, causal, stream)
    return o, lse


class VarlenBwdBuffers:
    """Outputs and scratch of one packed-sequence backward problem."""

    def __init__(self, q, k, n_seqs, max_seqlen_q, causal, use_atomic, max_seqlen_k=None):
        self.shape = varlen_shape_of(q, k, n_seqs, max_seqlen_q, max_seqlen_k)
        tq, hq, d = q.shape
        dev = q.device
        # The preprocess sees the packed query tensors as one batch.
        self.dense = attn_shape(1, tq, hq, self.shape.groups, d)
        self.delta = torch.empty((hq, tq), dtype=torch.float32, device=dev)
        self.dq_accum = torch.empty((hq, tq, d), dtype=torch.float32, device=dev)
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(k)
        self.dv = torch.empty_like(k)
        nbytes = attn_bwd_varlen_workspace_bytes(self.shape, causal, use_atomic)
        self.workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=dev) if nbytes else None


def backward_varlen(q, k, v, o, lse, do, cu_seqlens_q, max_seqlen_q, causal, scale, use_atomic=True,
                    buffers=None, cu_seqlens_k=None, max_seqlen_k=None, stream=None):
    """Packed sequences: dQ, dK, dV via preprocess -> bwd (-> sum) -> postprocess."""
    _require_gpu_inputs(q, k, v, o, do)
    cu_k = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
    _require_cu(cu_seqlens_q)
    _require_cu(cu_k)
    bb = buffers or VarlenBwdBuffers(q, k, cu_seqlens_q.numel() - 1, max_seqlen_q, causal, use_atomic,
                                     max_seqlen_k)
    if q.shape[0] > 0:
        attn_bwd_preprocess(o, do, bb.delta, bb.dq_accum if use_atomic else None, bb.dense, stream)
    attn_bwd_varlen(q, k, v, do, lse, bb.delta, bb.dq_accum, bb.dk, bb.dv, bb.workspace, cu_seqlens_q, cu_k,
                    bb.shape, scale, causal, use_atomic, stream)
    attn_bwd_varlen_postprocess(bb.dq_accum, bb.workspace, bb.dq, bb.dk, bb.dv, bb.shape, stream)
    return bb.dq, bb.dk, bb.dv


class GlaBuffers:
    """Outputs and workspace of one simple-GLA chunk backward problem."""

    def __init__(self, q):
        b, t, h, d = q.shape
        self.shape = gla_shape(b, t, h, d)
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(q)
        self.dv = torch.empty_like(q)
        self.dg = torch.empty((b, t, h), dtype=torch.float32, device=q.device)
        nbytes = gla_chunk_bwd_workspace_bytes(self.shape)
        self.workspace = torch.empty(nbytes // 4 + 1, dtype=torch.float32, device=q.device)


def gla_backward(q, k, v, g, do, scale, buffers=None, stream=None):
    """dq, dk, dv, dg of simple gated linear attention (q/k/v/do [B,T,H,128]
    bf16, g [B,T,H] fp32)."""
    _require_gpu_inputs(q, k, v, do)
    if not g.is_cuda or g.dtype != torch.float32 or not g.is_contiguous():
        raise ValueError("g must be a contiguous fp32 GPU tensor")
    bb = buffers or GlaBuffers(q)
    gla_chunk_bwd(q, k, v, g, do, bb.dq, bb.dk, bb.dv, bb.dg, bb.workspace, bb.shape, scale, stream)
    return bb.dq, bb.dk, bb.dv, bb.dg


def smla_shape_of(q, kv, indices):
    t, h, dqk = q.shape
    return smla_shape(t, kv.shape[0], h, indices.shape[1], dqk, 512)


def sparse_mla_forward(q, kv, indices, scale, stream=None):
    """O [T,H,512], LSE [T,H] of sparse MLA (q [T,H,576], kv [Tk,576] bf16,
    indices [T,K] int32 on the GPU)."""
    _require_gpu_inputs(q, kv)
    if not indices.is_cuda or indices.dtype != torch.int32 or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous int32 GPU tensor")
    shape = smla_shape_of(q, kv, indices)
    o = torch.empty((q.shape[0], q.shape[1], 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    attn_sparse_mla_fwd(q, kv, indices, o, lse, shape, scale, stream)
    return o, lse


class SmlaBwdBuffers:
    """Outputs and scratch of one sparse MLA backward problem: the fp32 dKV
    accumulator of the atomic path, or (use_atomic=False, given the index
    tensor) the deterministic path's workspace."""

    def __init__(self, q, kv, use_atomic=True, indices=None):
        t, h, _ = q.shape
        self.use_atomic = bool(use_atomic)
        self.delta = torch.empty((t, h), dtype=torch.float32, device=q.device)
        self.dq = torch.empty_like(q)
        self.dkv = torch.empty_like(kv)
        if self.use_atomic:
            self.dkv_accum = torch.empty((kv.shape[0], 576), dtype=torch.float32, device=q.device)
            self.workspace = None
        else:
            if indices is None:
                raise ValueError("the deterministic path sizes its workspace from the index tensor")
            n = attn_sparse_mla_bwd_split_workspace_bytes(smla_shape_of(q, kv, indices))
            if n == 0:
                raise ValueError("invalid sparse MLA shape")
            self.dkv_accum = None
            self.workspace = torch.empty(n, dtype=torch.uint8, device=q.device)


def sparse_mla_backward(q, kv, indices, o, lse, do, scale, buffers=None, stream=None, use_atomic=True):
    """dq [T,H,576], dkv [Tk,576] via preprocess -> backward -> postprocess
    (fp32 atomic dKV), or with use_atomic=False via preprocess -> the
    deterministic backward (per-entry partial rows, fixed-order sum)."""
    _require_gpu_inputs(q, kv, o, do)
    shape = smla_shape_of(q, kv, indices)
    bb = buffers or SmlaBwdBuffers(q, kv, use_atomic, indices)
    if bb.use_atomic:
        attn_sparse_mla_bwd_preprocess(o, do, bb.delta, bb.dkv_accum, shape, stream)
        attn_sparse_mla_bwd(q, kv, do, indices, lse, bb.delta, bb.dq, bb.dkv_accum, shape, scale, stream)
        attn_sparse_mla_bwd_postprocess(bb.dkv_accum, bb.dkv, shape, stream)
    else:
        attn_sparse_mla_bwd_preprocess(o, do, bb.delta, None, shape, stream)
        attn_sparse_mla_bwd_split(q, kv, do, indices, lse, bb.delta, bb.dq, bb.dkv, bb.workspace, shape, scale,
                                  stream)
    return bb.dq, bb.dkv
