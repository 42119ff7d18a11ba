"""ctypes front end of libmla_decode.so (C ABI: include/mla_decode.h).

Argument marshalling only: every step of the decode runs in the library's
HIP kernels.  Tensors are torch tensors on the current GPU; the library sees
their device pointers and the current torch stream.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

(MLA_OK, MLA_ERR_INVALID_ARGUMENT, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP,
 MLA_ERR_SCRATCH_LIMIT) = range(6)
STATIC_SCRATCH_BYTES = 64 << 20
MLA_OUT_BF16, MLA_OUT_F32 = 0, 1
MAX_KV_SPLITS = 256
EXPORTS = ("mla_status_string", "mla_num_kv_splits", "mla_launch_waves", "mla_workspace_size",
           "mla_decode", "mla_decode_fp8", "mla_decode_fp8_noalloc",
           "mla_sparse_decode", "mla_sparse_decode_fp8", "mla_merge_partials", "mla_dense_mha",
           "mla_dense_mha_workspace_size")
MHA_MAX_Q_LEN = 65536

_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libmla_decode.so not built at %s (run __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    c_int, c_float, c_size, vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [c_int]
    lib.mla_num_kv_splits.restype = c_int
    lib.mla_num_kv_splits.argtypes = [c_int] * 6
    lib.mla_launch_waves.restype = c_int
    lib.mla_launch_waves.argtypes = [c_int] * 6
    lib.mla_workspace_size.restype = c_size
    lib.mla_workspace_size.argtypes = [c_int] * 7
    common_tail = [c_float, vp, c_int, vp, vp, c_size, c_int, vp]
    lib.mla_decode.restype = c_int
    lib.mla_decode.argtypes = [vp, vp, vp, vp, vp] + [c_int] * 7 + common_tail
    lib.mla_decode_fp8.restype = c_int
    lib.mla_decode_fp8.argtypes = [vp, vp, vp, vp, vp] + [c_int] * 7 + [c_float, c_float, c_float] + common_tail[1:]
    lib.mla_decode_fp8_noalloc.restype = c_int
    lib.mla_decode_fp8_noalloc.argtypes = ([vp, vp, vp, vp, vp] + [c_int] * 7 + [c_float, c_float, c_float, vp, c_int, vp,
                                           c_int, vp])
    lib.mla_sparse_decode.restype = c_int
    lib.mla_sparse_decode.argtypes = [vp, vp, vp, vp, vp, vp, c_int] + [c_int] * 7 + common_tail
    lib.mla_sparse_decode_fp8.restype = c_int
    lib.mla_sparse_decode_fp8.argtypes = ([vp, vp, vp, vp, vp, vp, c_int] + [c_int] * 7 + [c_float, c_float, c_float]
                                          + common_tail[1:])
    lib.mla_dense_mha_workspace_size.restype = c_size
    lib.mla_dense_mha_workspace_size.argtypes = [c_int] * 3
    lib.mla_dense_mha.restype = c_int
    lib.mla_dense_mha.argtypes = [vp] * 7 + [c_int] * 7 + [c_float, vp, c_int, vp, vp, c_size, vp]
    lib.mla_merge_partials.restype = c_int
    lib.mla_merge_partials.argtypes = [vp, ctypes.c_int64, c_int, vp, c_int, vp, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mla_status_string(int(status)).decode()


def num_kv_splits(batch, q_len, num_heads, max_seq_len, topk=0, kv_fp8=False) -> int:
    return load().mla_num_kv_splits(batch, q_len, num_heads, max_seq_len, topk, int(bool(kv_fp8)))


def launch_waves(batch, q_len, num_heads, max_seq_len, topk=0, kv_fp8=False) -> int:
    """Waves per workgroup (1, 2 or 4) the library launches for this shape."""
    return load().mla_launch_waves(batch, q_len, num_heads, max_seq_len, topk, int(bool(kv_fp8)))


def workspace_size(batch, q_len, num_heads, max_seq_len, topk=0, kv_fp8=False, num_kv_splits=0) -> int:
    return load().mla_workspace_size(batch, q_len, num_heads, max_seq_len, topk, int(bool(kv_fp8)),
                                     num_kv_splits)




def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _out_code(out: Optional[torch.Tensor]) -> int:
    if out is None:
        return MLA_OUT_F32
    if out.dtype == torch.bfloat16:
        return MLA_OUT_BF16
    if out.dtype == torch.float32:
        return MLA_OUT_F32
    raise ValueError("out must be bfloat16 or float32")


def _check(status, where):
    if status != MLA_OK:
        raise MLAError(status, where)


def mla_decode(q_nope, q_pe, kv_cache, block_table, seq_lens, max_seq_len, softmax_scale, out, lse=None,
               workspace=None, num_kv_splits=0, stream=None):
    """Dense bf16 decode (mla_decode).  Shapes as in the C header."""
    B, T, H, _ = q_nope.shape
    NB, P, _ = kv_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().mla_decode(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), B, T, H,
                           NB, P, block_table.shape[1], int(max_seq_len), float(softmax_scale), _ptr(out),
                           _out_code(out), _ptr(lse), _ptr(workspace), ws_bytes, int(num_kv_splits),
                           _stream(stream))
    _check(st, "mla_decode")


def mla_decode_fp8(q_nope, q_pe, kv_cache, block_table, seq_lens, max_seq_len, softmax_scale, q_scale,
                   kv_scale, out, lse=None, workspace=None, num_kv_splits=0, stream=None):
    """Dense e4m3 decode (mla_decode_fp8).  q_nope / q_pe / kv_cache hold uint8 e4m3fn bytes."""
    B, T, H, _ = q_nope.shape
    NB, P, _ = kv_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().mla_decode_fp8(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), B, T,
                               H, NB, P, block_table.shape[1], int(max_seq_len), float(softmax_scale),
                               float(q_scale), float(kv_scale), _ptr(out), _out_code(out), _ptr(lse),
                               _ptr(workspace), ws_bytes, int(num_kv_splits), _stream(stream))
    _check(st, "mla_decode_fp8")


def mla_decode_fp8_noalloc(q_nope, q_pe, kv_cache, block_table, seq_lens, max_seq_len, softmax_scale, q_scale,
                           kv_scale, out, lse=None, num_kv_splits=0, stream=None):
    """mla_decode_fp8 with the split partials in the library's static buffer
    (mla_decode_fp8_noalloc): no workspace argument, nothing allocated."""
    B, T, H, _ = q_nope.shape
    NB, P, _ = kv_cache.shape
    st = load().mla_decode_fp8_noalloc(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
                                       B, T, H, NB, P, block_table.shape[1], int(max_seq_len), float(softmax_scale),
                                       float(q_scale), float(kv_scale), _ptr(out), _out_code(out), _ptr(lse),
                                       int(num_kv_splits), _stream(stream))
    _check(st, "mla_decode_fp8_noalloc")


def mla_sparse_decode(q_nope, q_pe, kv_cache, block_table, seq_lens, topk_indices, max_seq_len, softmax_scale,
                      out, lse=None, workspace=None, num_kv_splits=0, stream=None):
    """Top-k sparse bf16 decode (mla_sparse_decode)."""
    B, T, H, _ = q_nope.shape
    NB, P, _ = kv_cache.shape
    K = topk_indices.shape[2]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().mla_sparse_decode(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
                                  _ptr(topk_indices), K, B, T, H, NB, P, block_table.shape[1], int(max_seq_len),
                                  float(softmax_scale), _ptr(out), _out_code(out), _ptr(lse), _ptr(workspace),
                                  ws_bytes, int(num_kv_splits), _stream(stream))
    _check(st, "mla_sparse_decode")


def mla_sparse_decode_fp8(q_nope, q_pe, kv_cache, block_table, seq_lens, topk_indices, max_seq_len, softmax_scale,
                          q_scale, kv_scale, out, lse=None, workspace=None, num_kv_splits=0, stream=None):
    """Top-k sparse e4m3 decode (mla_sparse_decode_fp8)."""
    B, T, H, _ = q_nope.shape
    NB, P, _ = kv_cache.shape
    K = topk_indices.shape[2]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().mla_sparse_decode_fp8(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(topk_indices), K, B, T, H, NB, P, block_table.shape[1],
                                      int(max_seq_len), float(softmax_scale), float(q_scale), float(kv_scale),
                                      _ptr(out), _out_code(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                      int(num_kv_splits), _stream(stream))
    _check(st, "mla_sparse_decode_fp8")


def dense_mha_workspace_size(batch, num_heads, max_seq_len) -> int:
    return load().mla_dense_mha_workspace_size(batch, num_heads, max_seq_len)


def mla_dense_mha(q_nope, q_pe, kv_cache, block_table, seq_lens, w_uk, w_uv, max_seq_len, softmax_scale, out,
                  lse=None, workspace=None, stream=None):
    """Dense un-absorbed MHA (mla_dense_mha).  q_nope [B,T,H,128], q_pe [B,T,H,64],
    w_uk / w_uv [H,128,512] bf16; out [B,T,H,128].  Allocates the workspace with
    torch when not given; returns it."""
    B, T, H, _ = q_nope.shape
    NB, P, _ = kv_cache.shape
    if workspace is None:
        need = dense_mha_workspace_size(B, H, int(max_seq_len))
        workspace = torch.empty(max(1, (need + 1) // 2), device=q_nope.device, dtype=torch.bfloat16)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().mla_dense_mha(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
                              _ptr(w_uk), _ptr(w_uv), B, T, H, NB, P, block_table.shape[1], int(max_seq_len),
                              float(softmax_scale), _ptr(out), _out_code(out), _ptr(lse), _ptr(workspace), ws_bytes,
                              _stream(stream))
    _check(st, "mla_dense_mha")
    return workspace


def mla_merge_partials(workspace, rows, num_kv_splits, out, lse=None, stream=None):
    """Second stage alone (mla_merge_partials): LSE merge of [rows, S, 513] partials."""
    st = load().mla_merge_partials(_ptr(workspace), int(rows), int(num_kv_splits), _ptr(out), _out_code(out),
                                   _ptr(lse), _stream(stream))
    _check(st, "mla_merge_partials")


def decode(inp, num_kv_splits=0, out=None, lse=None, workspace=None, stream=None):
    """Run the entry point that matches a ``workloads.DecodeInputs`` on the GPU.

    Allocates out / lse / workspace with torch when not given (sizes from
    the library); returns (out, lse, workspace).
    """
    dev = inp.q_nope.device
    B, T, H = inp.B, inp.T, inp.H
    K = inp.K
    fp8 = inp.kv_dtype == "fp8"
    if out is None:
        out = torch.empty((B, T, H, 512), device=dev,
                          dtype=torch.float32 if inp.out_dtype == "f32" else torch.bfloat16)
    if lse is None:
        lse = torch.empty((B, T, H), device=dev, dtype=torch.float32)
    msl = inp.max_seq_len
    need = workspace_size(B, T, H, msl, K, fp8, num_kv_splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need + 3) // 4, device=dev, dtype=torch.float32)
    if K > 0 and fp8:
        mla_sparse_decode_fp8(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, inp.topk_indices,
                              msl, inp.softmax_scale, inp.q_scale, inp.kv_scale, out, lse, workspace,
                              num_kv_splits, stream)
    elif K > 0:
        mla_sparse_decode(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, inp.topk_indices, msl,
                          inp.softmax_scale, out, lse, workspace, num_kv_splits, stream)
    elif fp8:
        mla_decode_fp8(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, msl, inp.softmax_scale,
                       inp.q_scale, inp.kv_scale, out, lse, workspace, num_kv_splits, stream)
    else:
        mla_decode(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, msl, inp.softmax_scale, out,
                   lse, workspace, num_kv_splits, stream)
    return out, lse, workspace


def prepare_decode(inp, num_kv_splits=0, out=None, lse=None, workspace=None, stream=None):
    """The entry point that matches ``inp`` with its arguments marshalled once:
    returns a callable that makes the same C call each time it is invoked
    (for timing loops, where per-call marshalling would show up as host time).
    out = lse = None runs the first stage only, as the entry points do."""
    lib = load()
    B, T, H = inp.B, inp.T, inp.H
    NB, P, _ = inp.kv_cache.shape
    MB = inp.block_table.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fp8 = inp.kv_dtype == "fp8"
    head = [_ptr(inp.q_nope), _ptr(inp.q_pe), _ptr(inp.kv_cache), _ptr(inp.block_table), _ptr(inp.seq_lens)]
    scales = [float(inp.q_scale), float(inp.kv_scale)] if fp8 else []
    dims = [B, T, H, NB, P, MB, int(inp.max_seq_len), float(inp.softmax_scale)]
    tail = [_ptr(out), _out_code(out), _ptr(lse), _ptr(workspace), ws_bytes, int(num_kv_splits), _stream(stream)]
    if inp.K > 0:
        fn = lib.mla_sparse_decode_fp8 if fp8 else lib.mla_sparse_decode
        args = head + [_ptr(inp.topk_indices), inp.K] + dims + scales + tail
    else:
        fn = lib.mla_decode_fp8 if fp8 else lib.mla_decode
        args = head + dims + scales + tail
    name = fn.__name__

    def call():
        st = fn(*args)
        if st != MLA_OK:
            raise MLAError(st, name)
    return call


def prepare_merge(workspace, rows, num_kv_splits, out, lse=None, stream=None):
    """mla_merge_partials with its arguments marshalled once (see prepare_decode)."""
    lib = load()
    args = [_ptr(workspace), int(rows), int(num_kv_splits), _ptr(out), _out_code(out), _ptr(lse), _stream(stream)]

    def call():
        st = lib.mla_merge_partials(*args)
        if st != MLA_OK:
            raise MLAError(st, "mla_merge_partials")
    return call

