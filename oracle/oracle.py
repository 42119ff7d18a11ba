"""ctypes front end of the fp64 C oracle (``mla_oracle.c``).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the bench).

Arrays are numpy: bf16 tensors are passed as their raw ``uint16`` bits,
e4m3fn tensors as raw ``uint8`` bytes with a per-tensor scale, and fp64
tensors as ``float64``.  The C code dequantizes them itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

BF16, E4M3FN, F64 = 0, 1, 2
D_LATENT, D_ROPE, D_TOKEN = 512, 64, 576

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_ERRORS = {-1: "bad argument", -2: "block table entry out of range", -3: "out of memory"}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP, -O2, IEEE semantics kept)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-shared", "-fPIC", "-std=c11",
               "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
            lib.mla_oracle_decode.restype = ctypes.c_int
            lib.mla_oracle_decode.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_double, ctypes.c_int,
                ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ]
            lib.orc_e4m3fn_to_double.restype = ctypes.c_double
            lib.orc_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
            lib.orc_bf16_to_double.restype = ctypes.c_double
            lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
            _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3FN
    if a.dtype == np.float64:
        return F64
    raise TypeError("oracle takes uint16 (bf16 bits), uint8 (e4m3fn bytes) or float64, got %s" % a.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def decode(q_nope, q_pe, kv_cache, block_table, seq_lens, *, softmax_scale, q_scale=1.0,
           kv_scale=1.0, topk_indices=None, num_splits=0, rows=None, threads=None):
    """fp64 MLA decode.

    q_nope [B,T,H,512], q_pe [B,T,H,64], kv_cache [NB,P,576], block_table [B,MB]
    int32, seq_lens [B] int32, topk_indices [B,T,K] int32 or None (dense).
    Returns (out [n,512] float64, lse [n] float64) for the requested flattened
    rows (row = (b*T + t)*H + h), all rows when ``rows`` is None.
    """
    q_nope = np.ascontiguousarray(q_nope)
    q_pe = np.ascontiguousarray(q_pe)
    kv_cache = np.ascontiguousarray(kv_cache)
    qd, kd = _dtype_code(q_nope), _dtype_code(kv_cache)
    if _dtype_code(q_pe) != qd:
        raise TypeError("q_nope and q_pe must share a dtype")
    B, T, H, dn = q_nope.shape
    if dn != D_LATENT or q_pe.shape != (B, T, H, D_ROPE):
        raise ValueError("bad q shapes %s %s" % (q_nope.shape, q_pe.shape))
    NB, P, dt = kv_cache.shape
    if dt != D_TOKEN:
        raise ValueError("kv_cache last dim must be 576")
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if block_table.ndim != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("bad block_table / seq_lens shapes")
    MB = block_table.shape[1]
    K = 0
    if topk_indices is not None:
        topk_indices = np.ascontiguousarray(topk_indices, dtype=np.int32)
        if topk_indices.ndim != 3 or topk_indices.shape[:2] != (B, T):
            raise ValueError("topk_indices must be [B, T, K]")
        K = topk_indices.shape[2]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.shape[0]
    else:
        n = B * T * H
    out = np.zeros((n, D_LATENT), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    if threads is None:
        threads = os.cpu_count() or 1
    rc = _load().mla_oracle_decode(
        _ptr(q_nope), _ptr(q_pe), qd, float(q_scale), _ptr(kv_cache), kd, float(kv_scale),
        _ptr(block_table), _ptr(seq_lens), _ptr(topk_indices), K,
        B, T, H, NB, P, MB, float(softmax_scale), int(num_splits),
        _ptr(rows), n, _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its input: %s" % _ERRORS.get(rc, rc))
    return out, lse


def e4m3fn_to_float64(byte: int) -> float:
    """The oracle's own e4m3fn decoder (format definition), one byte."""
    return _load().orc_e4m3fn_to_double(int(byte))


def bf16_bits_to_float64(bits: int) -> float:
    return _load().orc_bf16_to_double(int(bits))
