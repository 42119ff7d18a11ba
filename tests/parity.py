"""Shared helpers of the parity tests: run the HIP path, run the oracle on the
same bytes, compare with the stated tolerances.

Tolerances (per output element, in fp64 on the GPU's converted values):
  out : max |gpu - oracle| <= 1e-2 for bf16 caches, 3e-2 for e4m3 caches,
        plus, where the output itself is bf16, half a bf16 ulp of the
        oracle's value (the output format's own rounding: 2^-9 |x| at most,
        0.0156 for |x| in [4, 8), which no kernel writing bf16 can avoid)
  lse : |gpu - oracle| <= 1e-3 * max(1, |oracle|); -inf must match -inf
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from mla_paged_latent_03_amd import workloads as wl

TOL_OUT = {"bf16": 1e-2, "fp8": 3e-2}
TOL_LSE_REL = 1e-3


def oracle_rows(inp: wl.DecodeInputs, rows=None, num_splits=0, threads=None):
    """fp64 oracle on the exact bytes of ``inp`` (moved to the CPU)."""
    q_nope = wl.as_numpy_bits(inp.q_nope)
    q_pe = wl.as_numpy_bits(inp.q_pe)
    kv = wl.as_numpy_bits(inp.kv_cache)
    topk = None if inp.topk_indices is None else inp.topk_indices.cpu().numpy()
    return oracle.decode(q_nope, q_pe, kv, inp.block_table.cpu().numpy(), inp.seq_lens.cpu().numpy(),
                         softmax_scale=inp.softmax_scale, q_scale=inp.q_scale, kv_scale=inp.kv_scale,
                         topk_indices=topk, num_splits=num_splits, rows=rows, threads=threads)


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values at |x| (8 significant bits): the most
    that rounding x to the nearest bf16 can change it, for normal x."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), 0.0)


def compare(out_gpu: torch.Tensor, lse_gpu: torch.Tensor, ref_out: np.ndarray, ref_lse: np.ndarray, kv_dtype: str,
            rows=None, what=""):
    """Element-wise check; returns (max out error, max lse error) for reporting."""
    o = out_gpu.detach().to(torch.float64).cpu().reshape(-1, 512).numpy()
    l = lse_gpu.detach().to(torch.float64).cpu().reshape(-1).numpy()
    if rows is not None:
        o = o[rows]
        l = l[rows]
    assert o.shape == ref_out.shape, (o.shape, ref_out.shape)
    assert np.all(np.isfinite(o)), "%s: non-finite output" % what
    err = np.abs(o - ref_out)
    max_err = float(err.max()) if err.size else 0.0
    tol = TOL_OUT[kv_dtype]
    # (at the larger of the two magnitudes: the rounded value may sit across a power of two)
    allowed = tol + (half_ulp_bf16(np.maximum(np.abs(ref_out), np.abs(o))) if out_gpu.dtype == torch.bfloat16
                     else 0.0)
    excess = err - allowed
    if excess.size and float(excess.max()) > 0.0:
        r, c = np.unravel_index(np.argmax(excess), err.shape)
        raise AssertionError("%s: |out - oracle| = %.3g > %.3g at row %d (oracle %.4g)"
                             % (what, float(err[r, c]), float(np.broadcast_to(allowed, err.shape)[r, c]), int(r),
                                float(ref_out[r, c])))
    ninf_ref = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), ninf_ref), "%s: -inf lse mismatch" % what
    fin = ~ninf_ref
    lerr = np.abs(l[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))
    max_lerr = float(lerr.max()) if lerr.size else 0.0
    assert max_lerr <= TOL_LSE_REL, "%s: lse rel err %.3g" % (what, max_lerr)
    return max_err, max_lerr


def sample_rows(n_total: int, n: int, seed: int) -> np.ndarray:
    """First, last, and random rows in between (sorted, distinct)."""
    g = np.random.default_rng(seed)
    picks = {0, n_total - 1}
    picks.update(g.choice(n_total, size=min(n, n_total), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)
