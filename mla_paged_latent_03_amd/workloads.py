"""Seeded synthetic decode inputs.

This module only builds inputs: random values, page tables, sequence lengths
and top-k index lists.  It holds none of the decode arithmetic, so both the
HIP path and the fp64 oracle can consume the same bytes.

Recipe (the pages run an unnamed microbenchmark at num_heads=32, bs=64,
kv_len=80k with MTP-3 / MTP-7 drafts, vLLM PR #41778 digest, "Motivation";
DeepSeek-R1 MLA dims, same digest, "Risks and impact" item 4; top-k sparse
decode with index_topk per query token, vLLM PR #47327 digest, "Key code
excerpt"):

* values ~ N(0, 1) drawn in fp32, rounded to bf16 (round-to-nearest-even);
  for fp8, one per-tensor scale amax / 448 and a saturating cast to OCP
  e4m3fn (one scale for q_nope and q_pe together, one for the cache);
* each sequence b owns ceil(L_b / 64) pages of 64 tokens; a random
  permutation of the page pool is handed out in order, so logical pages are
  scattered; unused block-table slots hold -1;
* top-k indices are, per (b, t), the first K entries of a random
  permutation of 0 .. L_b - 1 (distinct, unsorted), padded with -1 when
  L_b < K;
* structure (lengths, pages, indices) comes from a CPU generator seeded with
  ``seed``; values come from a generator on ``device`` seeded with ``seed``,
  so the bytes depend on the device that draws them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence, Tuple, Union

import torch

D_LATENT, D_ROPE, D_TOKEN = 512, 64, 576
PAGE = 64
E4M3_MAX = 448.0
BF16_NAN_BITS = 0x7FC0
E4M3_NAN_BYTE = 0x7F
DEFAULT_SOFTMAX_SCALE = 1.0 / math.sqrt(128 + 64)


@dataclass
class DecodeInputs:
    q_nope: torch.Tensor          # [B, T, H, 512] bf16, or uint8 e4m3fn bytes
    q_pe: torch.Tensor            # [B, T, H, 64]
    kv_cache: torch.Tensor        # [NB, P, 576] bf16, or uint8 e4m3fn bytes
    block_table: torch.Tensor     # [B, MB] int32, -1 = unused
    seq_lens: torch.Tensor        # [B] int32
    topk_indices: Optional[torch.Tensor]  # [B, T, K] int32 or None
    kv_dtype: str                 # "bf16" | "fp8"
    out_dtype: str                # "bf16" | "f32"
    softmax_scale: float
    q_scale: float = 1.0
    kv_scale: float = 1.0
    name: str = "custom"
    seed: int = 0
    meta: dict = field(default_factory=dict)
    max_len: Optional[int] = None   # host copy of max(seq_lens); taken once, never during graph capture

    def __post_init__(self):
        if self.max_len is None:
            self.max_len = int(self.seq_lens.max().item()) if self.seq_lens.numel() else 0

    @property
    def B(self) -> int:
        return self.q_nope.shape[0]

    @property
    def T(self) -> int:
        return self.q_nope.shape[1]

    @property
    def H(self) -> int:
        return self.q_nope.shape[2]

    @property
    def NB(self) -> int:
        return self.kv_cache.shape[0]

    @property
    def P(self) -> int:
        return self.kv_cache.shape[1]

    @property
    def MB(self) -> int:
        return self.block_table.shape[1]

    @property
    def K(self) -> int:
        return 0 if self.topk_indices is None else self.topk_indices.shape[2]

    @property
    def max_seq_len(self) -> int:
        return self.max_len

    def to(self, device) -> "DecodeInputs":
        def mv(t):
            return None if t is None else t.to(device)
        return DecodeInputs(mv(self.q_nope), mv(self.q_pe), mv(self.kv_cache), mv(self.block_table),
                            mv(self.seq_lens), mv(self.topk_indices), self.kv_dtype, self.out_dtype,
                            self.softmax_scale, self.q_scale, self.kv_scale, self.name, self.seed,
                            dict(self.meta), self.max_len)


# Workloads named by what they are.  Lengths: a list gives them outright, a
# (lo, hi) pair draws each one uniformly from [lo, hi].
WORKLOADS = {
    "tiny_b2_h16_kv37-300": dict(B=2, H=16, T=1, seq_lens=[37, 300], kv_dtype="bf16", out_dtype="f32", seed=1001),
    "r1_b128_h16_kv1k-8k_bf16": dict(B=128, H=16, T=1, seq_lens=(1024, 8192), kv_dtype="bf16", out_dtype="bf16",
                                     seed=1002),
    "mtp3_b64_h32_kv80k_fp8": dict(B=64, H=32, T=4, seq_lens=[80000] * 64, kv_dtype="fp8", out_dtype="bf16",
                                   seed=1003),
    "mtp7_b32_h128_kv16k-32k_bf16": dict(B=32, H=128, T=8, seq_lens=(16384, 32768), kv_dtype="bf16",
                                         out_dtype="bf16", seed=1004),
    "sparse_b64_h128_kv64k_top2048_bf16": dict(B=64, H=128, T=1, seq_lens=[65536] * 64, kv_dtype="bf16",
                                               out_dtype="bf16", topk=2048, seed=1005),
    # The same top-2048 selection over an e4m3 cache (the fp8 sparse variant).
    "sparse_b64_h128_kv64k_top2048_fp8": dict(B=64, H=128, T=1, seq_lens=[65536] * 64, kv_dtype="fp8",
                                              out_dtype="bf16", topk=2048, seed=1006),
}


def _quantize_e4m3(x: torch.Tensor) -> Tuple[torch.Tensor, float]:
    """Per-tensor scale amax / 448 and a saturating cast to e4m3fn bytes."""
    amax = float(x.abs().max().item()) if x.numel() else 0.0
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    scale = float(torch.tensor(scale, dtype=torch.float32).item())  # the fp32 value a kernel receives
    y = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return y.view(torch.uint8), scale


def make_inputs(B: int, H: int, T: int, seq_lens: Union[Sequence[int], Tuple[int, int]], *,
                kv_dtype: str = "bf16", out_dtype: str = "bf16", topk: Optional[int] = None,
                seed: int = 0, device: Union[str, torch.device] = "cpu", block_size: int = PAGE,
                softmax_scale: float = DEFAULT_SOFTMAX_SCALE, extra_pages: int = 0,
                extra_table_cols: int = 0, poison: bool = False, name: str = "custom",
                edit_values: Optional[Callable] = None) -> DecodeInputs:
    """Draw one decode batch.

    ``edit_values(kv, q, block_table, lens)``, if given, may change the fp32
    values in place after they are drawn and before they are rounded (kv
    [pool, 64, 576], q [B, T, H, 576] on ``device``; block_table and lens on
    the CPU); tests use it to shape particular rows.

    ``poison`` fills every page slot no sequence owns (the pages beyond the
    pool, and the slots past L_b in each sequence's last page) with NaN, so a
    kernel that reads them shows it.  ``extra_pages`` adds unreferenced pages
    to the pool; ``extra_table_cols`` adds -1 columns to the block table.
    """
    if kv_dtype not in ("bf16", "fp8"):
        raise ValueError("kv_dtype must be bf16 or fp8")
    device = torch.device(device)
    g_cpu = torch.Generator().manual_seed(seed)
    g_val = torch.Generator(device=device).manual_seed(seed)

    if isinstance(seq_lens, tuple):
        lo, hi = seq_lens
        lens = torch.randint(lo, hi + 1, (B,), generator=g_cpu, dtype=torch.int64)
    else:
        lens = torch.tensor(list(seq_lens), dtype=torch.int64)
        if lens.numel() != B:
            raise ValueError("need one length per sequence")
    n_pages = [(int(l) + block_size - 1) // block_size for l in lens]
    pool = sum(n_pages) + extra_pages
    perm = torch.randperm(pool, generator=g_cpu).to(torch.int32)
    MB = max(n_pages + [0]) + extra_table_cols
    block_table = torch.full((B, max(MB, 1)), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(n_pages):
        block_table[b, :n] = perm[off:off + n]
        off += n

    topk_indices = None
    if topk is not None:
        topk_indices = torch.full((B, T, topk), -1, dtype=torch.int32)
        for b in range(B):
            L = int(lens[b])
            for t in range(T):
                sel = torch.randperm(L, generator=g_cpu)[:topk].to(torch.int32)
                topk_indices[b, t, :sel.numel()] = sel

    # Values.
    kv32 = torch.randn((pool, block_size, D_TOKEN), generator=g_val, device=device, dtype=torch.float32)
    q32 = torch.randn((B, T, H, D_TOKEN), generator=g_val, device=device, dtype=torch.float32)
    if edit_values is not None:
        edit_values(kv32, q32, block_table, lens)
    q_scale = kv_scale = 1.0
    if kv_dtype == "bf16":
        kv = kv32.to(torch.bfloat16)
        q = q32.to(torch.bfloat16)
    else:
        kv, kv_scale = _quantize_e4m3(kv32)
        q, q_scale = _quantize_e4m3(q32)
    del kv32, q32

    if poison:
        owned = torch.zeros((pool, block_size), dtype=torch.bool)
        for b, n in enumerate(n_pages):
            for p in range(n):
                valid = min(block_size, int(lens[b]) - p * block_size)
                owned[int(block_table[b, p]), :valid] = True
        owned = owned.to(device)
        if kv_dtype == "bf16":
            nan = torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).to(device)
        else:
            nan = torch.tensor(E4M3_NAN_BYTE, dtype=torch.uint8).to(device)
        kv[~owned] = nan

    q_nope = q[..., :D_LATENT].contiguous()
    q_pe = q[..., D_LATENT:].contiguous()
    return DecodeInputs(q_nope=q_nope, q_pe=q_pe, kv_cache=kv.contiguous(), block_table=block_table.to(device),
                        seq_lens=lens.to(torch.int32).to(device),
                        topk_indices=None if topk_indices is None else topk_indices.to(device),
                        kv_dtype=kv_dtype, out_dtype=out_dtype, softmax_scale=softmax_scale,
                        q_scale=q_scale, kv_scale=kv_scale, name=name, seed=seed,
                        meta=dict(n_pages=n_pages, pool=pool), max_len=int(lens.max().item()) if B else 0)


def workload(name: str, device="cpu", **overrides) -> DecodeInputs:
    """One of the named workloads (see ``WORKLOADS``), drawn with its seed."""
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    return make_inputs(spec.pop("B"), spec.pop("H"), spec.pop("T"), spec.pop("seq_lens"), device=device,
                       name=name, **spec)


def as_numpy_bits(t: torch.Tensor):
    """CPU numpy view of a tensor's raw bits: bf16 -> uint16, e4m3fn bytes
    -> uint8, integers as they are."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def mha_inputs(inp: DecodeInputs, seed: int, device=None):
    """Inputs of the un-absorbed route for the same cache: an un-absorbed
    no-rope query [B, T, H, 128] and per-head up-projections W_UK, W_UV
    [H, 128, 512], bf16.  Queries ~ N(0, 1); projection entries
    ~ N(0, 1/512), so that the expanded keys and values are about N(0, 1)
    like the latents.  Drawn from a CPU generator."""
    device = inp.q_nope.device if device is None else device
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((inp.B, inp.T, inp.H, 128), generator=g, dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((2, inp.H, 128, D_LATENT), generator=g, dtype=torch.float32) / math.sqrt(D_LATENT))
    w = w.to(torch.bfloat16)
    return q.to(device), w[0].contiguous().to(device), w[1].contiguous().to(device)


def prefill_rows_as_sparse_decode(inp: DecodeInputs, q_abs: torch.Tensor, topk: int) -> DecodeInputs:
    """The same causal attention as a q_len-T call over ``inp``'s cache, laid
    out for the sparse decode: one single-query row per (sequence, query
    token), its index list holding every position that token sees
    (0 .. L - T + t, then -1 up to ``topk``).  ``q_abs`` [B, T, H, 512] is
    the absorbed query; the rope part is ``inp.q_pe``.  Needs
    L - T + t + 1 <= topk for every row."""
    B, T, H = inp.B, inp.T, inp.H
    dev = inp.q_nope.device
    lens = inp.seq_lens.to(torch.int64)
    n_vis = (lens[:, None] - T + torch.arange(T, device=dev)[None, :] + 1).clamp(min=0).reshape(-1)
    if int(n_vis.max().item()) > topk:
        raise ValueError("a row sees more positions than topk")
    pos = torch.arange(topk, device=dev, dtype=torch.int32)[None, :]
    idx = torch.where(pos < n_vis[:, None], pos, torch.full_like(pos, -1))
    return DecodeInputs(q_nope=q_abs.reshape(B * T, 1, H, D_LATENT).contiguous(),
                        q_pe=inp.q_pe.reshape(B * T, 1, H, D_ROPE).contiguous(), kv_cache=inp.kv_cache,
                        block_table=inp.block_table.repeat_interleave(T, dim=0).contiguous(),
                        seq_lens=inp.seq_lens.repeat_interleave(T).contiguous(),
                        topk_indices=idx.reshape(B * T, 1, topk).contiguous(), kv_dtype=inp.kv_dtype,
                        out_dtype=inp.out_dtype, softmax_scale=inp.softmax_scale, name=inp.name + "_as_rows",
                        seed=inp.seed, max_len=inp.max_len)
