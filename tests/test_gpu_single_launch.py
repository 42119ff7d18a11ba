"""GPU parity of the single-launch form (MLA_SINGLE_LAUNCH=1): the split
units merge their partials themselves inside the first kernel.

Each case compares the single-launch result with the two-launch result on
the same inputs (same plan and arithmetic, so the same bits) and with the
fp64 oracle.  The group words it uses live in the workspace and need no
clearing: a workspace of random bytes, graph replays and calls of other
shapes in between are covered.
"""
import os
import sys

import numpy as np
import pytest
import torch

from mla_paged_latent_03_amd import binding, workloads as wl
from parity import compare, oracle_rows, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class single_launch:
    """Requests the single-launch form for the calls inside the block."""

    def __enter__(self):
        self.old = os.environ.get("MLA_SINGLE_LAUNCH")
        os.environ["MLA_SINGLE_LAUNCH"] = "1"

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("MLA_SINGLE_LAUNCH", None)
        else:
            os.environ["MLA_SINGLE_LAUNCH"] = self.old


def _fused_planned(inp, splits):
    fp8 = inp.kv_dtype == "fp8"
    two = binding.workspace_size(inp.B, inp.T, inp.H, inp.max_seq_len, inp.K, fp8, splits)
    with single_launch():
        one = binding.workspace_size(inp.B, inp.T, inp.H, inp.max_seq_len, inp.K, fp8, splits)
    return one > two


def _both(inp, splits, what, rows=None, garbage=False):
    g = inp.to(DEV)
    _say("[gpu] single launch: %s (splits=%s)" % (what, splits))
    assert _fused_planned(inp, splits), "the single-launch form is not planned for this shape"
    o2, l2, _ = binding.decode(g, num_kv_splits=splits)
    with single_launch():
        fp8 = inp.kv_dtype == "fp8"
        need = binding.workspace_size(inp.B, inp.T, inp.H, inp.max_seq_len, inp.K, fp8, splits)
        ws = torch.empty((need + 3) // 4, device=DEV, dtype=torch.float32)
        if garbage:
            ws.view(torch.int32).random_(generator=torch.Generator(device=DEV).manual_seed(5))
        o1, l1, _ = binding.decode(g, num_kv_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "single launch differs from two launches"
    ref_o, ref_l = oracle_rows(inp, rows=rows)
    e = compare(o1, l1, ref_o, ref_l, inp.kv_dtype, rows=rows, what=what)
    _say("[gpu] single launch %s: max |out - oracle| %.4g, lse rel %.3g" % ((what,) + e))


def test_tiny_workload():
    _both(wl.workload("tiny_b2_h16_kv37-300", poison=True, extra_pages=3), 0, "tiny")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_skewed_lengths_balanced_pieces(kv_dtype):
    lens = [8192] + [1, 0, 10, 64, 65] * 12 + [130, 3000, 700]
    inp = wl.make_inputs(len(lens), 16, 1, lens, kv_dtype=kv_dtype, out_dtype="f32", seed=155, poison=True)
    _both(inp, 0, "skewed lengths %s" % kv_dtype, garbage=True)


@pytest.mark.parametrize("H,T,K,kv_dtype", [(128, 1, 2048, "bf16"), (128, 1, 2048, "fp8"), (64, 2, 512, "bf16")])
def test_sparse(H, T, K, kv_dtype):
    inp = wl.make_inputs(8, H, T, [6000, 1500] * 4, kv_dtype=kv_dtype, out_dtype="bf16", topk=K, seed=156 + H,
                         poison=True)
    _both(inp, 0, "sparse H=%d T=%d K=%d %s" % (H, T, K, kv_dtype))


def test_feature_split_long_units():
    """Four-wave feature-split fp8 units over 16384 tokens, four splits."""
    inp = wl.make_inputs(16, 32, 4, (70000, 80000), kv_dtype="fp8", out_dtype="bf16", seed=157)
    rows = sample_rows(16 * 128, 96, seed=157)
    _both(inp, 4, "feature split long units", rows=rows)


def test_graph_replay_and_calls_in_between():
    """A captured single-launch call replays with the same call number: its
    group words must be back at zero after every call, also with calls of
    other shapes on the same workspace in between."""
    inp = wl.make_inputs(4, 32, 4, [20000, 900, 7000, 64], kv_dtype="fp8", out_dtype="bf16", seed=158).to(DEV)
    small = wl.make_inputs(2, 16, 1, [300, 40], kv_dtype="fp8", out_dtype="bf16", seed=159).to(DEV)
    assert _fused_planned(inp, 3) and _fused_planned(small, 2)
    with single_launch():
        need = max(binding.workspace_size(inp.B, inp.T, inp.H, inp.max_seq_len, 0, True, 3),
                   binding.workspace_size(small.B, small.T, small.H, small.max_seq_len, 0, True, 2))
        ws = torch.empty((need + 3) // 4, device=DEV, dtype=torch.float32)
        eager_o, eager_l, _ = binding.decode(inp, num_kv_splits=3, workspace=ws)
        torch.cuda.synchronize()
        out = torch.empty_like(eager_o)
        lse = torch.empty_like(eager_l)
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            binding.decode(inp, num_kv_splits=3, out=out, lse=lse, workspace=ws)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                binding.decode(inp, num_kv_splits=3, out=out, lse=lse, workspace=ws, stream=s)
        _say("[gpu] single launch: graph replays")
        for rep in range(4):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager_o) and torch.equal(lse, eager_l), "replay %d differs" % rep
            so, sl, _ = binding.decode(small, num_kv_splits=2, workspace=ws)   # other shape, same workspace
            torch.cuda.synchronize()
    ref_o, ref_l = oracle_rows(small.to("cpu"))
    compare(so, sl, ref_o, ref_l, "fp8", what="call between replays")
    ref_o, ref_l = oracle_rows(inp.to("cpu"))
    compare(eager_o, eager_l, ref_o, ref_l, "fp8", what="captured call")


# A seeded random sweep of small shapes with the single-launch form
# requested (the library plans it where every unit is resident at once and
# falls back to two launches elsewhere), every row against the oracle.
def _random_cases(n=30, seed=20261206):
    import test_gpu_random_shapes as rs
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = ["bf16", "fp8", "sparse_bf16", "sparse_fp8"][i % 4]
        sparse = kind.startswith("sparse")
        B, T = int(g.integers(1, 7)), int(g.integers(1, 9))
        H = int(g.choice([1, 5, 16, 32, 40, 64, 128]))
        K = int(g.choice([32, 96, 200, 512])) if sparse else 0
        l_max = 8 * K + 100 if sparse else min(4000, max(8, rs.PAIR_CAP // (B * T * H)))
        lens = [int(g.choice(rs.SPECIAL_LENS)) if g.random() < 0.3 else int(g.integers(1, l_max + 1))
                for _ in range(B)]
        if max(lens) == 0:
            lens[0] = 1
        if sparse and B * T * H * K > rs.PAIR_CAP:
            H = max(1, rs.PAIR_CAP // (B * T * K))
        cases.append(dict(kind=kind, B=B, T=T, H=H, K=K, lens=lens, splits=int(g.choice([0, 2, 3, 5])),
                          seed=1200 + i))
    return cases


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=["%s-B%d-T%d-H%d-K%d-S%d" % (c["kind"], c["B"], c["T"], c["H"], c["K"],
                                                                          c["splits"]) for c in RANDOM])
def test_single_launch_random_shapes(case):
    kv_dtype = "fp8" if case["kind"].endswith("fp8") else "bf16"
    inp = wl.make_inputs(case["B"], case["H"], case["T"], case["lens"], kv_dtype=kv_dtype, out_dtype="f32",
                         topk=case["K"] or None, seed=case["seed"], poison=True)
    what = "single launch random %s lens=%s" % (case["kind"], case["lens"])
    _say("[gpu] %s" % what)
    with single_launch():
        out, lse, _ = binding.decode(inp.to(DEV), num_kv_splits=case["splits"])
        torch.cuda.synchronize()
    ref_o, ref_l = oracle_rows(inp)
    compare(out, lse, ref_o, ref_l, kv_dtype, what=what)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "sparse_bf16", "sparse_fp8"])
def test_device_data_rules_and_no_lse_match_two_launches(kind):
    """Invalid page ids, a seq_len past the block table (within max_seq_len)
    and lse = NULL through the single-launch form: the same bits as the two
    launches, with and without lse."""
    kv_dtype = "fp8" if kind.endswith("fp8") else "bf16"
    K = 200 if kind.startswith("sparse") else None
    inp = wl.make_inputs(2, 16, 2, [300, 700], kv_dtype=kv_dtype, out_dtype="f32", topk=K, seed=157)
    bad = inp.block_table.clone()
    bad[0, 2] = inp.NB + 5
    bad[1, 1] = -3
    inp.block_table = bad
    inp.seq_lens = torch.tensor([300, 5000], dtype=torch.int32)     # 5000 clamps to the 11-page table
    inp.max_len = 5000
    splits = 3
    assert _fused_planned(inp, splits)
    g = inp.to(DEV)
    fp8 = kv_dtype == "fp8"
    _say("[gpu] single launch: device-data rules, %s" % kind)
    results = []
    for fused in (False, True):
        old = os.environ.get("MLA_SINGLE_LAUNCH")
        if fused:
            os.environ["MLA_SINGLE_LAUNCH"] = "1"
        try:
            o, l, _ = binding.decode(g, num_kv_splits=splits)
            need = binding.workspace_size(g.B, g.T, g.H, g.max_seq_len, g.K, fp8, splits)
            ws = torch.empty((need + 3) // 4, device=DEV, dtype=torch.float32)
            o_nl = torch.full_like(o, float("nan"))
            if K is not None and fp8:
                binding.mla_sparse_decode_fp8(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.topk_indices,
                                              g.max_seq_len, g.softmax_scale, g.q_scale, g.kv_scale, o_nl, None, ws,
                                              splits)
            elif K is not None:
                binding.mla_sparse_decode(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.topk_indices,
                                          g.max_seq_len, g.softmax_scale, o_nl, None, ws, splits)
            elif fp8:
                binding.mla_decode_fp8(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.max_seq_len,
                                       g.softmax_scale, g.q_scale, g.kv_scale, o_nl, None, ws, splits)
            else:
                binding.mla_decode(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.max_seq_len,
                                   g.softmax_scale, o_nl, None, ws, splits)
            torch.cuda.synchronize()
        finally:
            if old is None:
                os.environ.pop("MLA_SINGLE_LAUNCH", None)
            else:
                os.environ["MLA_SINGLE_LAUNCH"] = old
        assert torch.isfinite(o).all().item() and torch.equal(o, o_nl)
        results.append((o, l))
    assert torch.equal(results[0][0], results[1][0]) and torch.equal(results[0][1], results[1][1])
