"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases compare every output element; they span several tiles, ragged
tails, empty rows, forced split counts, every row-block width and both
cache dtypes.  Full-size workloads run in the launch configuration the
benchmark times and compare sampled rows the oracle computes one by one.
"""
import dataclasses
import math
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


def run_case(inp, num_kv_splits=0, what=""):
    _say("[gpu] %s splits=%s B=%d T=%d H=%d kv=%s K=%d" % (what, num_kv_splits, inp.B, inp.T, inp.H, inp.kv_dtype,
                                                           inp.K))
    g = inp.to(DEV)
    out, lse, _ = binding.decode(g, num_kv_splits=num_kv_splits)
    torch.cuda.synchronize()
    return out, lse


def check_full(inp, num_kv_splits=0, what=""):
    out, lse = run_case(inp, num_kv_splits, what)
    ref_o, ref_l = oracle_rows(inp)
    return compare(out, lse, ref_o, ref_l, inp.kv_dtype, what=what)


def fixed_unit_tokens(max_seq_len, splits):
    """Tokens of a work unit when a call cuts fixed chunks (the rule of the
    C header for calls that are not cut by the actual lengths)."""
    pages = -(-max_seq_len // 64)
    return -(-pages // splits) * 64


# ------------------------------------------------------------------ tiny workload, every split count

@pytest.mark.parametrize("splits", [1, 2, 3, 4, 7, 0])
def test_tiny_workload_all_split_counts(splits):
    inp = wl.workload("tiny_b2_h16_kv37-300", poison=True, extra_pages=3, extra_table_cols=2)
    check_full(inp, splits, "tiny S=%d" % splits)


def test_tiny_workload_split_results_agree():
    # Runs with different split counts round P to bf16 against different
    # reference maxima, so they agree to the bf16 budget, not bit for bit.
    inp = wl.workload("tiny_b2_h16_kv37-300")
    res = [run_case(inp, s, "tiny agree") for s in (1, 2, 5)]
    for o, l in res[1:]:
        assert torch.max(torch.abs(o - res[0][0])).item() < 1e-2
        assert torch.max(torch.abs(l - res[0][1])).item() < 1e-5


# ------------------------------------------------------------------ dense bf16 shapes

@pytest.mark.parametrize("H,T,lens,splits", [
    (16, 1, [1, 63, 64, 65, 700], 0),         # one-token, page-edge and ragged tails
    (16, 1, [1, 63, 64, 65, 700], 3),
    (32, 1, [129, 2000], 0),                  # 32 rows: a two-wave block whose second wave is empty
    (16, 4, [3, 4, 5, 130, 1000], 0),         # MTP: first queries of short sequences see nothing
    (16, 4, [3, 4, 5, 130, 1000], 2),
    (64, 2, [77, 1500], 2),                   # two waves per workgroup
    (128, 1, [300, 1234], 0),                 # four waves per workgroup
    (32, 8, [9, 640, 1111], 3),               # 256 rows: two row blocks
    (128, 8, [100, 900], 0),                  # 1024 rows: eight row blocks
    (24, 3, [50, 513], 0),                    # rows not a multiple of 32
    (40, 8, [90, 2100], 0),                   # 320 rows: the third four-wave block half empty
    (40, 8, [90, 2100], 2),
])
def test_dense_bf16_shapes(H, T, lens, splits):
    inp = wl.make_inputs(len(lens), H, T, lens, kv_dtype="bf16", out_dtype="f32", seed=7 + H + T, poison=True,
                         extra_pages=2)
    check_full(inp, splits, "dense bf16 H=%d T=%d" % (H, T))



@pytest.mark.parametrize("kind", ["bf16", "fp8", "sparse_bf16", "sparse_fp8"])
@pytest.mark.parametrize("splits", [1, 3])
def test_no_lse_in_every_kind(kind, splits):
    """lse = NULL (out only) through each entry point, written by the partial
    kernel (one split) or by the merge (three)."""
    kv_dtype = "fp8" if kind.endswith("fp8") else "bf16"
    K = 160 if kind.startswith("sparse") else None
    inp = wl.make_inputs(3, 16, 2, [90, 400, 1], kv_dtype=kv_dtype, out_dtype="bf16", topk=K, seed=25)
    g = inp.to(DEV)
    out = torch.full((3, 2, 16, 512), float("nan"), device=DEV, dtype=torch.bfloat16)
    _say("[gpu] no lse %s splits=%d" % (kind, splits))
    fp8 = kv_dtype == "fp8"
    need = binding.workspace_size(g.B, g.T, g.H, g.max_seq_len, g.K, fp8, splits)
    ws = torch.empty((need + 3) // 4, device=DEV, dtype=torch.float32) if need > 0 else None
    assert (need > 0) == (splits > 1)
    if K is not None and fp8:
        binding.mla_sparse_decode_fp8(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.topk_indices,
                                      g.max_seq_len, g.softmax_scale, g.q_scale, g.kv_scale, out, None, ws, splits)
    elif K is not None:
        binding.mla_sparse_decode(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.topk_indices,
                                  g.max_seq_len, g.softmax_scale, out, None, ws, splits)
    elif fp8:
        binding.mla_decode_fp8(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.max_seq_len,
                               g.softmax_scale, g.q_scale, g.kv_scale, out, None, ws, splits)
    else:
        binding.mla_decode(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.max_seq_len, g.softmax_scale,
                           out, None, ws, splits)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_rows(inp)
    compare(out, torch.tensor(ref_l), ref_o, ref_l, kv_dtype, what="no lse %s" % kind)


def test_dense_bf16_out_bf16_and_no_lse():
    inp = wl.make_inputs(2, 16, 2, [90, 400], kv_dtype="bf16", out_dtype="bf16", seed=3)
    g = inp.to(DEV)
    out = torch.empty((2, 2, 16, 512), device=DEV, dtype=torch.bfloat16)
    _say("[gpu] dense bf16 no-lse")
    binding.mla_decode(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.max_seq_len, g.softmax_scale,
                       out, None, None, 1)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_rows(inp)
    compare(out, torch.tensor(ref_l), ref_o, ref_l, "bf16", what="no lse")


def test_empty_sequence_gives_zero_and_neg_inf():
    inp = wl.make_inputs(3, 16, 1, [0, 1, 100], kv_dtype="bf16", out_dtype="f32", seed=4)
    for s in (1, 2):
        out, lse = run_case(inp, s, "empty seq")
        assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
        check_full(inp, s, "empty seq")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_single_token_closed_form_is_exact(out_dtype):
    """kv_len 1: out = c_0 and lse = s_0.  The weight is 1; bf16 output is
    bit-exact.  O is normalized by the fp32 sum of the unrounded weight, a
    few fp32 ulps away from 1, so f32 output matches to 1e-6 relative."""
    inp = wl.make_inputs(2, 32, 1, [1, 1], kv_dtype="bf16", out_dtype=out_dtype, seed=5)
    out, lse = run_case(inp, 1, "single token %s" % out_dtype)
    kv = inp.kv_cache.to(torch.float32)
    for b in range(2):
        c0 = kv[int(inp.block_table[b, 0]), 0, :512]
        got = out[b, 0].cpu().float()
        if out_dtype == "bf16":
            assert torch.equal(got, c0.expand(32, 512)), "out must be the token's latent exactly"
        else:
            assert torch.allclose(got, c0.expand(32, 512), rtol=1e-6, atol=0)
        s0 = inp.softmax_scale * (inp.q_nope[b, 0].double() @ kv[int(inp.block_table[b, 0]), 0, :512].double() +
                                  inp.q_pe[b, 0].double() @ kv[int(inp.block_table[b, 0]), 0, 512:].double())
        assert torch.allclose(lse[b, 0].cpu().double(), s0, rtol=1e-5, atol=1e-5)


def test_page_permutation_bit_identical():
    inp = wl.make_inputs(2, 16, 2, [333, 1000], kv_dtype="bf16", out_dtype="f32", seed=6)
    o1, l1 = run_case(inp, 2, "perm a")
    perm = torch.randperm(inp.NB, generator=torch.Generator().manual_seed(1))
    inv = torch.argsort(perm)
    inp2 = wl.DecodeInputs(inp.q_nope, inp.q_pe, inp.kv_cache[perm].contiguous(),
                           torch.where(inp.block_table >= 0, inv[inp.block_table.clamp(min=0)].to(torch.int32),
                                       inp.block_table), inp.seq_lens, None, "bf16", "f32", inp.softmax_scale)
    o2, l2 = run_case(inp2, 2, "perm b")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_row_equals_single_query_call():
    T = 4
    inp = wl.make_inputs(2, 16, T, [70, 515], kv_dtype="bf16", out_dtype="f32", seed=8)
    o, l = run_case(inp, 0, "causal T=4")
    for t in range(T):
        sub = wl.DecodeInputs(inp.q_nope[:, t:t + 1].contiguous(), inp.q_pe[:, t:t + 1].contiguous(), inp.kv_cache,
                              inp.block_table, (inp.seq_lens - T + t + 1).to(torch.int32), None, "bf16", "f32",
                              inp.softmax_scale)
        o1, l1 = run_case(sub, 0, "causal t=%d" % t)
        assert torch.max(torch.abs(o[:, t] - o1[:, 0])).item() < 1e-5
        assert torch.max(torch.abs(l[:, t] - l1[:, 0])).item() < 1e-5


def test_scale_is_read_every_call():
    inp = wl.make_inputs(2, 16, 1, [200, 300], kv_dtype="bf16", out_dtype="f32", seed=9)
    for sc in (inp.softmax_scale, 0.5, 1.0 / 64):
        inp.softmax_scale = sc
        check_full(inp, 0, "scale %.4f" % sc)


# ------------------------------------------------------------------ fp8

@pytest.mark.parametrize("H,T,lens,splits", [
    (32, 4, [4, 100, 300, 700], 0),
    (32, 4, [4, 100, 300, 700], 3),
    (16, 1, [1, 64, 129], 2),
    (128, 2, [257, 1000], 0),
    (48, 5, [300, 3000], 0),                  # 240 rows: the second four-wave block partly empty
    (48, 5, [300, 3000], 3),
])
def test_dense_fp8_shapes(H, T, lens, splits):
    inp = wl.make_inputs(len(lens), H, T, lens, kv_dtype="fp8", out_dtype="f32", seed=11 + H, poison=True,
                         extra_pages=1)
    check_full(inp, splits, "fp8 H=%d T=%d" % (H, T))


def test_fp8_scales_are_read_every_call():
    inp = wl.make_inputs(2, 32, 4, [500, 900], kv_dtype="fp8", out_dtype="f32", seed=12)
    for ks in (inp.kv_scale, inp.kv_scale * 4.0, inp.kv_scale * 0.25):
        inp.kv_scale = ks
        check_full(inp, 0, "fp8 kv_scale %.3g" % ks)


# ------------------------------------------------------------------ edge and limit cases

def test_fp8_long_units_without_residual_product():
    """Units longer than 16384 tokens use one fp8 PV product per block (no
    residual); with 128 rows per sequence and many sequences they run on the
    four-wave feature-split kernel."""
    inp = wl.make_inputs(64, 32, 4, (17000, 19000), kv_dtype="fp8", out_dtype="f32", seed=51)
    assert binding.launch_waves(64, 4, 32, inp.max_len, 0, True) == 4
    out, lse = run_case(inp, 1, "fp8 long units, one split")
    rows = sample_rows(64 * 4 * 32, 96, seed=51)
    ref_o, ref_l = oracle_rows(inp, rows=rows)
    compare(out, lse, ref_o, ref_l, "fp8", rows=rows, what="fp8 long units")


def _plant_dominant_tokens(T, n_dominant, seed, rows=((0, 0),), offset_nats=6.0):
    """edit_values hook: in every sequence b, n_dominant(b) cache positions
    (after the first 64, visible to every draft token) get logits about
    `offset_nats` above the largest other logit of each listed row (t, h),
    within +-0.3 nats of each other, so those rows are dominated by a few
    comparable tokens.  The tokens keep their random latents; only their
    rope part is set (along the row's rope query), in fp32 before rounding."""
    sigma = wl.DEFAULT_SOFTMAX_SCALE

    def edit(kv, q, block_table, lens):
        g = torch.Generator().manual_seed(seed)
        for b in range(q.shape[0]):
            L = int(lens[b])
            n_vis = L - T + 1
            if n_vis <= 64 + 8:
                continue
            pages = block_table[b, :(L + 63) // 64].long().to(kv.device)
            toks = kv[pages].reshape(-1, wl.D_TOKEN)[:n_vis]
            for (t, h) in rows:
                qr = q[b, t, h]
                top = float((toks @ qr).max()) * sigma
                pos = (torch.randperm(n_vis - 64, generator=g)[:n_dominant(b)] + 64).tolist()
                for j in pos:
                    target = top + offset_nats + (float(torch.rand(1, generator=g)) - 0.5) * 0.6
                    pg, sl = int(block_table[b, j // 64]), j % 64
                    c = kv[pg, sl, :wl.D_LATENT]
                    qn, qp = qr[:wl.D_LATENT], qr[wl.D_LATENT:]
                    lam = (target / sigma - float(qn @ c)) / float(qp @ qp)
                    kv[pg, sl, wl.D_LATENT:] = lam * qp
                toks = kv[pages].reshape(-1, wl.D_TOKEN)[:n_vis]
    return edit


@pytest.mark.parametrize("lens,kind", [((20000, 40000), "dominant"), ((20000, 30000), "sink"),
                                       ((20000, 24000), "jump")])
def test_feature_split_long_units_dominant_tokens_and_jump(lens, kind):
    """The headline kernel (four-wave feature-split fp8 step, no residual
    product: units over 16384 tokens) on rows whose weight sits on 2-4
    comparable tokens (the unit reruns with the residual product), on rows
    with one heavy token (the residual product of its tile is added), and on
    a logit more than 2^64 (log2 domain) above the first tile's (the unit
    reruns against the exact maximum); every element of the shaped rows is
    compared."""
    B, T, H = 16, 4, 32
    edit = None
    if kind == "dominant":
        edit = _plant_dominant_tokens(T, lambda b: 2 + b % 3, seed=71, rows=((0, 0), (T - 1, H - 1)))
    elif kind == "sink":
        edit = _plant_dominant_tokens(T, lambda b: 1, seed=73, rows=((0, 0), (T - 1, H - 1)), offset_nats=3.0)
    inp = wl.make_inputs(B, H, T, lens, kv_dtype="fp8", out_dtype="f32", seed=71 + len(kind), device=DEV,
                         edit_values=edit)
    assert binding.launch_waves(B, T, H, inp.max_len, 0, True) == 4
    assert fixed_unit_tokens(int(inp.seq_lens.min()), 1) > 16384
    cpu = inp.to("cpu")
    if kind == "jump":
        _plant_large_logit(cpu, 12345)
        inp = cpu.to(DEV)
    out, lse = run_case(inp, 1, "feature split, %s, units %s" % (kind, lens))
    R = T * H
    shaped = np.array([b * R + r for b in range(B) for r in (0, R - 1)], dtype=np.int64)
    rows = np.unique(np.concatenate([shaped, np.arange(R, 2 * R), sample_rows(B * R, 64, seed=72)]))
    _say("[gpu] oracle on %d rows" % rows.size)
    ref_o, ref_l = oracle_rows(cpu, rows=rows)
    if kind == "jump":
        assert np.max(ref_l) > 80.0
    else:
        # the planted tokens carry much of each shaped row's weight
        assert np.all(ref_l[np.searchsorted(rows, shaped)] > 9.0)
    e = compare(out, lse, ref_o, ref_l, "fp8", rows=rows, what="feature split %s" % kind)
    _say("[gpu] feature split %s: max |out - oracle| %.4g, lse rel %.3g" % ((kind,) + e))


@pytest.mark.parametrize("H,waves", [(16, 2), (64, 1)])
@pytest.mark.parametrize("kind", ["dominant", "sink", "jump", "short"])
def test_narrow_blocks_long_fp8_units(H, waves, kind):
    """One- and two-wave fp8 kernels without the residual product (units
    over 16384 tokens): rows dominated by a few tokens, a large logit jump,
    and short sequences in the same call (their units rerun with the
    residual product)."""
    T = 1
    lens = [20000, 300, 18000, 1] if kind == "short" else [20000, 17500, 19000, 22000]
    B = len(lens)
    edit = None
    if kind == "dominant":
        edit = _plant_dominant_tokens(T, lambda b: 2 + b % 3, seed=81 + H)
    elif kind == "sink":
        edit = _plant_dominant_tokens(T, lambda b: 1, seed=83 + H, offset_nats=3.0)
    inp = wl.make_inputs(B, H, T, lens, kv_dtype="fp8", out_dtype="f32", seed=81 + H + len(kind),
                         poison=True, edit_values=edit)
    if kind == "jump":
        _plant_large_logit(inp, 9999)
    assert binding.launch_waves(B, T, H, inp.max_len, 0, True) == waves
    assert fixed_unit_tokens(inp.max_len, 1) > 16384
    e = check_full(inp, 1, "%d-wave long fp8 units, %s" % (waves, kind))
    _say("[gpu] %d-wave %s: max |out - oracle| %.4g, lse rel %.3g" % ((waves, kind) + e))


@pytest.mark.parametrize("lens,splits", [([300, 9000, 20000, 1], 1), ([40000] * 3 + [300], 2)])
def test_fp8_short_sequence_among_long_units(lens, splits):
    """A call planned for long fp8 units (no residual product) with a short
    sequence in the batch: the short units go to the residual-product launch,
    so their rows keep the fp8 tolerance."""
    inp = wl.make_inputs(len(lens), 32, 4, lens, kv_dtype="fp8", out_dtype="f32", seed=95, poison=True)
    check_full(inp, splits, "fp8 short among long, splits=%d" % splits)


def test_fp8_short_sequence_in_the_long_unit_workload_sampled_rows():
    """The 80k-token MTP-3 shape with its last sequence 300 tokens long, in the
    library's own launch plan: every row of the short sequence and a sample of
    the others."""
    lens = [80000] * 63 + [300]
    inp = wl.make_inputs(64, 32, 4, lens, kv_dtype="fp8", out_dtype="bf16", seed=96, device=DEV)
    out, lse, _ = binding.decode(inp)
    torch.cuda.synchronize()
    R = inp.T * inp.H
    rows = np.unique(np.concatenate([np.arange(63 * R, 64 * R), sample_rows(63 * R, 40, seed=96)]))
    _say("[gpu] short among 80k-token sequences: oracle on %d rows" % rows.size)
    ref_o, ref_l = oracle_rows(inp.to("cpu"), rows=rows)
    compare(out, lse, ref_o, ref_l, "fp8", rows=rows, what="fp8 short among 80k-token sequences")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sequence_past_the_split_cap_is_split(kv_dtype):
    """One split covers at most 1024 pages: a 70000-token sequence needs two,
    the library picks at least that many, and an explicit single split is
    refused before any launch."""
    inp = wl.make_inputs(1, 16, 1, [70000], kv_dtype=kv_dtype, out_dtype="f32", seed=52)
    assert binding.num_kv_splits(1, 1, 16, 70000, 0, kv_dtype == "fp8") >= 2
    check_full(inp, 0, "70000 tokens %s" % kv_dtype)
    with pytest.raises(binding.MLAError):
        binding.decode(inp.to(DEV), num_kv_splits=1)


def test_maximum_split_count_with_empty_splits():
    """MLA_MAX_KV_SPLITS splits over a five-page sequence: most splits see no
    token (lse -inf partials) and the merge must ignore them."""
    inp = wl.make_inputs(2, 16, 1, [300, 70], kv_dtype="bf16", out_dtype="f32", seed=53)
    check_full(inp, binding.MAX_KV_SPLITS, "256 splits")


# ------------------------------------------------------------------ length-balanced pieces

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_skewed_lengths_are_cut_into_balanced_pieces(kv_dtype):
    """One long sequence among many short, empty and one-token ones: the
    device cuts the long one into as many pieces as it has slots, the short
    ones stay whole and mark their other slots empty."""
    lens = [8192] + [1, 0, 10, 64, 65] * 12 + [130, 3000, 700]
    inp = wl.make_inputs(len(lens), 16, 1, lens, kv_dtype=kv_dtype, out_dtype="f32", seed=55, poison=True)
    check_full(inp, 0, "skewed lengths %s" % kv_dtype)


@pytest.mark.parametrize("H,T,kv_dtype", [(32, 4, "fp8"), (32, 8, "bf16"), (64, 2, "bf16"), (128, 1, "fp8")])
def test_mixed_lengths_balanced_pieces_every_row_block(H, T, kv_dtype):
    inp = wl.make_inputs(12, H, T, (200, 6000), kv_dtype=kv_dtype, out_dtype="f32", seed=56 + H + T, poison=True)
    check_full(inp, 0, "mixed lengths H=%d T=%d %s" % (H, T, kv_dtype))


@pytest.mark.parametrize("B,H,T,lens,kv_dtype", [
    (64, 128, 4, (0, 700), "bf16"),      # four row blocks, 64 slots per round: 64 sequences
    (64, 64, 8, (1, 900), "fp8"),
    (32, 128, 8, (300, 1500), "bf16"),   # eight row blocks, 32 slots per round
    (40, 128, 8, [0, 1, 64, 65, 2000] * 8, "fp8"),
])
def test_two_rounds_longest_first(B, H, T, lens, kv_dtype):
    """A matrix-bound batch that fills one round of workgroups but not two
    is cut into two pieces per sequence and run longest piece first."""
    inp = wl.make_inputs(B, H, T, lens, kv_dtype=kv_dtype, out_dtype="f32", seed=60 + B + H + T, poison=True)
    assert binding.num_kv_splits(B, T, H, inp.max_len, 0, kv_dtype == "fp8") == 2
    check_full(inp, 0, "two rounds longest first B=%d H=%d T=%d %s" % (B, H, T, kv_dtype))
    check_full(inp, 2, "two rounds longest first, explicit 2 splits")


def test_two_rounds_longest_first_largest_batch():
    """63 sequences with eight row blocks each: one short of two full rounds."""
    inp = wl.make_inputs(63, 128, 8, (1, 300), kv_dtype="bf16", out_dtype="f32", seed=65, poison=True)
    assert binding.num_kv_splits(63, 8, 128, inp.max_len, 0, False) == 2
    check_full(inp, 0, "two rounds, 63 sequences")


@pytest.mark.parametrize("splits", [1, 2])
def test_feature_split_rows_not_a_multiple_of_128(splits):
    """The feature-split fp8 step with 80 rows (row blocks 2 and 3 partly or
    wholly empty), written directly and as staged partials."""
    inp = wl.make_inputs(2, 40, 2, [40000, 34000], kv_dtype="fp8", out_dtype="f32", seed=66, poison=True)
    assert binding.launch_waves(2, 2, 40, inp.max_len, 0, True) == 4
    check_full(inp, splits, "feature split, 80 rows, %d split(s)" % splits)


def test_two_rounds_longest_first_long_fp8_units_sampled_rows():
    """Two rounds of longest-first pieces whose halves exceed 16384 tokens:
    the feature-split fp8 step without the residual product."""
    inp = wl.make_inputs(32, 128, 8, (34000, 40000), kv_dtype="fp8", out_dtype="bf16", seed=64, device=DEV)
    assert binding.num_kv_splits(32, 8, 128, inp.max_len, 0, True) == 2
    out, lse, _ = binding.decode(inp)
    torch.cuda.synchronize()
    n_total = inp.B * inp.T * inp.H
    rows = sample_rows(n_total, 64, seed=64)
    _say("[gpu] two rounds, long fp8 units: oracle on %d rows" % rows.size)
    ref_o, ref_l = oracle_rows(inp.to("cpu"), rows=rows)
    compare(out, lse, ref_o, ref_l, "fp8", rows=rows, what="two rounds long fp8 units")


def test_host_bound_far_above_the_lengths():
    """max_seq_len four times the longest sequence: the pieces follow the
    actual lengths, not the bound."""
    inp = wl.make_inputs(8, 16, 2, (100, 2500), kv_dtype="bf16", out_dtype="f32", seed=57, poison=True)
    inp.max_len = 4 * inp.max_len
    check_full(inp, 0, "bound 4x the lengths")
    check_full(inp, 3, "bound 4x the lengths, three splits")


def test_batch_above_the_balanced_limit_uses_fixed_chunks():
    """More sequences than the device-side cut takes: fixed page chunks."""
    inp = wl.make_inputs(1040, 16, 1, (1, 400), kv_dtype="bf16", out_dtype="f32", seed=58)
    check_full(inp, 2, "B=1040 two splits")


@pytest.mark.parametrize("H,T,kv_dtype", [(1, 1, "bf16"), (1, 8, "bf16"), (1, 8, "fp8"), (16, 8, "bf16")])
def test_degenerate_head_counts_and_longest_draft(H, T, kv_dtype):
    inp = wl.make_inputs(3, H, T, [5, 200, 1500], kv_dtype=kv_dtype, out_dtype="f32", seed=54 + H + T, poison=True)
    check_full(inp, 0, "H=%d T=%d %s" % (H, T, kv_dtype))


# ------------------------------------------------------------------ sparse

@pytest.mark.parametrize("H,T,lens,K,splits", [
    (16, 1, [100, 3000], 256, 0),      # first sequence shorter than K: -1 padding
    (16, 1, [100, 3000], 256, 2),
    (128, 1, [5000, 70], 512, 0),
    (64, 2, [900, 2500], 192, 0),      # MTP with per-token index lists
    (32, 4, [700, 3000], 256, 0),
    (16, 8, [300, 5000, 90], 512, 0),
    (32, 1, [4100], 4096, 0),          # K above one workgroup's index table: forced splits
])
def test_sparse_shapes(H, T, lens, K, splits):
    inp = wl.make_inputs(len(lens), H, T, lens, kv_dtype="bf16", out_dtype="f32", topk=K, seed=13 + H, poison=True)
    check_full(inp, splits, "sparse H=%d K=%d" % (H, K))


@pytest.mark.parametrize("H,T,lens,K,splits", [
    (16, 1, [100, 3000], 256, 0),      # first sequence shorter than K: -1 padding
    (16, 1, [100, 3000], 256, 2),
    (128, 1, [5000, 70], 512, 0),
    (64, 2, [900, 2500], 192, 0),      # MTP with per-token index lists
    (32, 4, [700, 3000], 256, 0),
    (16, 8, [300, 5000, 90], 512, 0),
    (32, 1, [4100], 4096, 0),          # K above one workgroup's index table: forced splits
])
def test_sparse_fp8_shapes(H, T, lens, K, splits):
    inp = wl.make_inputs(len(lens), H, T, lens, kv_dtype="fp8", out_dtype="f32", topk=K, seed=23 + H, poison=True)
    check_full(inp, splits, "sparse fp8 H=%d K=%d" % (H, K))


@pytest.mark.parametrize("kv_dtype,H,T,lens,K,splits", [
    ("bf16", 256, 1, [3000, 700], 512, 0),       # two head blocks of 128 rows
    ("fp8", 160, 2, [2000, 600], 256, 0),        # MTP; the second head block holds 32 real rows
    ("bf16", 40, 3, [900, 2500], 192, 0),        # a head count that is not a multiple of 32
    ("fp8", 1024, 1, [1500, 300], 128, 2),       # eight head blocks, two splits
    ("bf16", 80, 4, [5000, 40, 1200], 320, 1),   # one split, a sequence shorter than K
])
def test_sparse_heads_over_several_row_blocks(kv_dtype, H, T, lens, K, splits):
    """Sparse calls whose heads span several row blocks, or whose last block
    is partly padding: every block of a draft token reads that token's index
    list, and padding rows are neither read nor written."""
    inp = wl.make_inputs(len(lens), H, T, lens, kv_dtype=kv_dtype, out_dtype="f32", topk=K, seed=61 + H + T,
                         poison=True)
    waves = binding.launch_waves(inp.B, inp.T, inp.H, inp.max_len, K, kv_dtype == "fp8")
    assert H > 32 * waves or H % 32 != 0
    check_full(inp, splits, "sparse heads H=%d T=%d %s" % (H, T, kv_dtype))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sparse_out_of_range_and_duplicate_indices(kv_dtype):
    inp = wl.make_inputs(2, 16, 1, [300, 300], kv_dtype=kv_dtype, out_dtype="f32", topk=128, seed=14)
    idx = inp.topk_indices.clone()
    idx[0, 0, :10] = 7                      # duplicates
    idx[0, 0, 10:20] = 300                  # == L: out of range
    idx[1, 0, :5] = -5
    idx[1, 0, 5:9] = 1 << 30
    inp.topk_indices = idx
    check_full(inp, 0, "sparse odd indices")



@pytest.mark.parametrize("kind", ["bf16", "fp8", "sparse_bf16", "sparse_fp8"])
@pytest.mark.parametrize("splits", [0, 3])
def test_invalid_page_ids_follow_the_stated_rule(kind, splits):
    """Block-table entries inside a sequence that name no page of the pool
    (past it, negative, far past it), checked against the rule the C header
    states for each kind.  Dense: their tokens read as zero vectors, so the
    call equals the oracle run with those entries pointing at an appended
    all-zero page.  Sparse: an index whose page is invalid is skipped, so the
    call equals the oracle run with those indices replaced by -1."""
    kv_dtype = "fp8" if kind.endswith("fp8") else "bf16"
    K = 200 if kind.startswith("sparse") else None
    inp = wl.make_inputs(2, 16, 2, [300, 700], kv_dtype=kv_dtype, out_dtype="f32", topk=K, seed=23)
    NB = inp.NB
    bad = inp.block_table.clone()
    bad[0, 2] = NB + 5
    bad[1, 1] = -3
    bad[1, 7] = 1 << 30
    inp.block_table = bad
    out, lse = run_case(inp, splits, "invalid page ids %s" % kind)
    invalid = (bad < 0) | (bad >= NB)
    if K is None:
        zero_page = torch.zeros_like(inp.kv_cache[:1])
        ref_in = wl.DecodeInputs(inp.q_nope, inp.q_pe, torch.cat([inp.kv_cache, zero_page]),
                                 torch.where(invalid, torch.full_like(bad, NB), bad), inp.seq_lens, None,
                                 kv_dtype, "f32", inp.softmax_scale, inp.q_scale, inp.kv_scale)
    else:
        idx = inp.topk_indices.clone()
        for b in range(inp.B):
            slot = idx[b].clamp(min=0) // 64
            in_seq = (idx[b] >= 0) & (idx[b] < int(inp.seq_lens[b]))
            hit = in_seq & invalid[b][slot.clamp(max=inp.MB - 1).long()]
            idx[b][hit] = -1
        assert (idx != inp.topk_indices).any()
        ref_in = wl.DecodeInputs(inp.q_nope, inp.q_pe, inp.kv_cache, bad.clamp(min=0, max=NB - 1), inp.seq_lens,
                                 idx, kv_dtype, "f32", inp.softmax_scale, inp.q_scale, inp.kv_scale)
    ref_o, ref_l = oracle_rows(ref_in)
    compare(out, lse, ref_o, ref_l, kv_dtype, what="invalid page ids %s" % kind)



@pytest.mark.parametrize("kind", ["bf16", "fp8", "sparse_bf16", "sparse_fp8"])
@pytest.mark.parametrize("splits", [0, 3])
def test_seq_lens_outside_the_table_are_clamped(kind, splits):
    """seq_lens -4 and 1000 with a five-page block table (and max_seq_len
    1000): the kernels clamp them to [0, 320], as the C header states, so the
    call equals the oracle on lengths 0 and 320 (sparse: indices between 320
    and 1000 are then outside the sequence and skipped)."""
    kv_dtype = "fp8" if kind.endswith("fp8") else "bf16"
    K = 128 if kind.startswith("sparse") else None
    inp = wl.make_inputs(2, 16, 2, [300, 320], kv_dtype=kv_dtype, out_dtype="f32", topk=K, seed=24)
    assert inp.MB == 5
    idx = None
    if K is not None:
        idx = inp.topk_indices.clone()
        idx[1, :, :16] = torch.arange(320, 1000, 45, dtype=idx.dtype)[:16]
    ref_in = wl.DecodeInputs(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table,
                             torch.tensor([0, 320], dtype=torch.int32), idx, kv_dtype, "f32", inp.softmax_scale,
                             inp.q_scale, inp.kv_scale)
    call_in = wl.DecodeInputs(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table,
                              torch.tensor([-4, 1000], dtype=torch.int32), idx, kv_dtype, "f32", inp.softmax_scale,
                              inp.q_scale, inp.kv_scale, max_len=1000)
    out, lse = run_case(call_in, splits, "seq_lens clamped %s" % kind)
    ref_o, ref_l = oracle_rows(ref_in)
    compare(out, lse, ref_o, ref_l, kv_dtype, what="seq_lens clamped %s" % kind)
    assert torch.isneginf(lse[0]).all().item() and torch.count_nonzero(out[0]).item() == 0



@pytest.mark.parametrize("kind", ["bf16", "fp8", "sparse_bf16", "sparse_fp8"])
def test_lse_over_two_nearly_equal_keys(kind):
    """One query over two keys whose second weight lies just under 1 (swept
    over 64 heads across several rounding steps of the weights' format):
    lse = ln(1 + w2) exactly.  The weights enter the value product rounded
    to bf16 or e4m3; a sum of the rounded weights would be off by up to half
    a step of w2 over 1 + w2 (about 1e-3 for bf16, 3e-2 for e4m3), so the
    LSE must follow the unrounded weights."""
    H = 64
    fp8 = kind.endswith("fp8")
    K = 2 if kind.startswith("sparse") else None
    base = wl.make_inputs(1, H, 1, [2], kv_dtype="bf16", out_dtype="f32", topk=K, seed=27)
    page = int(base.block_table[0, 0])
    a = 1.0 + torch.arange(H, dtype=torch.float32) / H
    x = -0.02734375                                   # exact in bf16 and e4m3
    q_nope = torch.zeros((1, 1, H, 512), dtype=torch.float32)
    q_pe = torch.zeros((1, 1, H, 64), dtype=torch.float32)
    q_pe[0, 0, :, 0] = a
    kv = torch.zeros_like(base.kv_cache, dtype=torch.float32)
    kv[page, 1, 512] = x
    if fp8:
        enc = lambda t: t.to(torch.float8_e4m3fn).view(torch.uint8)   # noqa: E731
        q_nope, q_pe, kv = enc(q_nope), enc(q_pe), enc(kv)
        a = q_pe[0, 0, :, 0].view(torch.float8_e4m3fn).float()        # the query as stored
    else:
        q_nope, q_pe, kv = q_nope.to(torch.bfloat16), q_pe.to(torch.bfloat16), kv.to(torch.bfloat16)
        a = q_pe[0, 0, :, 0].float()
    idx = None if K is None else torch.tensor([[[0, 1]]], dtype=torch.int32)
    inp = wl.DecodeInputs(q_nope, q_pe, kv, base.block_table, base.seq_lens, idx, "fp8" if fp8 else "bf16", "f32",
                          base.softmax_scale, 1.0, 1.0)
    out, lse = run_case(inp, 0, "two near-equal keys %s" % kind)
    w2 = torch.exp(base.softmax_scale * a.double() * x)
    assert float(w2.min()) > 0.99 and float(w2.max()) < 1.0
    err = float((lse[0, 0].double().cpu() - torch.log1p(w2)).abs().max())
    _say("[gpu] two near-equal keys %s: w2 in [%.5f, %.5f], max |lse - ln(1 + w2)| %.3g"
         % (kind, float(w2.min()), float(w2.max()), err))
    assert err < 1e-5, "LSE follows rounded weights: %.3g" % err
    assert torch.count_nonzero(out).item() == 0



@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_lse_over_two_nearly_equal_keys_after_a_jump(kv_dtype):
    """Two 20000-token units, one split (the four-wave kernels; fp8: the
    feature-split kernel, over 16384 tokens) whose keys all score -32 to -64
    except two near-equal ones in the middle: for the heads with the larger
    scores the row maximum jumps by more than the 64 (log2) the first tile's
    reference allows, so the second pass runs, for the others it does not;
    either way the LSE must equal ln(1 + w2) to 1e-5."""
    B, T, H, L = 2, 1, 128, 20000
    fp8 = kv_dtype == "fp8"
    assert binding.launch_waves(B, T, H, L, 0, fp8) == 4
    base = wl.make_inputs(B, H, T, [L, L], kv_dtype="bf16", out_dtype="f32", seed=28)
    a = 1.0 + torch.arange(H, dtype=torch.float32) % 64 / 64
    x = -0.02734375
    q_nope = torch.zeros((B, T, H, 512), dtype=torch.float32)
    q_pe = torch.zeros((B, T, H, 64), dtype=torch.float32)
    q_pe[:, 0, :, 0] = a
    kv = torch.zeros_like(base.kv_cache, dtype=torch.float32)
    tok = torch.arange(L)
    for b, j in ((0, 10000), (1, 17)):
        pages = base.block_table[b].long()
        kv[pages[tok // 64], tok % 64, 512] = -448.0                  # weights below 1e-14
        kv[pages[j // 64], j % 64, 512] = 0.0
        kv[pages[(j + 1) // 64], (j + 1) % 64, 512] = x
    if fp8:
        enc = lambda t: t.to(torch.float8_e4m3fn).view(torch.uint8)   # noqa: E731
        q_nope, q_pe, kv = enc(q_nope), enc(q_pe), enc(kv)
        a = q_pe[0, 0, :, 0].view(torch.float8_e4m3fn).float()
    else:
        q_nope, q_pe, kv = q_nope.to(torch.bfloat16), q_pe.to(torch.bfloat16), kv.to(torch.bfloat16)
        a = q_pe[0, 0, :, 0].float()
    inp = wl.DecodeInputs(q_nope, q_pe, kv, base.block_table, base.seq_lens, None, kv_dtype, "f32",
                          base.softmax_scale, 1.0, 1.0)
    out, lse = run_case(inp, 1, "two near-equal keys after a jump %s" % kv_dtype)
    w2 = torch.exp(base.softmax_scale * a.double() * x)
    err = float((lse[:, 0].double().cpu() - torch.log1p(w2)[None, :]).abs().max())
    _say("[gpu] two near-equal keys after a jump %s: max |lse - ln(1 + w2)| %.3g" % (kv_dtype, err))
    assert err < 1e-5, "LSE off: %.3g" % err
    assert torch.count_nonzero(out).item() == 0

def test_sparse_index_probe_histogram_exact():
    """q = 0 and latent c_j = e_(j mod 512): n * out is the exact histogram."""
    L, K = 2000, 1024
    inp = wl.make_inputs(1, 16, 1, [L], kv_dtype="bf16", out_dtype="f32", topk=K, seed=15)
    inp.q_nope.zero_()
    inp.q_pe.zero_()
    kv = torch.zeros_like(inp.kv_cache, dtype=torch.float32)
    for j in range(L):
        kv[int(inp.block_table[0, j // 64]), j % 64, j % 512] = 1.0
    inp.kv_cache = kv.to(torch.bfloat16)
    idx = inp.topk_indices
    idx[0, 0, :50] = 3                      # duplicates count
    idx[0, 0, 50:60] = -1
    out, lse = run_case(inp, 0, "index probe")
    sel = idx[0, 0][(idx[0, 0] >= 0) & (idx[0, 0] < L)]
    n = sel.numel()
    hist = torch.bincount(sel.long() % 512, minlength=512)
    got = torch.round(out[0, 0].cpu().double() * n).long()
    for h in range(16):
        assert torch.equal(got[h], hist), "histogram mismatch in head %d" % h
    assert torch.allclose(lse.cpu().double(), torch.full_like(lse.cpu().double(), math.log(n)), atol=1e-6)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sparse_all_positions_equals_dense(kv_dtype):
    L, K = 300, 512
    inp = wl.make_inputs(1, 32, 1, [L], kv_dtype=kv_dtype, out_dtype="f32", topk=K, seed=16)
    o_s, l_s = run_case(inp, 0, "sparse all positions")
    dense = dataclasses.replace(inp, topk_indices=None)
    o_d, l_d = run_case(dense, 0, "dense twin")
    # Same tokens in another order: equal up to the rounding of P (bf16, or
    # e4m3 plus its residual).
    assert torch.max(torch.abs(o_s - o_d)).item() < (1e-2 if kv_dtype == "bf16" else 3e-2)
    assert torch.max(torch.abs(l_s - l_d)).item() < 1e-5


# ------------------------------------------------------------------ four-wave (pipelined) variants

# Shapes whose launch plan puts four waves (128 query rows) in a workgroup:
# the software-pipelined tile loop.  Few work units make the planner narrow
# the row block instead, so these batches are wide.
FOUR_WAVE = [
    ("bf16", 256, 128, 1, (32, 330), 0),
    ("bf16", 256, 32, 4, (3, 700), 0),
    ("bf16", 32, 128, 8, (60, 900), 0),
    ("fp8", 256, 32, 4, (3, 700), 0),
    ("fp8", 256, 128, 1, (32, 330), 0),
    ("fp8", 32, 32, 4, (3, 700), 0),
    ("sparse", 256, 128, 1, (100, 900), 96),
    ("sparse", 16, 128, 1, (100, 900), 96),
    ("sparse_fp8", 256, 128, 1, (100, 900), 96),
    ("sparse_fp8", 16, 128, 1, (100, 900), 96),
    ("sparse_fp8", 16, 128, 2, (100, 900), 160),
]


@pytest.mark.parametrize("kind,B,H,T,lens,K", FOUR_WAVE)
def test_four_wave_variants(kind, B, H, T, lens, K):
    kv_dtype = "fp8" if kind in ("fp8", "sparse_fp8") else "bf16"
    inp = wl.make_inputs(B, H, T, lens, kv_dtype=kv_dtype, out_dtype="f32", topk=K or None, seed=31 + B + H + T,
                         poison=True)
    assert binding.launch_waves(B, T, H, inp.max_len, K, kv_dtype == "fp8") == 4
    out, lse = run_case(inp, 0, "four-wave %s" % kind)
    # every row of the smaller batches, a sample of the larger ones
    rows = None if B * T * H <= 4096 else sample_rows(B * T * H, 1024, seed=B + H)
    ref_o, ref_l = oracle_rows(inp, rows=rows)
    compare(out, lse, ref_o, ref_l, kv_dtype, rows=rows, what="four-wave %s" % kind)


# ------------------------------------------------------------------ second pass (large logit jump)

def _plant_large_logit(inp, pos):
    """Cache position `pos` of every sequence becomes a key aligned with the
    query of that sequence's row (t=0, h=0), so that row's logit there lies
    far above its first tile's (more than 2^64 in the log2 domain): the
    kernel must rerun the unit against the exact row maximum."""
    for b in range(inp.B):
        pg = int(inp.block_table[b, pos // 64])
        if inp.kv_dtype == "bf16":
            q = torch.cat([inp.q_nope[b, 0, 0], inp.q_pe[b, 0, 0]]).float()
            inp.kv_cache[pg, pos % 64] = (3.0 * q).to(torch.bfloat16)
        else:
            q = torch.cat([inp.q_nope[b, 0, 0], inp.q_pe[b, 0, 0]]).view(torch.float8_e4m3fn).float()
            inp.kv_cache[pg, pos % 64] = torch.where(q >= 0, 448.0, -448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return inp


@pytest.mark.parametrize("kind,B,H,T,waves", [
    ("bf16", 256, 32, 4, 4), ("bf16", 256, 128, 1, 4), ("bf16", 4, 64, 1, 1), ("bf16", 512, 64, 1, 2),
    ("bf16", 4, 16, 1, 2), ("fp8", 256, 32, 4, 4), ("fp8", 4, 64, 1, 1), ("fp8", 4, 16, 1, 2),
    ("sparse", 256, 128, 1, 4), ("sparse", 4, 16, 1, 1),
    ("sparse_fp8", 256, 128, 1, 4), ("sparse_fp8", 4, 16, 1, 1),
])
def test_large_logit_jump_reruns_against_exact_maximum(kind, B, H, T, waves):
    L, pos = 300, 150
    kv_dtype = "fp8" if kind in ("fp8", "sparse_fp8") else "bf16"
    K = 96 if kind.startswith("sparse") else 0
    inp = wl.make_inputs(B, H, T, [L] * B, kv_dtype=kv_dtype, out_dtype="f32", topk=K or None, seed=41 + B + H)
    if K:
        inp.topk_indices[:, :, K // 2] = pos    # the planted position sits in the second index tile
    _plant_large_logit(inp, pos)
    assert binding.launch_waves(B, T, H, L, K, kv_dtype == "fp8") == waves
    out, lse = run_case(inp, 0, "logit jump %s" % kind)
    rows = np.unique(np.concatenate([sample_rows(B * T * H, 96, seed=B), np.arange(0, B * T * H, T * H)[:16]]))
    ref_o, ref_l = oracle_rows(inp, rows=rows)
    assert np.max(ref_l) > 80.0                 # the planted logit dominates row (b, 0, 0)
    compare(out, lse, ref_o, ref_l, kv_dtype, rows=rows, what="logit jump %s" % kind)


# ------------------------------------------------------------------ graph capture

@pytest.mark.parametrize("lens,splits", [([100, 800, 2000, 64], 3), ([40000, 300, 20000, 1], 2)])
def test_hip_graph_replay_matches_eager(lens, splits):
    """fp8 calls captured in one graph with their merge: short units (the
    residual-product kernel), and units over 16384 tokens next to short ones
    (the feature-split kernel, whose short units rerun with the residual
    product)."""
    B, T, H = 4, 4, 32
    long_units = fixed_unit_tokens(max(lens), splits) > 16384
    if long_units:
        assert binding.launch_waves(B, T, H, max(lens), 0, True) == 4
    inp = wl.make_inputs(B, H, T, lens, kv_dtype="fp8", out_dtype="bf16", seed=17).to(DEV)
    _say("[gpu] graph capture, lengths %s, %d splits, long units %s" % (lens, splits, long_units))
    assert long_units == (max(lens) > 20000)
    eager_o, eager_l, ws = binding.decode(inp, num_kv_splits=splits)
    torch.cuda.synchronize()
    out = torch.empty_like(eager_o)
    lse = torch.empty_like(eager_l)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        binding.decode(inp, num_kv_splits=splits, out=out, lse=lse, workspace=ws)   # warm the stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            binding.decode(inp, num_kv_splits=splits, out=out, lse=lse, workspace=ws, stream=s)
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l), "replay %d differs" % rep
        binding.decode(inp, num_kv_splits=1)   # unrelated eager work between replays
        torch.cuda.synchronize()
    ref_o, ref_l = oracle_rows(inp.to("cpu"))
    compare(eager_o, eager_l, ref_o, ref_l, "fp8", what="graph replay %s" % lens)



@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_hip_graph_replay_sparse_matches_eager(kv_dtype):
    """Sparse calls (per-draft-token index lists, several splits, the merge)
    captured in one graph: four replays with NaN-filled outputs and other
    eager calls between them equal the eager call bit for bit."""
    B, T, H, K = 3, 2, 40, 300
    inp = wl.make_inputs(B, H, T, [5000, 90, 1], kv_dtype=kv_dtype, out_dtype="bf16", topk=K, seed=18).to(DEV)
    splits = 3
    _say("[gpu] sparse graph capture %s: K=%d, %d splits" % (kv_dtype, K, splits))
    eager_o, eager_l, ws = binding.decode(inp, num_kv_splits=splits)
    torch.cuda.synchronize()
    out, lse = torch.empty_like(eager_o), torch.empty_like(eager_l)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        binding.decode(inp, num_kv_splits=splits, out=out, lse=lse, workspace=ws)   # warm the stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            binding.decode(inp, num_kv_splits=splits, out=out, lse=lse, workspace=ws, stream=s)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l), "replay %d differs" % rep
        binding.decode(inp, num_kv_splits=1)   # unrelated eager work between replays
        torch.cuda.synchronize()
    ref_o, ref_l = oracle_rows(inp.to("cpu"))
    compare(eager_o, eager_l, ref_o, ref_l, kv_dtype, what="sparse graph replay %s" % kv_dtype)



def test_hip_graph_replay_two_rounds_bf16():
    """A dense bf16 call planned as two rounds of longest-first pieces (the
    device cuts and ranks the pieces from seq_lens inside the graph): four
    replays equal to the eager call bit for bit; then the lengths are cut
    down in place on the device (the captured max_seq_len bound still
    holds) and a replay equals a fresh eager call on the new lengths."""
    B, T, H = 32, 8, 128
    g_len = np.random.default_rng(19)
    lens = [int(x) for x in g_len.integers(100, 1501, size=B)]
    assert binding.num_kv_splits(B, T, H, max(lens), 0, False) == 2
    inp = wl.make_inputs(B, H, T, lens, kv_dtype="bf16", out_dtype="bf16", seed=19).to(DEV)
    _say("[gpu] graph capture, two rounds longest first, B=%d H=%d T=%d" % (B, H, T))
    eager_o, eager_l, ws = binding.decode(inp)
    torch.cuda.synchronize()
    out, lse = torch.empty_like(eager_o), torch.empty_like(eager_l)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        binding.decode(inp, out=out, lse=lse, workspace=ws)   # warm the stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            binding.decode(inp, out=out, lse=lse, workspace=ws, stream=s)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l), "replay %d differs" % rep
        binding.decode(inp, num_kv_splits=1)   # unrelated eager work between replays
        torch.cuda.synchronize()
    n = B * T * H
    rows = np.unique(np.concatenate([np.arange(0, T * H), sample_rows(n, 256, seed=19)]))
    ref_o, ref_l = oracle_rows(inp.to("cpu"), rows=rows)
    compare(eager_o, eager_l, ref_o, ref_l, "bf16", rows=rows, what="graph replay two rounds bf16")
    # New, shorter lengths written into the captured seq_lens buffer.
    new_lens = [max(1, L - int(g_len.integers(0, L // 2 + 1))) for L in lens]
    inp.seq_lens.copy_(torch.tensor(new_lens, dtype=inp.seq_lens.dtype))
    torch.cuda.synchronize()
    _say("[gpu] graph replay after the lengths changed on the device")
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    fresh_o, fresh_l, _ = binding.decode(inp)
    torch.cuda.synchronize()
    assert torch.equal(out, fresh_o) and torch.equal(lse, fresh_l), "replay on new lengths differs"
    ref_o, ref_l = oracle_rows(inp.to("cpu"), rows=rows)
    compare(fresh_o, fresh_l, ref_o, ref_l, "bf16", rows=rows, what="graph replay on new lengths")


# ------------------------------------------------------------------ full-size workloads (sampled rows)

FULL = ["r1_b128_h16_kv1k-8k_bf16", "mtp3_b64_h32_kv80k_fp8", "mtp7_b32_h128_kv16k-32k_bf16",
        "sparse_b64_h128_kv64k_top2048_bf16", "sparse_b64_h128_kv64k_top2048_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_sampled_rows(name):
    _say("[gpu] full-size %s: drawing inputs" % name)
    inp = wl.workload(name, device=DEV)
    out, lse, _ = binding.decode(inp)          # default (library-chosen) launch configuration
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all().item()
    assert torch.isfinite(lse).all().item()
    n_total = inp.B * inp.T * inp.H
    R = inp.T * inp.H
    # all rows of the first and last sequences, and 512 random others
    rows = np.unique(np.concatenate([np.arange(0, R), np.arange(n_total - R, n_total),
                                     sample_rows(n_total, 512, seed=sum(name.encode()))]))
    cpu = inp.to("cpu")
    _say("[gpu] full-size %s: oracle on %d rows" % (name, rows.size))
    ref_o, ref_l = oracle_rows(cpu, rows=rows)
    e = compare(out, lse, ref_o, ref_l, inp.kv_dtype, rows=rows, what=name)
    _say("[gpu] full-size %s: max |out - oracle| %.4g, lse rel %.3g over %d rows" % ((name,) + e + (rows.size,)))


# ------------------------------------------------------------------ two-stage form

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_stage_one_then_merge_equals_one_call(kv_dtype):
    inp = wl.make_inputs(3, 32, 2, [100, 700, 1500], kv_dtype=kv_dtype, out_dtype="f32", seed=21).to(DEV)
    _say("[gpu] two-stage %s" % kv_dtype)
    ref_o, ref_l, ws = binding.decode(inp, num_kv_splits=3)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    ws.fill_(float("nan"))
    if kv_dtype == "fp8":
        binding.mla_decode_fp8(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, inp.max_seq_len,
                               inp.softmax_scale, inp.q_scale, inp.kv_scale, None, None, ws, 3)
    else:
        binding.mla_decode(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, inp.max_seq_len,
                           inp.softmax_scale, None, None, ws, 3)
    binding.mla_merge_partials(ws, inp.B * inp.T * inp.H, 3, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)



@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_partials_of_page_slices_merge_to_the_whole_sequence(kv_dtype):
    """Stage two fed with partials from separate calls, as a sequence sharded
    over W holders would produce them: each sequence's pages are cut into
    W = 3 contiguous slices and stage one runs per slice.  Draft tokens are
    flattened into the batch (q_len 1 per entry), so that each entry's length
    is the prefix of the slice its query sees: the whole slice before the
    causal limit, part of it at the limit, none after.  The slices' outputs
    and LSEs, packed as [rows, W, 513] partials, are merged by
    mla_merge_partials and compared with the oracle on the whole sequences
    (empty slices and queries that see none of a slice included)."""
    B, T, H, W = 3, 3, 16, 3
    lens = [1000, 130, 2600]
    full = wl.make_inputs(B, H, T, lens, kv_dtype=kv_dtype, out_dtype="f32", seed=22, poison=True)
    n_pages = [(L + 63) // 64 for L in lens]
    cuts = [[round(w * n / W) for w in range(W + 1)] for n in n_pages]
    width = max(c[w + 1] - c[w] for c in cuts for w in range(W))
    dev_kv = full.kv_cache.to(DEV)
    rows = B * T * H
    ws = torch.empty((rows, W, 513), device=DEV, dtype=torch.float32)
    for w in range(W):
        bt = torch.full((B * T, max(1, width)), -1, dtype=torch.int32)
        sl = torch.zeros(B * T, dtype=torch.int32)
        for b in range(B):
            p0, p1 = cuts[b][w], cuts[b][w + 1]
            slice_tokens = max(0, min(lens[b], p1 * 64) - p0 * 64)
            for t in range(T):
                bt[b * T + t, :p1 - p0] = full.block_table[b, p0:p1]
                n_vis = lens[b] - T + t + 1                       # tokens query t sees in the whole sequence
                sl[b * T + t] = min(max(n_vis - p0 * 64, 0), slice_tokens)
        g = wl.DecodeInputs(full.q_nope.reshape(B * T, 1, H, -1).to(DEV), full.q_pe.reshape(B * T, 1, H, -1).to(DEV),
                            dev_kv, bt.to(DEV), sl.to(DEV), None, kv_dtype, "f32", full.softmax_scale,
                            full.q_scale, full.kv_scale, max_len=width * 64)
        _say("[gpu] slice %d of %d (%s): lengths %s" % (w, W, kv_dtype, sl.tolist()))
        o, l, _ = binding.decode(g, num_kv_splits=1)
        torch.cuda.synchronize()
        ws[:, w, :512] = o.reshape(rows, 512)
        ws[:, w, 512] = l.reshape(rows)
    out = torch.empty((B, T, H, 512), device=DEV, dtype=torch.float32)
    lse = torch.empty((B, T, H), device=DEV, dtype=torch.float32)
    binding.mla_merge_partials(ws, rows, W, out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_rows(full)
    e = compare(out, lse, ref_o, ref_l, kv_dtype, what="merged page slices %s" % kv_dtype)
    _say("[gpu] merged page slices %s: max |out - oracle| %.4g, lse rel %.3g" % ((kv_dtype,) + e))



@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sparse_stage_one_then_merge_equals_one_call(kv_dtype):
    """The two-stage form through the sparse entry points (per-draft-token
    lists): stage one alone (out = lse = NULL) into a workspace of NaN, then
    mla_merge_partials, equal to the one-call form bit for bit."""
    inp = wl.make_inputs(3, 40, 2, [100, 700, 1500], kv_dtype=kv_dtype, out_dtype="f32", topk=300,
                         seed=26).to(DEV)
    _say("[gpu] two-stage sparse %s" % kv_dtype)
    ref_o, ref_l, ws = binding.decode(inp, num_kv_splits=3)
    out, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    ws.fill_(float("nan"))
    if kv_dtype == "fp8":
        binding.mla_sparse_decode_fp8(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens,
                                      inp.topk_indices, inp.max_seq_len, inp.softmax_scale, inp.q_scale,
                                      inp.kv_scale, None, None, ws, 3)
    else:
        binding.mla_sparse_decode(inp.q_nope, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens,
                                  inp.topk_indices, inp.max_seq_len, inp.softmax_scale, None, None, ws, 3)
    binding.mla_merge_partials(ws, inp.B * inp.T * inp.H, 3, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


# ------------------------------------------------------------------ the largest shapes the calls accept

@pytest.mark.parametrize("kind", ["bf16", "fp8", "sparse", "sparse_fp8"])
def test_maximum_heads_and_draft_length(kind):
    """H = 1024 heads with q_len = 8: 8192 rows per sequence (64 four-wave row
    blocks, or 8 head blocks per draft token for sparse lists), next to a short
    sequence; the first and last sequence's edge rows and a random sample."""
    kv_dtype = "fp8" if kind.endswith("fp8") else "bf16"
    K = 256 if kind.startswith("sparse") else None
    inp = wl.make_inputs(2, 1024, 8, [700, 40], kv_dtype=kv_dtype, out_dtype="bf16", topk=K, seed=91, poison=True)
    out, lse = run_case(inp, 0, "max heads %s" % kind)
    n = inp.B * inp.T * inp.H
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(n - 64, n), sample_rows(n, 384, seed=91)]))
    ref_o, ref_l = oracle_rows(inp, rows=rows)
    e = compare(out, lse, ref_o, ref_l, kv_dtype, rows=rows, what="max heads %s" % kind)
    _say("[gpu] max heads %s: max |out - oracle| %.4g, lse rel %.3g" % ((kind,) + e))


@pytest.mark.parametrize("kind,T", [("bf16", 1), ("fp8", 4), ("sparse", 2), ("sparse_fp8", 1)])
def test_every_sequence_empty(kind, T):
    """A batch in which no sequence holds a token (max_seq_len 0): every row
    comes out as zeros with lse -inf, in every kind."""
    kv_dtype = "fp8" if kind.endswith("fp8") else "bf16"
    K = 64 if kind.startswith("sparse") else None
    inp = wl.make_inputs(3, 16, T, [0, 0, 0], kv_dtype=kv_dtype, out_dtype="f32", topk=K, seed=93, extra_pages=1)
    out, lse = run_case(inp, 0, "all empty %s" % kind)
    assert torch.count_nonzero(out).item() == 0
    assert torch.isneginf(lse).all().item()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sparse_list_longer_than_many_splits(kv_dtype):
    """A top-k list of 20000 indices over 30000 tokens: at least 20 splits of
    the 1024-entry index table, every row against the oracle."""
    inp = wl.make_inputs(1, 16, 1, [30000], kv_dtype=kv_dtype, out_dtype="f32", topk=20000, seed=94, poison=True)
    assert binding.num_kv_splits(1, 1, 16, inp.max_len, 20000, kv_dtype == "fp8") >= 20
    check_full(inp, 0, "sparse K=20000 %s" % kv_dtype)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_zero_query_is_the_mean_of_the_visible_latents(kv_dtype):
    """q = 0 makes every weight equal: out is the mean of the latents a row
    sees and lse = ln(tokens seen), over long units (a dropped or repeated
    tile shows at once).  Checked against that closed form in fp64."""
    lens = [50000, 7777, 1]
    inp = wl.make_inputs(3, 16, 4, lens, kv_dtype=kv_dtype, out_dtype="f32", seed=95)
    inp.q_nope.zero_()
    inp.q_pe.zero_()
    out, lse = run_case(inp, 0, "zero query %s" % kv_dtype)
    kv = inp.kv_cache
    if kv_dtype == "fp8":
        lat = kv.view(torch.float8_e4m3fn).to(torch.float64)[..., :512] * inp.kv_scale
    else:
        lat = kv.to(torch.float64)[..., :512]
    o = out.double().cpu()
    for b, L in enumerate(lens):
        pages = [int(p) for p in inp.block_table[b, :(L + 63) // 64]]
        toks = torch.cat([lat[p] for p in pages], dim=0)[:L]
        csum = torch.cumsum(toks, dim=0)
        for t in range(4):
            n = L - 4 + t + 1
            if n <= 0:
                assert torch.count_nonzero(o[b, t]).item() == 0 and torch.isneginf(lse[b, t]).all().item()
                continue
            mean = csum[n - 1] / n
            err = float((o[b, t] - mean).abs().max())
            assert err < 1e-4, "b=%d t=%d n=%d: max |out - mean| = %.3g" % (b, t, n, err)
            lerr = float((lse[b, t].double().cpu() - math.log(n)).abs().max())
            assert lerr < 1e-5 * max(1.0, math.log(n)), "b=%d t=%d: lse %.3g off" % (b, t, lerr)
