"""GPU parity of the dense un-absorbed MHA route (mla_dense_mha) against the
fp64 un-absorbed oracle (oracle/mha_bruteforce.mha_paged) on the same bytes,
the oracle rounding the up-projected keys and values to bf16 as the route
materialises them.

Cases: decode-sized and prefill-sized query counts (causal, queries that see
nothing, T = L), ragged tails across key tiles, NaN-poisoned cache slots no
sequence owns, shuffled pages, empty sequences, a workspace of NaN before
the call, and the absorbed route on the same inputs (latent output projected
by W_UV) agreeing within the bf16 tolerance.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.mha_bruteforce as mb
from mla_paged_latent_03_amd import binding, workloads as wl
from parity import TOL_LSE_REL, half_ulp_bf16, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_mha(inp, q_nope, w_uk, w_uv, out_dtype="f32", workspace=None):
    g = inp.to(DEV)
    out = torch.empty((inp.B, inp.T, inp.H, 128), device=DEV,
                      dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)
    lse = torch.empty((inp.B, inp.T, inp.H), device=DEV, dtype=torch.float32)
    binding.mla_dense_mha(q_nope.to(DEV), g.q_pe, g.kv_cache, g.block_table,
                          g.seq_lens, w_uk.to(DEV), w_uv.to(DEV), g.max_seq_len, g.softmax_scale, out, lse,
                          workspace)
    torch.cuda.synchronize()
    return out, lse


def oracle_mha(inp, q_nope, w_uk, w_uv, rows=None):
    f = lambda t: mb.bf16_bits_to_f64(wl.as_numpy_bits(t))   # noqa: E731
    return mb.mha_paged(f(q_nope), f(inp.q_pe), f(inp.kv_cache), inp.block_table.cpu().numpy(),
                        inp.seq_lens.cpu().numpy(), f(w_uk), f(w_uv), inp.softmax_scale, rows=rows,
                        expanded="bf16")


def check(inp, q_nope, w_uk, w_uv, what, rows=None, out_dtype="f32"):
    _say("[gpu] mha: %s B=%d T=%d H=%d" % (what, inp.B, inp.T, inp.H))
    out, lse = run_mha(inp, q_nope, w_uk, w_uv, out_dtype)
    ref_o, ref_l = oracle_mha(inp, q_nope, w_uk, w_uv, rows)
    o = out.double().cpu().reshape(-1, 128).numpy()
    l = lse.double().cpu().reshape(-1).numpy()
    if rows is not None:
        o, l = o[rows], l[rows]
    assert np.all(np.isfinite(o)), what
    err_all = np.abs(o - ref_o)
    err = float(err_all.max()) if o.size else 0.0
    # bf16 outputs: plus the format's own rounding (half an ulp of the value)
    allowed = TOL + (half_ulp_bf16(np.maximum(np.abs(ref_o), np.abs(o))) if out_dtype == "bf16" else 0.0)
    assert np.all(err_all <= allowed), "%s: max |out - oracle| = %.3g" % (what, err)
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l)), what
    fin = ~np.isneginf(ref_l)
    lerr = float((np.abs(l[fin] - ref_l[fin]) / np.maximum(1.0, np.abs(ref_l[fin]))).max()) if fin.any() else 0.0
    assert lerr <= TOL_LSE_REL, "%s: lse rel err %.3g" % (what, lerr)
    _say("[gpu] mha %s: max |out - oracle| %.4g, lse rel %.3g" % (what, err, lerr))
    return out, lse


@pytest.mark.parametrize("H,T,lens", [
    (4, 1, [1, 50, 200]),            # decode
    (4, 4, [3, 4, 5, 130]),          # MTP: first queries of short sequences see nothing
    (8, 37, [37, 100, 300]),         # a query block of 37 (two blocks, ragged)
    (2, 96, [96, 64]),               # a prefill (T = L) and a shorter sequence
    (16, 8, [0, 700, 1]),            # empty and one-token sequences
])
def test_dense_mha_shapes(H, T, lens):
    inp = wl.make_inputs(len(lens), H, T, lens, kv_dtype="bf16", out_dtype="f32", seed=201 + H + T, poison=True,
                         extra_pages=2)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=301 + T)
    check(inp, q, w_uk, w_uv, "H=%d T=%d lens=%s" % (H, T, lens))


def test_dense_mha_bf16_out_and_stale_workspace():
    inp = wl.make_inputs(2, 8, 16, [40, 333], kv_dtype="bf16", out_dtype="bf16", seed=211, poison=True)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=311)
    need = binding.dense_mha_workspace_size(inp.B, inp.H, inp.max_seq_len)
    ws = torch.full(((need + 1) // 2,), float("nan"), device=DEV, dtype=torch.bfloat16)
    _say("[gpu] mha: workspace of NaN")
    out, lse = run_mha(inp, q, w_uk, w_uv, "bf16", ws)
    ref_o, ref_l = oracle_mha(inp, q, w_uk, w_uv)
    o = out.double().cpu().reshape(-1, 128).numpy()
    allowed = TOL + half_ulp_bf16(np.maximum(np.abs(ref_o), np.abs(o)))
    assert np.all(np.abs(o - ref_o) <= allowed) and torch.isfinite(out.float()).all()


def test_dense_mha_long_prefill_sampled_rows():
    """A 1536-token prefill next to a 700-token one, 16 heads: sampled rows."""
    inp = wl.make_inputs(2, 16, 1536, [1536, 700], kv_dtype="bf16", out_dtype="bf16", seed=212)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=312)
    n = inp.B * inp.T * inp.H
    rows = np.unique(np.concatenate([sample_rows(n, 160, seed=212), np.arange(0, 16), np.arange(n - 16, n)]))
    check(inp, q, w_uk, w_uv, "long prefill", rows=rows, out_dtype="bf16")


def test_dense_mha_page_permutation_bit_identical():
    inp = wl.make_inputs(2, 4, 8, [200, 90], kv_dtype="bf16", out_dtype="f32", seed=213)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=313)
    o1, l1 = run_mha(inp, q, w_uk, w_uv)
    perm = torch.randperm(inp.NB, generator=torch.Generator().manual_seed(2))
    inv = torch.argsort(perm)
    inp2 = wl.DecodeInputs(inp.q_nope, inp.q_pe, inp.kv_cache[perm].contiguous(),
                           torch.where(inp.block_table >= 0, inv[inp.block_table.clamp(min=0)].to(torch.int32),
                                       inp.block_table), inp.seq_lens, None, "bf16", "f32", inp.softmax_scale)
    o2, l2 = run_mha(inp2, q, w_uk, w_uv)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dense_mha_matches_the_absorbed_route():
    """Sparse MLA with every position listed (L <= top-k) through the absorbed
    MQA call, its latent output projected by W_UV, against the dense MHA call
    on the same cache and queries (absorption and projection in fp32)."""
    L, K, H = 300, 512, 16
    inp = wl.make_inputs(2, H, 1, [L, 120], kv_dtype="bf16", out_dtype="f32", topk=K, seed=214)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=314)
    q_abs = torch.einsum("bthd,hdk->bthk", q.float(), w_uk.float()).to(torch.bfloat16)
    absorbed = wl.DecodeInputs(q_abs.contiguous(), inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens,
                               inp.topk_indices, "bf16", "f32", inp.softmax_scale)
    g = absorbed.to(DEV)
    _say("[gpu] mha vs absorbed sparse call")
    lat, lat_lse, _ = binding.decode(g)
    torch.cuda.synchronize()
    proj = torch.einsum("bthk,hdk->bthd", lat.double().cpu(), w_uv.double())
    out, lse = run_mha(inp, q, w_uk, w_uv)
    assert torch.max(torch.abs(out.double().cpu() - proj)).item() < 2 * TOL
    assert torch.max(torch.abs(lse.cpu() - lat_lse.cpu())).item() < 0.05


def test_dense_mha_argument_errors():
    inp = wl.make_inputs(1, 4, 2, [10], kv_dtype="bf16", out_dtype="f32", seed=215).to(DEV)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=315)
    out = torch.empty((1, 2, 4, 128), device=DEV)
    small = torch.empty(8, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(binding.MLAError) as ei:
        binding.mla_dense_mha(q, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, w_uk, w_uv, 10,
                              inp.softmax_scale, out, None, small)
    assert ei.value.status == binding.MLA_ERR_WORKSPACE_TOO_SMALL


def test_dense_mha_bench_size_sampled_rows():
    """The benchmark's shape (4 sequences of 2048 tokens, q_len = 2048, 128
    heads): the first and last rows of each sequence and 48 random ones."""
    inp = wl.make_inputs(4, 128, 2048, [2048] * 4, kv_dtype="bf16", out_dtype="bf16", seed=216)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=316)
    n = inp.B * inp.T * inp.H
    per_seq = inp.T * inp.H
    edges = np.concatenate([np.arange(b * per_seq, b * per_seq + 4) for b in range(4)] +
                           [np.arange((b + 1) * per_seq - 4, (b + 1) * per_seq) for b in range(4)])
    rows = np.unique(np.concatenate([edges, sample_rows(n, 48, seed=216)]))
    check(inp, q, w_uk, w_uv, "bench size", rows=rows, out_dtype="bf16")


# A seeded random sweep of shapes: batch, heads, lengths (empty, one-token and
# page-edge ones among them), q_len from a decode step to a whole prefill, and
# the output dtype, drawn together.  Rows beyond a few hundred are sampled
# (first and last rows included), since the oracle expands each row's keys.
def _draw_mha_cases(n=40, seed=20261204):
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(g.integers(1, 5))
        H = int(g.choice([1, 2, 3, 8, 16, 33]))
        lens = [int(g.choice([0, 1, 127, 128, 129])) if g.random() < 0.3 else int(g.integers(1, 701))
                for _ in range(B)]
        if max(lens) == 0:
            lens[0] = 1
        T = [1, int(g.integers(2, 17)), max(lens)][i % 3]
        out_dtype = "f32" if g.random() < 0.5 else "bf16"
        cases.append(dict(B=B, H=H, T=T, lens=lens, out_dtype=out_dtype, seed=900 + i))
    return cases


MHA_CASES = _draw_mha_cases()


@pytest.mark.parametrize("case", MHA_CASES,
                         ids=["B%d-T%d-H%d-%s" % (c["B"], c["T"], c["H"], c["out_dtype"]) for c in MHA_CASES])
def test_dense_mha_random_shapes(case):
    inp = wl.make_inputs(case["B"], case["H"], case["T"], case["lens"], kv_dtype="bf16", out_dtype=case["out_dtype"],
                         seed=case["seed"], poison=True, extra_pages=1)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=case["seed"] + 50)
    n = inp.B * inp.T * inp.H
    rows = None if n <= 256 else np.unique(np.concatenate([sample_rows(n, 64, seed=case["seed"]),
                                                            np.arange(min(8, n)), np.arange(n - min(8, n), n)]))
    check(inp, q, w_uk, w_uv, "random lens=%s" % case["lens"], rows=rows, out_dtype=case["out_dtype"])


def test_dense_mha_graph_replay():
    """mla_dense_mha captured in a HIP graph: four replays, each after the
    outputs were overwritten with NaN and with an unrelated eager MHA call in
    between, equal the eager call bit for bit; the eager call matches the
    oracle.  The call allocates nothing and records no memset."""
    inp = wl.make_inputs(3, 8, 24, [24, 300, 5], kv_dtype="bf16", out_dtype="bf16", seed=214)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=314)
    g_in = inp.to(DEV)
    qd, ukd, uvd = q.to(DEV), w_uk.to(DEV), w_uv.to(DEV)
    need = binding.dense_mha_workspace_size(inp.B, inp.H, inp.max_seq_len)
    ws = torch.empty((need + 1) // 2, device=DEV, dtype=torch.bfloat16)

    def call(out, lse, stream=None):
        binding.mla_dense_mha(qd, g_in.q_pe, g_in.kv_cache, g_in.block_table, g_in.seq_lens, ukd, uvd,
                              g_in.max_seq_len, g_in.softmax_scale, out, lse, ws, stream=stream)

    eager_o = torch.empty((inp.B, inp.T, inp.H, 128), device=DEV, dtype=torch.bfloat16)
    eager_l = torch.empty((inp.B, inp.T, inp.H), device=DEV, dtype=torch.float32)
    _say("[gpu] mha graph: eager call")
    call(eager_o, eager_l)
    torch.cuda.synchronize()
    out, lse = torch.empty_like(eager_o), torch.empty_like(eager_l)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call(out, lse, stream=s)            # warm the stream
        torch.cuda.synchronize()
        _say("[gpu] mha graph: capture")
        with torch.cuda.graph(g, stream=s):
            call(out, lse, stream=s)
    other_o, other_l = torch.empty_like(eager_o), torch.empty_like(eager_l)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        _say("[gpu] mha graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l), "replay %d differs" % rep
        call(other_o, other_l)              # unrelated eager work between replays
        torch.cuda.synchronize()
    ref_o, ref_l = oracle_mha(inp, q, w_uk, w_uv)
    o = eager_o.double().cpu().reshape(-1, 128).numpy()
    allowed = TOL + half_ulp_bf16(np.maximum(np.abs(ref_o), np.abs(o)))
    assert np.all(np.abs(o - ref_o) <= allowed)
    l = eager_l.double().cpu().reshape(-1).numpy()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l))


def test_dense_mha_invalid_pages_clamped_lengths_and_no_lse():
    """The cache rules the C header gives the decode calls, through the MHA
    route: block-table entries naming no page (past the pool, negative) read
    as zero latents and zero rope parts, seq_lens -4 and 1000 with a
    five-page table (max_seq_len 1000) clamp to 0 and 320, and lse = NULL.
    Checked against the oracle on the equivalent valid input (the bad
    entries pointing at an appended zero page, the clamped lengths)."""
    inp = wl.make_inputs(3, 8, 4, [300, 320, 200], kv_dtype="bf16", out_dtype="f32", seed=215)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=315)
    assert inp.MB == 5
    NB = inp.NB
    bad = inp.block_table.clone()
    bad[2, 1] = NB + 3
    bad[2, 3] = -2
    call_in = wl.DecodeInputs(inp.q_nope, inp.q_pe, inp.kv_cache, bad, torch.tensor([-4, 1000, 200], dtype=torch.int32),
                              None, "bf16", "f32", inp.softmax_scale, max_len=1000)
    g = call_in.to(DEV)
    out = torch.full((inp.B, inp.T, inp.H, 128), float("nan"), device=DEV, dtype=torch.float32)
    _say("[gpu] mha: invalid pages, clamped lengths, no lse")
    binding.mla_dense_mha(q.to(DEV), g.q_pe, g.kv_cache, g.block_table, g.seq_lens, w_uk.to(DEV), w_uv.to(DEV),
                          g.max_seq_len, g.softmax_scale, out, None)
    torch.cuda.synchronize()
    invalid = (bad < 0) | (bad >= NB)
    ref_in = wl.DecodeInputs(inp.q_nope, inp.q_pe, torch.cat([inp.kv_cache, torch.zeros_like(inp.kv_cache[:1])]),
                             torch.where(invalid, torch.full_like(bad, NB), bad),
                             torch.tensor([0, 320, 200], dtype=torch.int32), None, "bf16", "f32", inp.softmax_scale)
    ref_o, _ = oracle_mha(ref_in, q, w_uk, w_uv)
    o = out.double().cpu().reshape(-1, 128).numpy()
    err = float(np.abs(o - ref_o).max())
    assert np.all(np.isfinite(o)) and err <= TOL, "max |out - oracle| = %.3g" % err
    assert not np.any(o[: inp.T * inp.H]), "the empty sequence's rows must be 0"
    _say("[gpu] mha invalid pages / clamped lengths: max |out - oracle| %.4g" % err)


def test_dense_mha_maximum_query_count():
    """The largest q_len the route accepts (MLA_MHA_MAX_Q_LEN = 65536): one
    65536-token prefill, one head; the first and last 64 queries and a random
    sample against the oracle."""
    T = binding.MHA_MAX_Q_LEN
    inp = wl.make_inputs(1, 1, T, [T], kv_dtype="bf16", out_dtype="bf16", seed=216)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=316)
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(T - 64, T), sample_rows(T, 96, seed=216)]))
    check(inp, q, w_uk, w_uv, "q_len %d" % T, rows=rows, out_dtype="bf16")


def test_dense_mha_lse_over_two_nearly_equal_keys():
    """One query over two keys whose second weight lies just under 1 (swept
    over 64 heads across several bf16 steps): lse = ln(1 + w2) exactly.  A
    sum of the bf16-rounded weights would be off by up to about 0.001 here
    (half a bf16 step of w2, over 1 + w2), at the 1e-3 bound; the LSE must
    follow the unrounded weights."""
    H = 64
    inp = wl.make_inputs(1, H, 1, [2], kv_dtype="bf16", out_dtype="f32", seed=217)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=317)
    q = torch.zeros_like(q)                                  # no-rope part: no contribution
    q_pe = torch.zeros_like(inp.q_pe)
    q_pe[0, 0, :, 0] = (1.0 + torch.arange(H, dtype=torch.float32) / H).to(q_pe.dtype)
    kv = inp.kv_cache.clone()
    page = int(inp.block_table[0, 0])
    kv[page, :2] = 0
    kv[page, 1, 512] = torch.tensor(-0.0271, dtype=torch.float32).to(kv.dtype)   # rope dim 0 of key 1
    inp = wl.DecodeInputs(inp.q_nope, q_pe, kv, inp.block_table, inp.seq_lens, None, "bf16", "f32",
                          inp.softmax_scale)
    out, lse = run_mha(inp, q, w_uk, w_uv)
    x = float(kv[page, 1, 512].float())
    a = q_pe[0, 0, :, 0].double()
    w2 = torch.exp(inp.softmax_scale * a * x)
    assert float(w2.min()) > 0.99 and float(w2.max()) < 1.0
    ref = torch.log1p(w2)
    err = float((lse[0, 0].double().cpu() - ref).abs().max())
    _say("[gpu] mha two near-equal keys: w2 in [%.5f, %.5f], max |lse - ln(1 + w2)| %.3g"
         % (float(w2.min()), float(w2.max()), err))
    assert err < 1e-5, "LSE follows rounded weights: %.3g" % err
    ref_o, _ = oracle_mha(inp, q, w_uk, w_uv)
    assert np.abs(out.double().cpu().reshape(-1, 128).numpy() - ref_o).max() <= TOL
