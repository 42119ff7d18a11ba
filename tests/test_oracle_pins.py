"""Pins of the fp64 oracle against facts fixed outside itself.

Each test ties one part of the oracle to the mathematics or to an
independent routine, so that a dropped term, a wrong sign or index, a
transposed operand or an off-by-one in the causal list fails at least one:

* absorption: brute-force un-absorbed MHA with explicit W_UK / W_UV
  (catches the q_pe term, the scale, the value = latent reading, paging);
* closed forms: one visible token (out = its latent, lse = its logit);
  q = 0 (uniform weights: out = mean latent, lse = ln n), which fixes the
  natural log and the causal count n = L - T + t + 1;
* invariances: split count, physical page permutation, causal reduction
  (query t of a T-token draft = a single query over L - T + t + 1 tokens);
* sparse: all positions as indices equals dense; the one-hot index probe
  gives the exact histogram of selected indices;
* dequantization: the e4m3fn and bf16 decoders against torch's casts.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mha_bruteforce as mha
from mla_paged_latent_03_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _paged(latents_per_seq, ropes_per_seq, P, rng, extra_pages=0, dtype=np.float64):
    """Lay sequences out in a shuffled page pool; returns kv [NB,P,576], block_table."""
    n_pages = [(len(c) + P - 1) // P for c in latents_per_seq]
    pool = sum(n_pages) + extra_pages
    perm = rng.permutation(pool)
    kv = np.full((pool, P, 576), np.nan, dtype=dtype)
    MB = max(n_pages)
    bt = np.full((len(n_pages), MB), -1, dtype=np.int32)
    off = 0
    for b, (c, r) in enumerate(zip(latents_per_seq, ropes_per_seq)):
        for p in range(n_pages[b]):
            page = perm[off + p]
            bt[b, p] = page
            lo, hi = p * P, min(len(c), (p + 1) * P)
            kv[page, :hi - lo, :512] = c[lo:hi]
            kv[page, :hi - lo, 512:] = r[lo:hi]
        off += n_pages[b]
    return kv, bt


def _tiny_f64(rng, B=2, T=1, H=3, lens=(5, 70), P=16):
    lat = [rng.standard_normal((L, 512)) for L in lens]
    rope = [rng.standard_normal((L, 64)) for L in lens]
    kv, bt = _paged(lat, rope, P, rng)
    qn = rng.standard_normal((B, T, H, 512))
    qp = rng.standard_normal((B, T, H, 64))
    return lat, rope, kv, bt, np.array(lens, dtype=np.int32), qn, qp


# ---------------------------------------------------------------- dequantization

def test_e4m3fn_decoder_matches_torch_all_256_bytes(oracle_lib):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for byte in range(256):
        mine = oracle.e4m3fn_to_float64(byte)
        want = ref[byte].item()
        if math.isnan(want):
            assert math.isnan(mine), byte
        else:
            assert mine == want, (byte, mine, want)
            assert math.copysign(1.0, mine) == math.copysign(1.0, want), byte


def test_e4m3fn_decoder_landmarks(oracle_lib):
    # Format facts: max finite 448, min normal 2^-6, min subnormal 2^-9, 0x7F NaN.
    assert oracle.e4m3fn_to_float64(0x7E) == 448.0
    assert oracle.e4m3fn_to_float64(0x08) == 2.0 ** -6
    assert oracle.e4m3fn_to_float64(0x01) == 2.0 ** -9
    assert oracle.e4m3fn_to_float64(0x38) == 1.0
    assert math.isnan(oracle.e4m3fn_to_float64(0x7F)) and math.isnan(oracle.e4m3fn_to_float64(0xFF))


def test_bf16_decoder_matches_torch(oracle_lib):
    bits = np.array([0, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x007F, 0x7F7F, 0x7F80, 0xFF80, 0x4049, 0x1234],
                    dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    for i, b in enumerate(bits):
        assert oracle.bf16_bits_to_float64(int(b)) == ref[i].item()


# ---------------------------------------------------------------- absorption pin

@pytest.mark.parametrize("P", [16, 64])
def test_absorbed_equals_unabsorbed_mha(oracle_lib, P):
    rng = np.random.default_rng(7)
    B, T, H, lens = 2, 3, 4, (5, 70)
    lat = [rng.standard_normal((L, 512)) for L in lens]
    rope = [rng.standard_normal((L, 64)) for L in lens]
    kv, bt = _paged(lat, rope, P, rng, extra_pages=2)
    w_uk = rng.standard_normal((H, mha.QK_NOPE, 512)) / math.sqrt(512)
    w_uv = rng.standard_normal((H, mha.V_HEAD, 512)) / math.sqrt(512)
    qn_heads = rng.standard_normal((B, T, H, mha.QK_NOPE))
    qp = rng.standard_normal((B, T, H, 64))
    q_abs = np.stack([np.stack([mha.absorb_query(qn_heads[b, t], w_uk) for t in range(T)]) for b in range(B)])
    scale = 1.0 / math.sqrt(mha.QK_NOPE + mha.QK_ROPE)
    out, lse = oracle.decode(q_abs, qp, kv, bt, np.array(lens, np.int32), softmax_scale=scale)
    out = out.reshape(B, T, H, 512)
    lse = lse.reshape(B, T, H)
    for b in range(B):
        for t in range(T):
            visible = list(range(lens[b] - T + t + 1))
            o_ref, lse_ref = mha.mha_decode(qn_heads[b, t], qp[b, t], lat[b], rope[b], w_uk, w_uv, scale, visible)
            o_abs = mha.project_output(out[b, t], w_uv)
            np.testing.assert_allclose(o_abs, o_ref, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(lse[b, t], lse_ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_single_token_closed_form(oracle_lib):
    rng = np.random.default_rng(11)
    lat, rope, kv, bt, lens, qn, qp = _tiny_f64(rng, B=1, T=1, H=5, lens=(1,), P=64)
    out, lse = oracle.decode(qn, qp, kv, bt, lens, softmax_scale=0.3)
    for h in range(5):
        assert np.array_equal(out[h], lat[0][0])          # weight exactly 1
        s0 = 0.3 * (qn[0, 0, h] @ lat[0][0] + qp[0, 0, h] @ rope[0][0])
        assert abs(lse[h] - s0) <= 1e-12 * max(1.0, abs(s0))


@pytest.mark.parametrize("T", [1, 3])
def test_zero_query_gives_uniform_weights(oracle_lib, T):
    rng = np.random.default_rng(12)
    lens = (7, 130)
    lat, rope, kv, bt, lens_a, qn, qp = _tiny_f64(rng, B=2, T=T, H=2, lens=lens, P=64)
    qn[:] = 0.0
    qp[:] = 0.0
    out, lse = oracle.decode(qn, qp, kv, bt, lens_a, softmax_scale=0.1)
    out = out.reshape(2, T, 2, 512)
    lse = lse.reshape(2, T, 2)
    for b in range(2):
        for t in range(T):
            n = lens[b] - T + t + 1
            mean = lat[b][:n].mean(axis=0)
            for h in range(2):
                np.testing.assert_allclose(out[b, t, h], mean, rtol=1e-12, atol=1e-13)
                assert abs(lse[b, t, h] - math.log(n)) < 1e-13


def test_empty_visible_list(oracle_lib):
    rng = np.random.default_rng(13)
    lat, rope, kv, bt, lens, qn, qp = _tiny_f64(rng, B=1, T=4, H=2, lens=(2,), P=64)
    out, lse = oracle.decode(qn, qp, kv, bt, lens, softmax_scale=0.2)
    out = out.reshape(4, 2, 512)
    lse = lse.reshape(4, 2)
    # Query t sees L - T + t + 1 = t - 1 tokens: t = 0, 1 see nothing.
    assert np.all(lse[:2] == -np.inf) and np.all(out[:2] == 0.0)
    assert np.all(np.isfinite(lse[2:]))
    assert np.array_equal(out[2, 0], lat[0][0])


# ---------------------------------------------------------------- invariances

@pytest.mark.parametrize("splits", [1, 2, 3, 7, 500])
def test_split_count_invariance(oracle_lib, splits):
    rng = np.random.default_rng(21)
    lat, rope, kv, bt, lens, qn, qp = _tiny_f64(rng, B=2, T=2, H=3, lens=(9, 150), P=64)
    ref_o, ref_l = oracle.decode(qn, qp, kv, bt, lens, softmax_scale=0.2)
    o, l = oracle.decode(qn, qp, kv, bt, lens, softmax_scale=0.2, num_splits=splits)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, ref_l, rtol=1e-13, atol=1e-13)


def test_page_permutation_invariance_is_exact(oracle_lib):
    rng = np.random.default_rng(22)
    lat, rope, kv, bt, lens, qn, qp = _tiny_f64(rng, B=2, T=2, H=3, lens=(40, 200), P=64)
    o1, l1 = oracle.decode(qn, qp, kv, bt, lens, softmax_scale=0.2)
    perm = rng.permutation(kv.shape[0])        # new physical page of old page p: inv[p]
    inv = np.argsort(perm)
    kv2 = kv[perm]
    bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1).astype(np.int32)
    o2, l2 = oracle.decode(qn, qp, kv2, bt2, lens, softmax_scale=0.2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_causal_reduction_to_single_query(oracle_lib):
    rng = np.random.default_rng(23)
    T = 4
    lat, rope, kv, bt, lens, qn, qp = _tiny_f64(rng, B=2, T=T, H=3, lens=(66, 129), P=64)
    o, l = oracle.decode(qn, qp, kv, bt, lens, softmax_scale=0.15)
    o = o.reshape(2, T, 3, 512)
    l = l.reshape(2, T, 3)
    for t in range(T):
        lens_t = (lens - T + t + 1).astype(np.int32)
        o1, l1 = oracle.decode(qn[:, t:t + 1], qp[:, t:t + 1], kv, bt, lens_t, softmax_scale=0.15)
        assert np.array_equal(o[:, t].reshape(-1, 512), o1)
        assert np.array_equal(l[:, t].reshape(-1), l1)


def test_bad_block_table_is_rejected(oracle_lib):
    rng = np.random.default_rng(24)
    lat, rope, kv, bt, lens, qn, qp = _tiny_f64(rng, B=1, T=1, H=1, lens=(10,), P=64)
    bt[0, 0] = kv.shape[0]
    with pytest.raises(ValueError):
        oracle.decode(qn, qp, kv, bt, lens, softmax_scale=0.1)


# ---------------------------------------------------------------- sparse

def test_sparse_all_positions_equals_dense(oracle_lib):
    rng = np.random.default_rng(31)
    lens = (37, 100)
    K = 128
    lat, rope, kv, bt, lens_a, qn, qp = _tiny_f64(rng, B=2, T=1, H=3, lens=lens, P=64)
    idx = np.full((2, 1, K), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        idx[b, 0, :L] = rng.permutation(L)
    o_d, l_d = oracle.decode(qn, qp, kv, bt, lens_a, softmax_scale=0.2)
    o_s, l_s = oracle.decode(qn, qp, kv, bt, lens_a, softmax_scale=0.2, topk_indices=idx)
    np.testing.assert_allclose(o_s, o_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_s, l_d, rtol=1e-13, atol=1e-13)


def test_sparse_index_probe_histogram(oracle_lib):
    """q = 0 and c_j = e_(j mod 512): n * out is the histogram of the selected
    in-range indices mod 512 (duplicates counted, out-of-range skipped)."""
    rng = np.random.default_rng(32)
    L, K, T = 1500, 700, 2
    lat = [np.eye(512)[np.arange(L) % 512]]
    rope = [rng.standard_normal((L, 64))]
    kv, bt = _paged(lat, rope, 64, rng)
    qn = np.zeros((1, T, 2, 512))
    qp = np.zeros((1, T, 2, 64))
    idx = rng.integers(-3, L + 3, size=(1, T, K)).astype(np.int32)  # includes -1..-3 and >= L
    idx[0, 0, :5] = 17                                               # duplicates
    o, l = oracle.decode(qn, qp, kv, bt, np.array([L], np.int32), softmax_scale=0.5, topk_indices=idx)
    o = o.reshape(T, 2, 512)
    l = l.reshape(T, 2)
    for t in range(T):
        sel = idx[0, t][(idx[0, t] >= 0) & (idx[0, t] < L)]
        n = sel.size
        hist = np.bincount(sel % 512, minlength=512)
        for h in range(2):
            assert np.array_equal(np.rint(n * o[t, h]).astype(np.int64), hist)
            assert np.max(np.abs(n * o[t, h] - hist)) < 1e-9
            assert abs(l[t, h] - math.log(n)) < 1e-12


# ---------------------------------------------------------------- fp8

def test_e4m3_with_power_of_two_scales_equals_dequantized_bf16(oracle_lib):
    inp = wl.make_inputs(2, 4, 2, [50, 130], kv_dtype="fp8", seed=5)
    # Replace the amax scales by powers of two: every e4m3fn value times 2^k is a bf16 value.
    qs, ks = 2.0 ** -5, 2.0 ** -7
    qn8, qp8 = wl.as_numpy_bits(inp.q_nope), wl.as_numpy_bits(inp.q_pe)
    kv8 = wl.as_numpy_bits(inp.kv_cache)
    bt, lens = inp.block_table.numpy(), inp.seq_lens.numpy()
    o8, l8 = oracle.decode(qn8, qp8, kv8, bt, lens, softmax_scale=inp.softmax_scale, q_scale=qs, kv_scale=ks)

    def to_bf16_bits(u8, s):
        v = torch.from_numpy(u8).view(torch.float8_e4m3fn).to(torch.float32) * s
        b = v.to(torch.bfloat16)
        assert torch.equal(b.to(torch.float32), v)   # exact
        return wl.as_numpy_bits(b)

    ob, lb = oracle.decode(to_bf16_bits(qn8, qs), to_bf16_bits(qp8, qs), to_bf16_bits(kv8, ks), bt, lens,
                           softmax_scale=inp.softmax_scale)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


# ---------------------------------------------------------------- brute force on the tiny workload

def test_tiny_workload_against_numpy_dense_softmax(oracle_lib):
    inp = wl.workload("tiny_b2_h16_kv37-300")
    qn = inp.q_nope.to(torch.float64).numpy()
    qp = inp.q_pe.to(torch.float64).numpy()
    kv = inp.kv_cache.to(torch.float64).numpy()
    bt, lens = inp.block_table.numpy(), inp.seq_lens.numpy()
    o, l = oracle.decode(wl.as_numpy_bits(inp.q_nope), wl.as_numpy_bits(inp.q_pe), wl.as_numpy_bits(inp.kv_cache),
                         bt, lens, softmax_scale=inp.softmax_scale)
    o = o.reshape(inp.B, inp.H, 512)
    l = l.reshape(inp.B, inp.H)
    for b in range(inp.B):
        L = int(lens[b])
        pos = np.arange(L)
        toks = kv[bt[b, pos // 64], pos % 64]           # [L, 576]
        q = np.concatenate([qn[b, 0], qp[b, 0]], axis=1)  # [H, 576]
        s = inp.softmax_scale * q @ toks.T               # [H, L]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        ref = (w @ toks[:, :512]) / w.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(o[b], ref, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(l[b], (m[:, 0] + np.log(w.sum(axis=1))), rtol=1e-13)


def test_paged_unabsorbed_mha_equals_projected_absorbed_oracle(oracle_lib):
    """The un-absorbed paged oracle (mha_bruteforce.mha_paged: its own paging,
    causal list and per-head expansion) against the C oracle's absorbed
    decode of q_abs = W_UK^T q_nope, projected by W_UV: the same attention,
    so equal to rounding (W_UK absorbed exactly in fp64), MTP rows that see
    nothing included."""
    import oracle.mha_bruteforce as mb
    rng = np.random.default_rng(31)
    B, T, H, P = 3, 3, 4, 16
    lens = [1, 20, 45]
    pages = [(L + P - 1) // P for L in lens]
    NB = sum(pages) + 2
    perm = rng.permutation(NB)
    bt = np.full((B, max(pages)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    kv = rng.standard_normal((NB, P, 576))
    q_nope = rng.standard_normal((B, T, H, 128))
    q_pe = rng.standard_normal((B, T, H, 64))
    w_uk = rng.standard_normal((H, 128, 512)) / np.sqrt(512)
    w_uv = rng.standard_normal((H, 128, 512)) / np.sqrt(512)
    scale = 1 / np.sqrt(192)
    o_mha, l_mha = mb.mha_paged(q_nope, q_pe, kv, bt, np.array(lens), w_uk, w_uv, scale)
    q_abs = np.stack([[mb.absorb_query(q_nope[b, t], w_uk) for t in range(T)] for b in range(B)])
    o_lat, l_lat = oracle.decode(q_abs, q_pe, kv, bt, np.array(lens, dtype=np.int32), softmax_scale=scale)
    o_proj = np.stack([mb.project_output(o_lat.reshape(B, T, H, 512)[b, t], w_uv) for b in range(B)
                       for t in range(T)]).reshape(-1, 128)
    fin = np.isfinite(l_lat)
    assert np.array_equal(np.isneginf(l_mha), np.isneginf(l_lat)) and (~fin).sum() == H * 2   # b=0: t=0,1 empty
    assert np.allclose(l_mha[fin], l_lat[fin], atol=1e-10, rtol=0)
    assert np.allclose(o_mha, o_proj, atol=1e-10, rtol=0)


def test_round_bf16_ties_and_one_step_rounding():
    """bf16 keeps 8 significant bits: the quantum at 1 is 2^-7; ties go to
    the even neighbour; the rounding is taken once from the float64 value
    (1 + 2^-8 + 2^-30 is above the tie, though float32 would first round it
    onto the tie and then down to 1)."""
    r = mha.round_bf16
    cases = [(1.0 + 2.0 ** -8, 1.0), (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6), (1.0 + 2.0 ** -8 + 2.0 ** -30,
             1.0 + 2.0 ** -7), (-(1.0 + 2.0 ** -8 + 2.0 ** -40), -(1.0 + 2.0 ** -7)), (0.0, 0.0),
             (3.0, 3.0), (255.5, 256.0), (257.0, 256.0), (259.0, 260.0), (2.0 ** -130 * 1.25, 2.0 ** -130 * 1.25),
             (2.0 ** -133 * 1.5, 2.0 ** -132), (2.0 ** -134, 0.0)]
    for x, want in cases:
        assert r(np.float64(x)) == want, (x, r(np.float64(x)), want)


def test_round_bf16_agrees_with_torch_on_float32_inputs():
    """On float32 inputs one-step rounding is torch's float32 -> bfloat16 cast
    (round to nearest even), normals and subnormals alike."""
    g = torch.Generator().manual_seed(41)
    x = torch.randn(20000, generator=g) * torch.exp2(torch.randint(-140, 60, (20000,), generator=g).float())
    x = torch.cat([x, torch.tensor([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.0 ** -127, 2.0 ** -149])])
    want = x.to(torch.bfloat16).double().numpy()
    got = mha.round_bf16(x.double().numpy())
    assert np.array_equal(got, want)


def test_bf16_expanded_mha_rounds_the_expanded_keys_and_values():
    """With selection matrices for W_UK and W_UV (each output row picks one
    latent feature), the up-projection copies latents, so rounding the
    expanded keys and values equals rounding the cache's latent part first
    and expanding exactly; with bf16-exact latents the two modes agree."""
    import oracle.mha_bruteforce as mb
    rng = np.random.default_rng(43)
    B, T, H, P = 2, 2, 3, 16
    lens = [20, 33]
    bt = np.array([[0, 1, -1], [2, 3, 4]], dtype=np.int32)
    kv = rng.standard_normal((5, P, 576))
    q_nope = rng.standard_normal((B, T, H, 128))
    q_pe = rng.standard_normal((B, T, H, 64))
    w_uk = np.zeros((H, 128, 512))
    w_uv = np.zeros((H, 128, 512))
    for h in range(H):
        w_uk[h, np.arange(128), rng.permutation(512)[:128]] = 1.0
        w_uv[h, np.arange(128), rng.permutation(512)[:128]] = 1.0
    scale = 1 / np.sqrt(192)
    o_b, l_b = mb.mha_paged(q_nope, q_pe, kv, bt, np.array(lens), w_uk, w_uv, scale, expanded="bf16")
    kv_r = kv.copy()
    kv_r[..., :512] = mb.round_bf16(kv[..., :512])
    o_f, l_f = mb.mha_paged(q_nope, q_pe, kv_r, bt, np.array(lens), w_uk, w_uv, scale, expanded="f64")
    assert np.array_equal(o_b, o_f) and np.array_equal(l_b, l_f)
    o_u, _ = mb.mha_paged(q_nope, q_pe, kv, bt, np.array(lens), w_uk, w_uv, scale, expanded="f64")
    assert np.abs(o_u - o_b).max() > 1e-6          # the rounding is not a no-op
    o_e, l_e = mb.mha_paged(q_nope, q_pe, kv_r, bt, np.array(lens), w_uk, w_uv, scale, expanded="bf16")
    assert np.array_equal(o_e, o_f) and np.array_equal(l_e, l_f)



def test_mha_oracle_two_keys_closed_form():
    """Zero latents (so zero no-rope keys and zero values) and rope keys 0 and
    x along one dimension: for a query whose rope part is a along it, the
    weights are 1 and exp(scale a x), so lse = ln(1 + exp(scale a x)) and the
    output is 0; a query that sees only the first key gets lse = 0.  Holds in
    both expansion modes."""
    import oracle.mha_bruteforce as mb
    H, T, P = 4, 2, 16
    a = np.array([1.0, 1.25, 1.5, 1.75])
    x = -0.02734375
    kv = np.zeros((1, P, 576))
    kv[0, 1, 512] = x
    bt = np.array([[0]], dtype=np.int32)
    q_nope = np.random.default_rng(44).standard_normal((1, T, H, 128))
    q_pe = np.zeros((1, T, H, 64))
    q_pe[0, :, :, 0] = a
    w = np.random.default_rng(45).standard_normal((H, 128, 512))
    scale = 1 / np.sqrt(192)
    for mode in ("f64", "bf16"):
        o, l = mb.mha_paged(q_nope, q_pe, kv, bt, np.array([2]), w, w, scale, expanded=mode)
        l = l.reshape(1, T, H)
        assert np.abs(o).max() == 0.0
        assert np.allclose(l[0, 0], 0.0, atol=1e-15)                       # draft token 0 sees key 0 only
        assert np.allclose(l[0, 1], np.log1p(np.exp(scale * a * x)), rtol=0, atol=1e-14)


def test_parity_bound_half_ulp_of_bf16():
    """The parity bound for bf16 outputs adds half a bf16 ulp of the value:
    exact at powers of two, and never exceeded by torch's round-to-nearest
    fp32 -> bf16 conversion."""
    from parity import half_ulp_bf16
    assert list(half_ulp_bf16(np.array([0.0, 1.0, 1.99, 2.0, -4.0, 7.9, 0.25]))) == \
        [0.0, 2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -10]
    x = np.random.default_rng(5).normal(0.0, 3.0, 100000).astype(np.float32)
    r = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    d = np.abs(r.astype(np.float64) - x)
    assert np.all(d <= half_ulp_bf16(np.maximum(np.abs(x), np.abs(r))))
    assert np.any(d > 0.99 * half_ulp_bf16(np.abs(x)))   # and it is tight: some roundings reach it
