"""GPU test of mla_decode_fp8_noalloc (split partials in the library's static
buffer) against mla_decode_fp8 with a caller-owned workspace."""
import sys

import pytest
import torch

from mla_paged_latent_03_amd import binding, workloads as wl
from parity import TOL_OUT, TOL_LSE_REL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_the_workspace_entry_point_twice_then_refuses_oversize():
    # the second call is smaller than the first: it must not see stale partials
    cases = [([30000, 5000, 300, 20000], 32, 4, 4), ([700, 90], 16, 2, 3)]
    for lens, H, T, splits in cases:
        _say("[gpu] noalloc: lengths %s H=%d T=%d splits=%d" % (lens, H, T, splits))
        inp = wl.make_inputs(len(lens), H, T, lens, kv_dtype="fp8", out_dtype="bf16", seed=91 + H, poison=True)
        g = inp.to(DEV)
        need = binding.workspace_size(g.B, g.T, g.H, g.max_seq_len, 0, True, splits)
        assert 0 < need <= binding.STATIC_SCRATCH_BYTES
        ref_o, ref_l, _ = binding.decode(g, num_kv_splits=splits)
        out = torch.full_like(ref_o, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        binding.mla_decode_fp8_noalloc(g.q_nope, g.q_pe, g.kv_cache, g.block_table, g.seq_lens, g.max_seq_len,
                                       g.softmax_scale, g.q_scale, g.kv_scale, out, lse, splits)
        torch.cuda.synchronize()
        err_o = (out.float() - ref_o.float()).abs().max().item()
        fin = torch.isfinite(ref_l)
        assert torch.equal(torch.isneginf(lse), torch.isneginf(ref_l))
        err_l = ((lse[fin] - ref_l[fin]).abs() / ref_l[fin].abs().clamp(min=1.0)).max().item() if fin.any() else 0.0
        _say("[gpu] noalloc vs workspace call: max |out diff| %.3g, lse rel %.3g, identical %s"
             % (err_o, err_l, torch.equal(out, ref_o) and torch.equal(lse, ref_l)))
        assert err_o <= TOL_OUT["fp8"] and err_l <= TOL_LSE_REL
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)   # same plan and kernels
    # beyond the buffer: refused, nothing written
    big = wl.make_inputs(2, 32, 4, [2000, 2000], kv_dtype="fp8", out_dtype="bf16", seed=95).to(DEV)
    assert binding.workspace_size(2, 4, 32, big.max_seq_len, 0, True, binding.MAX_KV_SPLITS) > \
        binding.STATIC_SCRATCH_BYTES
    out = torch.zeros((2, 4, 32, 512), device=DEV, dtype=torch.bfloat16)
    with pytest.raises(binding.MLAError) as ei:
        binding.mla_decode_fp8_noalloc(big.q_nope, big.q_pe, big.kv_cache, big.block_table, big.seq_lens,
                                       big.max_seq_len, big.softmax_scale, big.q_scale, big.kv_scale, out, None,
                                       binding.MAX_KV_SPLITS)
    assert ei.value.status == binding.MLA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_noalloc_replayed_from_a_graph():
    """Captured in a HIP graph (its partials in the static buffer, no memset
    recorded): three replays, each after the outputs were overwritten with
    NaN and with a differently shaped eager call of the same entry point in
    between (which reuses the buffer), equal the eager call bit for bit."""
    inp = wl.make_inputs(3, 32, 4, [25000, 800, 18000], kv_dtype="fp8", out_dtype="bf16", seed=96).to(DEV)
    other = wl.make_inputs(2, 16, 2, [3000, 40], kv_dtype="fp8", out_dtype="bf16", seed=97).to(DEV)
    splits = 4

    def call(x, out, lse, stream=None):
        binding.mla_decode_fp8_noalloc(x.q_nope, x.q_pe, x.kv_cache, x.block_table, x.seq_lens, x.max_seq_len,
                                       x.softmax_scale, x.q_scale, x.kv_scale, out, lse, splits, stream=stream)

    shape = (inp.B, inp.T, inp.H, 512)
    eager_o = torch.empty(shape, device=DEV, dtype=torch.bfloat16)
    eager_l = torch.empty(shape[:3], device=DEV, dtype=torch.float32)
    _say("[gpu] noalloc graph: eager call")
    call(inp, eager_o, eager_l)
    torch.cuda.synchronize()
    out, lse = torch.empty_like(eager_o), torch.empty_like(eager_l)
    o2 = torch.empty((other.B, other.T, other.H, 512), device=DEV, dtype=torch.bfloat16)
    l2 = torch.empty((other.B, other.T, other.H), device=DEV, dtype=torch.float32)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call(inp, out, lse, stream=s)       # warm the stream
        torch.cuda.synchronize()
        _say("[gpu] noalloc graph: capture")
        with torch.cuda.graph(g, stream=s):
            call(inp, out, lse, stream=s)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        _say("[gpu] noalloc graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l), "replay %d differs" % rep
        call(other, o2, l2)                 # reuses the static buffer between replays
        torch.cuda.synchronize()


def test_noalloc_at_the_largest_workspace_it_holds():
    """B = 127 sequences of 128 rows with two splits need 99.4% of the static
    buffer (one more sequence would not fit and is refused): the call equals
    the workspace entry point bit for bit, and a smaller call after it too."""
    splits = 2
    inp = wl.make_inputs(127, 32, 4, (150, 260), kv_dtype="fp8", out_dtype="bf16", seed=98).to(DEV)
    need = binding.workspace_size(inp.B, inp.T, inp.H, inp.max_seq_len, 0, True, splits)
    assert 0.99 * binding.STATIC_SCRATCH_BYTES < need <= binding.STATIC_SCRATCH_BYTES
    assert binding.workspace_size(inp.B + 1, inp.T, inp.H, inp.max_seq_len, 0, True, splits) > \
        binding.STATIC_SCRATCH_BYTES
    for x in (inp, wl.make_inputs(3, 32, 4, [220, 90, 1], kv_dtype="fp8", out_dtype="bf16", seed=99).to(DEV)):
        _say("[gpu] noalloc near the buffer limit: B=%d, workspace %d bytes" %
             (x.B, binding.workspace_size(x.B, x.T, x.H, x.max_seq_len, 0, True, splits)))
        ref_o, ref_l, _ = binding.decode(x, num_kv_splits=splits)
        out = torch.full_like(ref_o, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        binding.mla_decode_fp8_noalloc(x.q_nope, x.q_pe, x.kv_cache, x.block_table, x.seq_lens, x.max_seq_len,
                                       x.softmax_scale, x.q_scale, x.kv_scale, out, lse, splits)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
