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
