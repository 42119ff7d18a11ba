"""GPU parity over a seeded random sweep of call shapes: cache dtype, dense or
sparse, q_len, head count, batch, length mix (with page edges, empty and
one-token sequences), top-k, requested split count and output dtype drawn
together, so that combinations the hand-picked cases do not list are
exercised too.  Small calls compare every output row with the fp64 oracle on
the same bytes; larger calls, drawn to land in the split planner's different
regimes, compare the first and last sequence's rows and a random sample.  The
draw happens at collection time from a fixed seed, so each case keeps its id;
sizes are capped so that the oracle finishes each in about a second.
"""
import sys

import numpy as np
import pytest
import torch

from mla_paged_latent_03_amd import binding, workloads as wl
from parity import compare, oracle_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 100
PAIR_CAP = 1_200_000          # (row, attended token) pairs per case
SPECIAL_LENS = [0, 1, 63, 64, 65, 127, 128, 129]


def _draw_cases():
    g = np.random.default_rng(20261203)
    cases = []
    for i in range(N_CASES):
        kind = ["bf16", "fp8", "sparse_bf16", "sparse_fp8"][i % 4]
        sparse = kind.startswith("sparse")
        T = int(g.integers(1, 9))
        H = int(g.choice([1, 2, 5, 8, 16, 24, 32, 40, 48, 64, 80, 96, 128, 160]))
        B = int(g.integers(1, 7))
        K = int(g.choice([32, 64, 96, 200, 512])) if sparse else 0
        if sparse:
            l_max = 8 * K + 100            # lengths below and above K; the cost is set by K
        else:
            l_max = min(4000, max(8, PAIR_CAP // (B * T * H)))
        lens = []
        for _ in range(B):
            if g.random() < 0.3:
                lens.append(int(g.choice(SPECIAL_LENS)))
            else:
                lens.append(int(g.integers(1, l_max + 1)))
        if max(lens) == 0:
            lens[0] = 1
        if sparse and B * T * H * K > PAIR_CAP:
            H = max(1, PAIR_CAP // (B * T * K))
        splits = int(g.choice([0, 0, 0, 1, 2, 3, 5]))
        out_dtype = "f32" if g.random() < 0.5 else "bf16"
        extra = int(g.integers(0, 3))
        cases.append(dict(kind=kind, B=B, T=T, H=H, K=K, lens=lens, splits=splits, out_dtype=out_dtype,
                          extra_pages=extra, seed=700 + i))
    return cases


CASES = _draw_cases()


def _id(c):
    return "%s-B%d-T%d-H%d-K%d-S%d-%s" % (c["kind"], c["B"], c["T"], c["H"], c["K"], c["splits"], c["out_dtype"])


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_against_oracle(case):
    kv_dtype = "fp8" if case["kind"].endswith("fp8") else "bf16"
    inp = wl.make_inputs(case["B"], case["H"], case["T"], case["lens"], kv_dtype=kv_dtype,
                         out_dtype=case["out_dtype"], topk=case["K"] or None, seed=case["seed"], poison=True,
                         extra_pages=case["extra_pages"])
    what = "random %s lens=%s" % (_id(case), case["lens"])
    print("[gpu] %s" % what, flush=True)
    sys.stdout.flush()
    g = inp.to(DEV)
    out, lse, _ = binding.decode(g, num_kv_splits=case["splits"])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_rows(inp)
    e = compare(out, lse, ref_o, ref_l, kv_dtype, what=what)
    print("[gpu] %s: max |out - oracle| %.4g, lse rel %.3g" % ((what,) + e), flush=True)


# Larger calls, drawn to land in the planner's different regimes (fixed
# chunks, length-balanced pieces, two longest-first rounds, several row
# blocks per sequence, long fp8 units with and without the residual product,
# sparse lists over long sequences), with sampled rows against the oracle.
N_LARGE = 20
TOKEN_CAP = 1_500_000        # cached tokens per call (bf16: 1.7 GB)


def _draw_large_cases():
    g = np.random.default_rng(20261205)
    cases = []
    for i in range(N_LARGE):
        kind = ["bf16", "fp8", "sparse_bf16", "sparse_fp8"][i % 4]
        sparse = kind.startswith("sparse")
        B = int(g.choice([1, 3, 17, 32, 64, 100, 200, 300]))
        T = int(g.integers(1, 9))
        H = int(g.choice([1, 8, 16, 32, 64, 128]))
        l_hi = int(g.choice([2000, 20000, 70000]))
        l_hi = max(64, min(l_hi, TOKEN_CAP // B))
        l_lo = int(g.integers(1, l_hi + 1)) if g.random() < 0.5 else l_hi
        lens = [int(x) for x in g.integers(l_lo, l_hi + 1, size=B)]
        K = int(g.choice([256, 1024, 2048])) if sparse else 0
        splits = int(g.choice([0, 0, 0, 2, 4]))
        cases.append(dict(kind=kind, B=B, T=T, H=H, K=K, lens=lens, splits=splits, seed=800 + i,
                          lo=l_lo, hi=l_hi))
    return cases


LARGE = _draw_large_cases()


def _large_id(c):
    return "%s-B%d-T%d-H%d-L%d..%d-K%d-S%d" % (c["kind"], c["B"], c["T"], c["H"], c["lo"], c["hi"], c["K"],
                                               c["splits"])


@pytest.mark.parametrize("case", LARGE, ids=[_large_id(c) for c in LARGE])
def test_random_large_call_sampled_rows(case):
    kv_dtype = "fp8" if case["kind"].endswith("fp8") else "bf16"
    inp = wl.make_inputs(case["B"], case["H"], case["T"], case["lens"], kv_dtype=kv_dtype, out_dtype="bf16",
                         topk=case["K"] or None, seed=case["seed"], device=DEV)
    what = "random large %s" % _large_id(case)
    waves = binding.launch_waves(inp.B, inp.T, inp.H, inp.max_len, case["K"], kv_dtype == "fp8")
    splits = binding.num_kv_splits(inp.B, inp.T, inp.H, inp.max_len, case["K"], kv_dtype == "fp8")
    print("[gpu] %s: planner %d waves, %d splits" % (what, waves, splits), flush=True)
    sys.stdout.flush()
    out, lse, _ = binding.decode(inp, num_kv_splits=case["splits"])
    torch.cuda.synchronize()
    n = inp.B * inp.T * inp.H
    R = inp.T * inp.H
    rows = np.unique(np.concatenate([np.arange(min(R, 64)), np.arange(max(0, n - min(R, 64)), n),
                                     np.random.default_rng(case["seed"]).choice(n, size=min(n, 96), replace=False)]))
    ref_o, ref_l = oracle_rows(inp, rows=rows)
    e = compare(out, lse, ref_o, ref_l, kv_dtype, rows=rows, what=what)
    print("[gpu] %s: max |out - oracle| %.4g, lse rel %.3g over %d rows" % ((what,) + e + (rows.size,)), flush=True)
