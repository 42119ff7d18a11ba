#!/usr/bin/env python3
"""Benchmark of the MLA paged-latent decode hot path on one MI355X.

One step = one full decode call over one batch of synthetic input (the
split-KV partial kernel and, with more than one split, the LSE merge
kernel), inputs already resident in HBM.  Default workload: the 80k-token
MTP-3 fp8 decode (B=64, H=32, q_len=4, block 64), the configuration the
target is quoted on.  Prints ONE JSON line on stdout; details go to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0                  # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}   # dense MFMA
FLOPS_PER_PAIR = 2 * 576 + 2 * 512     # QK over 576 features + PV over 512
DEFAULT_WORKLOAD = "mtp3_b64_h32_kv80k_fp8"
KERNEL_SOURCES = [os.path.join(ROOT, "mla_paged_latent_03_amd", "csrc", f)
                  for f in ("mla_decode_kernels.hip", "mla_decode_api.cpp", "mla_decode_internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_cost(inp):
    """Bytes the method must move and FLOPs it must do, from the host copy of
    the lengths / indices (tokens attended read once per sequence)."""
    lens = inp.seq_lens.cpu().numpy().astype(np.int64)
    B, T, H = inp.B, inp.T, inp.H
    elt = 1 if inp.kv_dtype == "fp8" else 2
    out_elt = 4 if inp.out_dtype == "f32" else 2
    rows = B * T * H
    if inp.topk_indices is None:
        kv_tokens = int(lens.sum())
        pairs = sum(H * max(0, int(L) - T + t + 1) for L in lens for t in range(T))
        meta = int(((lens + 63) // 64).sum()) * 4                       # block-table entries
    else:
        idx = inp.topk_indices.cpu().numpy()
        valid = (idx >= 0) & (idx < lens[:, None, None])
        kv_tokens = int(valid.sum())                                   # gathered rows (per query token)
        pairs = H * kv_tokens
        meta = idx.size * 4 * 2                                        # indices + their block-table entries
    kv_bytes = kv_tokens * 576 * elt
    q_bytes = rows * 576 * elt
    out_bytes = rows * 512 * out_elt + rows * 4
    flops = pairs * FLOPS_PER_PAIR
    return dict(kv_bytes=kv_bytes, q_bytes=q_bytes, out_bytes=out_bytes, meta_bytes=meta,
                total_bytes=kv_bytes + q_bytes + out_bytes + meta, partial_bytes=kv_bytes + q_bytes + meta,
                flops=flops, kv_tokens=kv_tokens)


def cpu_baseline(inp, seconds: float):
    """The fp64 oracle, as it stands, on a bounded sample of rows; scaled to
    the whole call (every row costs the same visible-list work for the
    uniform-length workloads, and the sample is drawn uniformly otherwise)."""
    import oracle
    from mla_paged_latent_03_amd import workloads as wl
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cpu = inp.to("cpu")
    args = dict(q_nope=wl.as_numpy_bits(cpu.q_nope), q_pe=wl.as_numpy_bits(cpu.q_pe),
                kv_cache=wl.as_numpy_bits(cpu.kv_cache), block_table=cpu.block_table.numpy(),
                seq_lens=cpu.seq_lens.numpy())
    topk = None if cpu.topk_indices is None else cpu.topk_indices.numpy()
    total = inp.B * inp.T * inp.H
    rng = np.random.default_rng(0)
    n = min(total, max(cores, 16))
    t_first = None
    while True:
        rows = np.sort(rng.choice(total, size=n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.decode(args["q_nope"], args["q_pe"], args["kv_cache"], args["block_table"], args["seq_lens"],
                      softmax_scale=inp.softmax_scale, q_scale=inp.q_scale, kv_scale=inp.kv_scale,
                      topk_indices=topk, rows=rows, threads=cores)
        dt = time.perf_counter() - t0
        if t_first is None and dt < seconds / 4 and n < total:
            t_first = dt
            n = int(min(total, max(n + 1, n * seconds / max(dt, 1e-3))))
            continue
        break
    us_per_call = dt * (total / n) * 1e6
    return dict(value=us_per_call, unit="us/call", cores=cores, kind="oracle",
                sample="%d of %d output rows (random, seed 0), fp64 oracle, %.1f s wall, scaled to all rows"
                       % (n, total, dt))


def stream_reference_lib():
    """The benchmark's streaming-read reference kernel, if built."""
    path = os.path.join(ROOT, "mla_paged_latent_03_amd", "libmla_stream_ref.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mla_stream_read_reference.restype = ctypes.c_int
    lib.mla_stream_read_reference.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_void_p]
    return lib


def lds_rate(args):
    """LDS read rate of this GPU, from the reference library's read-rate
    kernel: bytes per shader clock for 16-byte ds_read_b128 reads, by waves
    per workgroup and reads each lane keeps in flight, one workgroup per
    compute unit.  Prints one JSON line."""
    import torch
    lib = stream_reference_lib()
    if lib is None:
        raise SystemExit("libmla_stream_ref.so is not built: run __graft_entry__.build() first")
    fn = lib.mla_lds_read_rate_reference
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    dev = torch.device("cuda:0")
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev).cuda_stream
    rows = []
    for waves in (1, 2, 4, 8, 16):
        for inflight in (2, 4, 8, 16):
            iters = 64000 // inflight                      # 64000 reads per lane
            sink = torch.empty(n_cu * 64 * waves, dtype=torch.int32, device=dev)
            clocks = torch.zeros(2 * n_cu, dtype=torch.int64, device=dev)
            khz = ctypes.c_int(0)
            for _ in range(2):                             # the first launch warms up
                rc = fn(waves, inflight, n_cu, iters, sink.data_ptr(), clocks.data_ptr(), ctypes.byref(khz), stream)
                if rc != 0:
                    raise SystemExit("mla_lds_read_rate_reference failed (%d)" % rc)
            torch.cuda.synchronize()
            c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
            cyc, ticks = float(np.median(c[:, 0])), float(np.median(c[:, 1]))
            per_wg = 64.0 * waves * iters * inflight * 16 / cyc
            rows.append({"waves": waves, "reads_in_flight_per_wave": inflight,
                         "bytes_per_clk_per_workgroup": round(per_wg, 1),
                         "bytes_per_clk_per_wave": round(per_wg / waves, 1),
                         "clock_MHz": round(cyc / (ticks / (khz.value * 1e3)) / 1e6, 0)})
            log("[bench] lds rate: %2d waves, %2d reads in flight: %6.1f B/clk per workgroup (%5.1f per wave)"
                % (waves, inflight, per_wg, per_wg / waves))
    print(json.dumps({"mode": "lds_rate", "read": "ds_read_b128, 16 B per lane, 64 KiB LDS array",
                      "workgroups": n_cu, "rows": rows}), flush=True)


def load_traffic(workload: str):
    """HBM bytes per launch of the partial kernel from the rocprofv3 PMC runs
    recorded for this workload, if they were taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def _timed(fn, steps, warmup, stream):
    """Median / p10 / p90 of per-call HIP-event times (us) of fn() on stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2), "mean": round(float(us.mean()), 2)}


def mha_vs_mqa(args):
    """A prefill batch (q_len = L for every sequence, causal) whose sequences
    all fit in top-k, run both ways on the same cache, queries and
    up-projections:
      * dense MHA: one mla_dense_mha call (expansion of the latents by
        [W_UK; W_UV] and the attention, both in the library);
      * sparse MQA: the query absorbed by W_UK (torch bmm), one
        mla_sparse_decode call over one single-query row per token whose
        index list holds every position it sees, the latent output
        projected by W_UV (torch bmm).
    Prints one JSON line: both times, the speed-up, the dense call's MFMA
    roofline, and the largest difference between the two outputs."""
    import torch
    from mla_paged_latent_03_amd import binding, workloads as wl

    B, L, H, K = args.mha_batch, args.mha_len, args.mha_heads, 2048
    if L > K:
        raise SystemExit("--mha-len must be <= top-k (2048): the dense route serves sequences that fit in top-k")
    binding.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    name = "prefill_b%d_h%d_len%d_top%d_bf16" % (B, H, L, K)
    log("[bench] drawing %s" % name)
    inp = wl.make_inputs(B, H, L, [L] * B, kv_dtype="bf16", out_dtype="bf16", seed=1101, device=dev, name=name)
    q, w_uk, w_uv = wl.mha_inputs(inp, seed=1102, device=dev)
    rows = B * L

    out_mha = torch.empty((B, L, H, 128), device=dev, dtype=torch.bfloat16)
    lse_mha = torch.empty((B, L, H), device=dev, dtype=torch.float32)
    ws_mha = torch.empty((binding.dense_mha_workspace_size(B, H, L) + 1) // 2, device=dev, dtype=torch.bfloat16)

    def mha():
        binding.mla_dense_mha(q, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, w_uk, w_uv, L,
                              inp.softmax_scale, out_mha, lse_mha, ws_mha, stream)

    # MQA side: per-head batched products with contiguous operands.
    q_h = q.reshape(rows, H, 128).transpose(0, 1).contiguous()            # [H, rows, 128]
    w_uv_t = w_uv.transpose(1, 2).contiguous()                            # [H, 512, 128]
    q_abs_h = torch.empty((H, rows, 512), device=dev, dtype=torch.bfloat16)
    q_abs = torch.empty((rows, H, 512), device=dev, dtype=torch.bfloat16)
    sp = wl.prefill_rows_as_sparse_decode(inp, q_abs.reshape(B, L, H, 512), K)
    assert sp.q_nope.data_ptr() == q_abs.data_ptr()
    lat = torch.empty((rows, 1, H, 512), device=dev, dtype=torch.bfloat16)
    lse_mqa = torch.empty((rows, 1, H), device=dev, dtype=torch.float32)
    S = binding.num_kv_splits(rows, 1, H, L, K, False)
    need = binding.workspace_size(rows, 1, H, L, K, False, S)
    ws_mqa = torch.empty(max(1, (need + 3) // 4), device=dev, dtype=torch.float32)
    lat_h = torch.empty((H, rows, 512), device=dev, dtype=torch.bfloat16)
    out_mqa_h = torch.empty((H, rows, 128), device=dev, dtype=torch.bfloat16)

    def absorb():
        torch.bmm(q_h, w_uk, out=q_abs_h)
        q_abs.copy_(q_abs_h.transpose(0, 1))        # sp.q_nope is a view of q_abs

    def attend():
        binding.mla_sparse_decode(sp.q_nope, sp.q_pe, sp.kv_cache, sp.block_table, sp.seq_lens, sp.topk_indices,
                                  L, sp.softmax_scale, lat, lse_mqa, ws_mqa, S, stream)

    def project():
        lat_h.copy_(lat.view(rows, H, 512).transpose(0, 1))
        torch.bmm(lat_h, w_uv_t, out=out_mqa_h)

    def mqa():
        absorb()
        attend()
        project()

    t_mha = _timed(mha, args.steps, args.warmup, stream)
    t_mqa = _timed(mqa, args.steps, args.warmup, stream)
    t_attend = _timed(attend, args.steps, args.warmup, stream)
    mha()
    mqa()
    torch.cuda.synchronize()
    diff = float((out_mha.float().reshape(rows, H, 128) - out_mqa_h.float().transpose(0, 1)).abs().max())
    lse_diff = float((lse_mha.reshape(-1) - lse_mqa.reshape(-1)).abs().max())
    pairs = H * B * L * (L + 1) // 2
    flops_expand = 2 * B * L * H * 256 * 512
    flops_attn = pairs * 2 * (192 + 128)
    flops = flops_expand + flops_attn
    ach = flops / (t_mha["median"] * 1e-6) / 1e12
    res = {
        "metric": "dense MHA vs sparse MQA on a prefill batch that fits in top-k: us per batch",
        "value": t_mha["median"], "unit": "us/batch", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic (seeded N(0,1) latents and queries, "
        "N(0,1/512) up-projections, shuffled pages)",
        "config": {"workload": name, "batch": B, "heads": H, "q_len": L, "seq_len": L, "topk": K,
                   "mqa_rows": rows, "mqa_kv_splits": S},
        "mha_us": t_mha, "mqa_us": t_mqa, "mqa_attention_only_us": t_attend,
        "speedup_mha_over_mqa": round(t_mqa["median"] / t_mha["median"], 3),
        "roofline": {"bound": "mfma", "kernel": "mla_dense_mha (expand + attention)",
                     "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                     "frac": round(ach / MFMA_PEAK_TFLOPS["bf16"], 4), "flops": flops,
                     "flops_expand": flops_expand, "flops_attention": flops_attn},
        "max_abs_out_diff_mha_vs_mqa": round(diff, 5), "max_abs_lse_diff_mha_vs_mqa": round(lse_diff, 5),
    }
    print(json.dumps(res), flush=True)


def _smi():
    """(amdsmi module, handle of GPU 0), or None when the library cannot
    reach the device."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        return amdsmi, amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:   # library missing or no device
        log("[bench] amdsmi unavailable: %s" % e)
        return None


def sustain(args):
    """Socket power, GFX clock and power-limit residency under a sustained
    load: the workload's whole decode call back to back (rotating input sets
    as the timed benchmark does), the streaming-read reference over the same
    KV bytes, the dense MHA call of --mha-vs-mqa, or nothing (idle).  Prints
    one JSON line."""
    import threading
    import torch
    from mla_paged_latent_03_amd import binding, workloads as wl

    smi = _smi()
    if smi is None:
        raise SystemExit("--sustain needs amdsmi and a GPU")
    amdsmi, h = smi
    binding.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    run = None
    bytes_per_call = flops_per_call = 0
    if args.sustain_kind in ("decode", "stream"):
        log("[bench] drawing %s on %s" % (args.workload, dev))
        inp = wl.workload(args.workload, device=dev)
    if args.sustain_kind == "decode":
        fp8 = inp.kv_dtype == "fp8"
        S = binding.num_kv_splits(inp.B, inp.T, inp.H, inp.max_seq_len, inp.K, fp8)
        out = torch.empty((inp.B, inp.T, inp.H, 512), device=dev,
                          dtype=torch.float32 if inp.out_dtype == "f32" else torch.bfloat16)
        lse = torch.empty((inp.B, inp.T, inp.H), device=dev, dtype=torch.float32)
        ws_bytes = binding.workspace_size(inp.B, inp.T, inp.H, inp.max_seq_len, inp.K, fp8, S)
        ws = torch.empty(max(1, (ws_bytes + 3) // 4), device=dev, dtype=torch.float32) if ws_bytes else None
        sets = [inp]
        if algorithmic_cost(inp)["total_bytes"] < (512 << 20):
            seed0 = wl.WORKLOADS[args.workload]["seed"]
            sets += [wl.workload(args.workload, device=dev, seed=seed0 + 100 * k) for k in (1, 2)]
        calls = [binding.prepare_decode(x, S, out, lse, ws, stream) for x in sets]
        cost = algorithmic_cost(inp)
        bytes_per_call, flops_per_call = cost["total_bytes"], cost["flops"]

        def run(k):
            calls[k % len(calls)]()
    elif args.sustain_kind == "mha":
        B, L, H = args.mha_batch, args.mha_len, args.mha_heads
        inp = wl.make_inputs(B, H, L, [L] * B, kv_dtype="bf16", out_dtype="bf16", seed=1101, device=dev)
        q, w_uk, w_uv = wl.mha_inputs(inp, seed=1102, device=dev)
        out = torch.empty((B, L, H, 128), device=dev, dtype=torch.bfloat16)
        lse = torch.empty((B, L, H), device=dev, dtype=torch.float32)
        ws = torch.empty((binding.dense_mha_workspace_size(B, H, L) + 1) // 2, device=dev, dtype=torch.bfloat16)
        flops_per_call = 2 * 256 * 512 * B * L * H + 2 * (192 + 128) * H * B * L * (L + 1) // 2

        def run(k):
            binding.mla_dense_mha(q, inp.q_pe, inp.kv_cache, inp.block_table, inp.seq_lens, w_uk, w_uv, L,
                                  inp.softmax_scale, out, lse, ws, stream)
    elif args.sustain_kind == "stream":
        ref_lib = stream_reference_lib()
        if ref_lib is None:
            raise SystemExit("the streaming reference library is not built")
        nbytes = (inp.kv_cache.numel() * inp.kv_cache.element_size() // 36864) * 36864
        sink = torch.empty(256, dtype=torch.int32, device=dev)
        bytes_per_call = nbytes

        def run(k):
            rc = ref_lib.mla_stream_read_reference(ctypes.c_void_p(inp.kv_cache.data_ptr()), nbytes, 256,
                                                   ctypes.c_void_p(sink.data_ptr()),
                                                   ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError("stream reference failed (%d)" % rc)

    def metrics():
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        e = amdsmi.amdsmi_get_energy_count(h)
        return m, e["energy_accumulator"] * e["counter_resolution"] * 1e-6   # J

    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, int)]
            samples.append((m.get("current_socket_power"), float(np.mean(clks)) if clks else None))
            stop.wait(0.1)

    if run is not None:   # a short burst first, so that the sampled window is the sustained state
        t_end = time.perf_counter() + 0.5
        k = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                run(k)
                k += 1
            torch.cuda.synchronize()
    m0, j0 = metrics()
    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    next_note = t0 + 1.0
    while time.perf_counter() - t0 < args.sustain:
        if run is None:
            time.sleep(0.05)
        else:
            for _ in range(16):
                run(n)
                n += 1
            torch.cuda.synchronize()
        if time.perf_counter() >= next_note:
            log("[bench] sustain %s: %.0f s, %d calls" % (args.sustain_kind, time.perf_counter() - t0, n))
            next_note += 1.0
    dt = time.perf_counter() - t0
    m1, j1 = metrics()
    stop.set()
    th.join()
    d_acc = m1["accumulation_counter"] - m0["accumulation_counter"]

    def residency(key):
        try:
            return round((m1[key] - m0[key]) / d_acc, 4) if d_acc else None
        except TypeError:   # counter not reported ("N/A")
            return None

    pw = np.array([s[0] for s in samples if isinstance(s[0], (int, float))], dtype=float)
    ck = np.array([s[1] for s in samples if s[1] is not None], dtype=float)

    def stats(x):
        return ({"median": round(float(np.median(x)), 1), "p10": round(float(np.percentile(x, 10)), 1),
                 "p90": round(float(np.percentile(x, 90)), 1)} if x.size else None)

    try:
        cap = amdsmi.amdsmi_get_power_cap_info(h)
    except Exception:
        cap = {}
    res = {"mode": "sustain", "kind": args.sustain_kind,
           "workload": ("prefill_b%d_h%d_len%d_bf16" % (args.mha_batch, args.mha_heads, args.mha_len)
                        if args.sustain_kind == "mha" else args.workload if run is not None else None),
           "seconds": round(dt, 2), "calls": n,
           "us_per_call": round(dt / n * 1e6, 2) if n else None,
           "socket_power_W": stats(pw), "gfx_clock_MHz": stats(ck), "samples": int(pw.size),
           "energy_J": round(j1 - j0, 2), "mean_power_W": round((j1 - j0) / dt, 1),
           "energy_per_call_mJ": round((j1 - j0) / n * 1e3, 3) if n else None,
           "ppt_residency": residency("ppt_residency_acc"),
           "socket_thermal_residency": residency("socket_thm_residency_acc"),
           "hbm_thermal_residency": residency("hbm_thm_residency_acc"),
           "power_cap_W": (cap.get("power_cap") / 1e6 if isinstance(cap.get("power_cap"), (int, float)) else None),
           "achieved_TBps": round(bytes_per_call * n / dt / 1e12, 3) if n and bytes_per_call else None,
           "achieved_TFLOPs": round(flops_per_call * n / dt / 1e12, 1) if n and flops_per_call else None,
           "source_hash": source_hash()}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="run calls for this long before the warm-up, past the clock transient (0: none)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's choice")
    ap.add_argument("--single-launch", action="store_true",
                    help="request the single-launch form (MLA_SINGLE_LAUNCH=1): split units merge in-kernel")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mha-vs-mqa", action="store_true",
                    help="instead: a prefill batch whose sequences all fit in top-k, through the dense "
                         "un-absorbed MHA call and through the sparse absorbed MQA call on the same inputs")
    ap.add_argument("--mha-batch", type=int, default=4)
    ap.add_argument("--mha-len", type=int, default=2048, help="sequence length = query tokens (prefill)")
    ap.add_argument("--mha-heads", type=int, default=128)
    ap.add_argument("--copy-calibration-gib", type=int, default=0,
                    help="first copy a buffer of this many GiB three times, so that a counter run over the "
                         "benchmark also reads the counters for a plain copy of known size")
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="instead of the timed benchmark: run the load back to back for this many seconds and "
                         "report socket power, GFX clock and power-limit residency (amdsmi)")
    ap.add_argument("--sustain-kind", choices=("decode", "stream", "mha", "idle"), default="decode",
                    help="load of --sustain: the workload's decode call, the streaming-read reference over its "
                         "KV bytes, the dense MHA call of --mha-vs-mqa, or none")
    ap.add_argument("--lds-rate", action="store_true",
                    help="instead of the timed benchmark: measure the LDS read rate (bytes per clock) by waves "
                         "per workgroup and reads in flight per wave")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this decode library runs on a single GPU "
              "(its sequence-sharded multi-GPU form is not implemented). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.mha_vs_mqa:
        mha_vs_mqa(args)
        return
    if args.sustain > 0:
        sustain(args)
        return
    if args.lds_rate:
        lds_rate(args)
        return
    if args.single_launch:
        os.environ["MLA_SINGLE_LAUNCH"] = "1"
    else:
        os.environ.pop("MLA_SINGLE_LAUNCH", None)
    import torch
    from mla_paged_latent_03_amd import binding, workloads as wl

    binding.load()
    dev = torch.device("cuda:0")
    log("[bench] drawing %s on %s" % (args.workload, dev))
    inp = wl.workload(args.workload, device=dev)
    fp8 = inp.kv_dtype == "fp8"
    S = args.splits or binding.num_kv_splits(inp.B, inp.T, inp.H, inp.max_seq_len, inp.K, fp8)
    out = torch.empty((inp.B, inp.T, inp.H, 512), device=dev,
                      dtype=torch.float32 if inp.out_dtype == "f32" else torch.bfloat16)
    lse = torch.empty((inp.B, inp.T, inp.H), device=dev, dtype=torch.float32)
    ws_bytes = binding.workspace_size(inp.B, inp.T, inp.H, inp.max_seq_len, inp.K, fp8, S)
    partial_bytes = inp.B * inp.T * inp.H * S * 513 * 4 if S > 1 else 0
    single = ws_bytes > partial_bytes          # the plan adds the group words of the single-launch form
    ws = torch.empty(max(1, (ws_bytes + 3) // 4), device=dev, dtype=torch.float32) if ws_bytes else None
    stream = torch.cuda.current_stream()

    # A working set that fits the 256 MB last-level cache (MALL) would be
    # timed from that cache on repeated calls, so small workloads rotate over
    # three independently drawn input sets of the same shape.
    sets = [inp]
    if algorithmic_cost(inp)["total_bytes"] < (512 << 20):
        seed0 = wl.WORKLOADS[args.workload]["seed"]
        sets += [wl.workload(args.workload, device=dev, seed=seed0 + 100 * k) for k in (1, 2)]
        log("[bench] rotating %d input sets (working set below the last-level cache)" % len(sets))
    calls = [0]
    # Each call's C arguments are marshalled once, outside the timed region.
    stage1 = [binding.prepare_decode(x, S, None, None, ws, stream) for x in sets]
    whole = [binding.prepare_decode(x, S, out, lse, ws, stream) for x in sets]
    merge = binding.prepare_merge(ws, inp.B * inp.T * inp.H, S, out, lse, stream) if S > 1 else None

    def launch(stage1_only):
        k = calls[0] % len(sets)
        (stage1 if stage1_only else whole)[k]()

    def step(ev=None):
        """One decode call.  With more than one split it is issued as its two
        stages (first stage, then the merge: the same launches, bit for bit,
        as one call), so that an event can sit between them; ev = (start,
        after the first stage, end) events or None."""
        if ev is not None:
            ev[0].record(stream)
        if S > 1 and not single:
            launch(stage1_only=True)
            if ev is not None:
                ev[1].record(stream)
            merge()
        else:
            launch(stage1_only=False)
            if ev is not None:
                ev[1].record(stream)
        if ev is not None:
            ev[2].record(stream)
        calls[0] += 1

    if args.copy_calibration_gib > 0:
        src = torch.ones(args.copy_calibration_gib << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied %d GiB three times" % args.copy_calibration_gib)
        del src, dst

    # The GPU clock moves for the first ~15 ms of a burst of decode calls
    # (fast on an idle GPU, then a dip below the sustained rate, then steady:
    # power management under full-rate HBM reads plus matrix products).  The
    # settle phase runs calls until that has passed, so that the warm-up and
    # timed steps see the sustained rate whatever --warmup is.
    settle_calls = 0
    if args.settle_ms > 0:
        t_end = time.perf_counter() + args.settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(4):
                step()
                settle_calls += 1
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("[bench] settled with %d calls, %d warm-up; timing %d steps (splits=%d)"
        % (settle_calls, args.warmup, args.steps, S))
    # The timed region: exactly K calls issued back to back, with events only
    # at its two ends (an event recorded between a call's two stages adds
    # about 10 us to the call, which a caller does not pay).
    t_a = torch.cuda.Event(enable_timing=True)
    t_b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_a.record(stream)
    for _ in range(args.steps):
        step()
    t_b.record(stream)
    torch.cuda.synchronize()
    ms_step = t_a.elapsed_time(t_b) / args.steps                     # whole timed region per step
    # The kernel window: K more calls right after, in the same settled state,
    # with events around each call's stages, for the partial kernel's own
    # duration and the per-call distribution.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    call_us = np.array([e[0].elapsed_time(e[2]) * 1e3 for e in evs])   # per call, partial + merge
    part_us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])   # per call, first stage
    ms_partial = float(part_us.mean()) * 1e-3
    if not bool(torch.isfinite(out.float()).all()):
        raise RuntimeError("non-finite output")

    def dist(x):
        return {"median": round(float(np.median(x)), 2), "p10": round(float(np.percentile(x, 10)), 2),
                "p90": round(float(np.percentile(x, 90)), 2), "mean": round(float(np.mean(x)), 2)}

    # Reference points on the same device.  (1) The streaming-read reference:
    # the same bytes as the KV cache, read once into LDS through the decode's
    # DMA path with no arithmetic (libmla_stream_ref.so).  (2) A plain
    # device-to-device copy (read + write) of 1 GiB.
    stream_ref = None
    kv_bytes_all = inp.kv_cache.numel() * inp.kv_cache.element_size()
    ref_lib = stream_reference_lib()
    if ref_lib is not None:
        nbytes = (kv_bytes_all // 36864) * 36864
        grid = 256
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        def ref_run():
            rc = ref_lib.mla_stream_read_reference(ctypes.c_void_p(inp.kv_cache.data_ptr()), nbytes, grid,
                                                   ctypes.c_void_p(sink.data_ptr()),
                                                   ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError("stream reference failed (%d)" % rc)
        for _ in range(3):
            ref_run()
        torch.cuda.synchronize()
        r_us = []
        for _ in range(10):
            r0 = torch.cuda.Event(enable_timing=True)
            r1 = torch.cuda.Event(enable_timing=True)
            r0.record(stream)
            ref_run()
            r1.record(stream)
            torch.cuda.synchronize()
            r_us.append(r0.elapsed_time(r1) * 1e3)
        r_med = float(np.median(r_us))
        stream_ref = {"GBps": round(nbytes / (r_med * 1e-6) / 1e9, 1), "us": round(r_med, 2), "bytes": nbytes,
                      "kind": "read once into LDS by buffer_load ... lds DMAs (36 KiB tiles, 4-tile ring, "
                              "256 workgroups of 4 waves), no arithmetic",
                      "frac_of_peak": round(nbytes / (r_med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst

    cost = algorithmic_cost(inp)
    kdt = "fp8" if fp8 else "bf16"
    t_hbm = cost["total_bytes"] / (HBM_PEAK_GBPS * 1e9)
    t_mfma = cost["flops"] / (MFMA_PEAK_TFLOPS[kdt] * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    part_bytes = cost["partial_bytes"] + (cost["out_bytes"] if S == 1 else 0)
    if bound == "hbm":
        achieved = part_bytes / (ms_partial * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4))
        if stream_ref is not None:
            roof["frac_of_stream_reference"] = round(achieved / stream_ref["GBps"], 4)
    else:
        achieved = cost["flops"] / (ms_partial * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=MFMA_PEAK_TFLOPS[kdt], unit="TFLOP/s",
                    frac=round(achieved / MFMA_PEAK_TFLOPS[kdt], 4))
    roof["kernel"] = "mla_partial_kernel"
    roof["us_per_launch"] = round(ms_partial * 1e3, 2)
    roof["us_per_launch_dist"] = dist(part_us)
    roof["timed"] = ("HIP events around each call's first-stage launch, over K calls issued right after the K timed "
                     "calls (the timed calls carry no events between their stages)")
    roof["traffic"] = load_traffic(args.workload)

    step_s = ms_step * 1e-3
    res = {
        "metric": "MLA decode us/call + achieved HBM TB/s & MFMA TFLOP/s as % of roofline",
        "value": round(ms_step * 1e3, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) values, shuffled pages)",
        "config": {"workload": args.workload, "batch": inp.B, "heads": inp.H, "q_len": inp.T,
                   "max_seq_len": inp.max_seq_len, "block_size": 64, "topk": inp.K, "kv_splits": S,
                   "out_dtype": inp.out_dtype, "launches": "one" if (single or S == 1) else "two"},
        "step": {"hbm_TBps": round(cost["total_bytes"] / step_s / 1e12, 3),
                 "mfma_TFLOPs": round(cost["flops"] / step_s / 1e12, 1),
                 "frac_hbm": round(cost["total_bytes"] / step_s / 1e12 / (HBM_PEAK_GBPS / 1e3), 4),
                 "frac_mfma": round(cost["flops"] / step_s / 1e12 / MFMA_PEAK_TFLOPS[kdt], 4),
                 "roofline_frac": round(max(t_hbm, t_mfma) / step_s, 4),
                 "algorithmic_bytes": cost["total_bytes"], "algorithmic_flops": cost["flops"]},
        "call_us": dict(dist(call_us), window="the K calls with events around their stages"),
        "clock_settle": {"ms": args.settle_ms, "calls": settle_calls},
        "roofline": roof,
        "stream_read_reference": stream_ref,
        "hbm_copy_reference": {"GBps": round(copy_gbps, 1), "kind": "torch copy_ of 1 GiB, read + write bytes",
                               "frac_of_peak": round(copy_gbps / HBM_PEAK_GBPS, 4)},
        "cpu_baseline": None,
        "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a row sample, ~%.0f s)" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
