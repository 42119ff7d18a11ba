"""Build libmla_decode.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_decode.so")
SOURCES = [os.path.join(CSRC, "mla_decode_kernels.hip"), os.path.join(CSRC, "mla_decode_api.cpp"),
           os.path.join(CSRC, "mla_mha_kernels.hip"), os.path.join(CSRC, "mla_mha_api.cpp")]
# Benchmark-only: the streaming-read reference kernel (not part of the decode ABI).
STREAM_LIB = os.path.join(HERE, "libmla_stream_ref.so")
STREAM_SRC = os.path.join(CSRC, "stream_ref.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from forming v_pk_{add,mul,fma}_f32 on its own.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _device_asm_cmd(out: str, src: str):
    flags = [f for f in FLAGS if f not in ("-shared", "-Wall")]
    return [HIPCC] + flags + ["--offload-device-only", "-S", "-o", out, src]


def _build_one(lib: str, sources, scanned, verbose: bool) -> str:
    """Compile `sources` into `lib`; the device assembly of each file in
    `scanned` is checked for hazards before inline-asm memory instructions."""
    from mla_paged_latent_03_amd import asm_hazards

    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    found = []
    with tempfile.TemporaryDirectory() as td:
        asm_paths = [os.path.join(td, "kernels%d.s" % i) for i in range(len(scanned))]
        asm_procs = [subprocess.Popen(_device_asm_cmd(a, src), stdout=subprocess.DEVNULL, stderr=subprocess.PIPE,
                                      text=True) for a, src in zip(asm_paths, scanned)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        asm_errs = [pr.communicate()[1] for pr in asm_procs]
        noise = ("packed-fp32-ops", "unknown target feature")
        err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + err)
        for pr, e in zip(asm_procs, asm_errs):
            if pr.returncode != 0:
                raise RuntimeError("hipcc (device assembly) failed:\n" + e)
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        for a, src in zip(asm_paths, scanned):
            with open(a) as f:
                found += ["%s: %s" % (os.path.basename(src), x) for x in asm_hazards.scan(f.read())]
    if found:
        os.remove(tmp)
        raise RuntimeError("hazards before inline-asm memory instructions:\n" + "\n".join(found[:20]))
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the decode library and the benchmark's streaming-read
    reference, each with its kernels' gfx950 assembly alongside; fail if the
    assembly shows a hazard before an inline-asm memory instruction."""
    _build_one(STREAM_LIB, [STREAM_SRC], [STREAM_SRC], verbose)
    return _build_one(LIB, SOURCES, [f for f in SOURCES if f.endswith(".hip")], verbose)


if __name__ == "__main__":
    print(build(verbose=True))
