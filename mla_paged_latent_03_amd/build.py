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


def _build_one(lib: str, sources, scanned: str, verbose: bool) -> str:
    from mla_paged_latent_03_amd import asm_hazards

    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    with tempfile.TemporaryDirectory() as td:
        asm_path = os.path.join(td, "kernels.s")
        asm_proc = subprocess.Popen(_device_asm_cmd(asm_path, scanned), stdout=subprocess.DEVNULL,
                                    stderr=subprocess.PIPE, text=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        asm_err = asm_proc.communicate()[1]
        noise = ("packed-fp32-ops", "unknown target feature")
        err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + err)
        if asm_proc.returncode != 0:
            raise RuntimeError("hipcc (device assembly) failed:\n" + asm_err)
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        with open(asm_path) as f:
            found = asm_hazards.scan(f.read())
    if found:
        os.remove(tmp)
        raise RuntimeError("hazards before inline-asm memory instructions:\n" + "\n".join(found[:20]))
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the decode library and the benchmark's streaming-read
    reference, each with its kernels' gfx950 assembly alongside; fail if the
    assembly shows a hazard before an inline-asm memory instruction."""
    _build_one(STREAM_LIB, [STREAM_SRC], STREAM_SRC, verbose)
    return _build_one(LIB, SOURCES, SOURCES[0], verbose)


if __name__ == "__main__":
    print(build(verbose=True))
