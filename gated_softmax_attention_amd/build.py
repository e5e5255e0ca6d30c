"""Compile the HIP sources into gated_softmax_attention_amd/libfixattn.so (gfx950).

Every translation unit is compiled with hipcc in parallel into _build/, then
linked into a shared library next to this file.  Usage:
    python -m gated_softmax_attention_amd.build [--force]
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfixattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I", INCLUDE, "-I", CSRC,
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Backward kernels: MFMA results in the VGPR form.  These kernels run one wave
# per SIMD with their dk/dv accumulators in AGPRs; with the compiler's default
# choice every product then writes AGPRs, and the score and dP tiles (read by
# vector code right after) displace accumulators into VGPRs and back on every
# step.  In the VGPR form the allocator places each product's result where its
# readers want it.
EXTRA_FLAGS = {"bwd_d": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def flags_for(src: str) -> list:
    name = os.path.basename(src)
    return [f for key, fl in EXTRA_FLAGS.items() if name.startswith(key) for f in fl]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp")]


def _headers_mtime() -> float:
    hs = glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(INCLUDE, "fixattn.h")]
    return max(os.path.getmtime(h) for h in hs)


def _compile(src: str, force: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if not force and os.path.exists(obj):
        if os.path.getmtime(obj) >= max(os.path.getmtime(src), _headers_mtime()):
            return obj
    cmd = [HIPCC, "-x", "hip", *COMMON_FLAGS, *flags_for(src), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(force: bool = True, jobs: int | None = None, verbose: bool = True) -> str:
    """Compile (all sources when force, else only stale ones) and link libfixattn.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    # largest translation units first
    srcs.sort(key=lambda p: -os.path.getsize(p) - (1 << 20) * ("fwd_d" in p or "bwd_d" in p))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp,
           "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probe(verbose=verbose)
    return LIB


PROBE_SRC = os.path.join(HERE, "probe", "peak_probe.hip")
PROBE_LIB = os.path.join(HERE, "libfixprobe.so")


def build_probe(verbose: bool = True) -> str:
    """The peak-probe library (matrix-product, exponential and copy loops) that
    `bench.py --peak-probe` times; separate from the attention library."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, "-x", "hip", *COMMON_FLAGS, "-shared", PROBE_SRC, "-o", tmp, "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(force="--force" in sys.argv)
