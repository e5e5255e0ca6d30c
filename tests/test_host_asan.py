"""The library's host code under AddressSanitizer (CPU only).  api.cpp is compiled with ASan on
its host side (device code untouched) and linked with the library's other objects into
tests/host_asan/host_paths.cpp, which drives every host path of the C ABI that runs without a
GPU: descriptor validation, workspace and cache sizing, and the rejections the entry points make
before enqueueing anything.  The program must exit 0 with no sanitizer report."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "gated_softmax_attention_amd", "csrc")
INC = os.path.join(ROOT, "include")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_paths_under_address_sanitizer(tmp_path):
    from gated_softmax_attention_amd import build as hipbuild
    hipbuild.build(force=False, verbose=False)  # the kernels' objects (compiles only what is stale)
    others = [o for o in glob.glob(os.path.join(ROOT, "_build", "*.o")) if not o.endswith("api.cpp.o")]
    api = str(tmp_path / "api_asan.o")
    drv = str(tmp_path / "host_paths.o")
    exe = str(tmp_path / "host_paths")
    san = ["-Xarch_host", "-fsanitize=address", "-fno-omit-frame-pointer"]
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I", INC, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-c", os.path.join(CSRC, "api.cpp"),
          "-o", api])
    _run([HIPCC, "-x", "c++", "-O1", "-g", "-std=c++17", "-I", INC, *san, "-c",
          os.path.join(ROOT, "tests", "host_asan", "host_paths.cpp"), "-o", drv])
    _run([HIPCC, "--offload-arch=gfx950", *san, drv, api, *others, "-o", exe, "-Wl,-rpath,/opt/rocm/lib"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env={**os.environ, "ASAN_OPTIONS": "abort_on_error=0:halt_on_error=1"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr
    assert "all expectations hold" in r.stdout
