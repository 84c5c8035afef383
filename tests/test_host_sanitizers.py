"""libpark's host code (argument validation, workspace sizing) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.  The C ABI source is compiled with both sanitizers on
its host code only (the device code is never sanitized), linked with the kernel sources and a
small C driver (tests/sanitize_driver.c) that calls every entry point with arguments each
host-side check must reject, and workspace sizes up to the library's maxima and beyond.  No
call reaches a GPU, so the test runs anywhere hipcc does."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_response_amd", "csrc")
KERNELS = ["park_noalloc.hip", "k_retrieve.hip", "k_attn.hip", "k_cluster.hip"]
ARCH = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        pytest.skip("hipcc not available")
    return p


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-4000:]}"


def test_host_code_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    objs = []
    jobs = []
    api = str(tmp_path / "park_api.o")
    jobs.append([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", *ARCH, *SAN, "-c",
                 os.path.join(CSRC, "park_api.hip"), "-o", api])
    objs.append(api)
    for src in KERNELS:
        o = str(tmp_path / (src + ".o"))
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src == "k_attn.hip" else []
        jobs.append([hipcc, "-O3", "-std=c++17", "-fPIC", *ARCH, *extra, "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    with ThreadPoolExecutor(4) as ex:
        list(ex.map(_run, jobs))
    # the driver is plain C, compiled by the host compiler on a line of its own
    gcc = shutil.which("gcc") or pytest.skip("gcc not available")
    drv = str(tmp_path / "sanitize_driver.o")
    _run([gcc, "-O1", "-g", "-std=c11", "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "sanitize_driver.c"), "-o", drv])
    exe = str(tmp_path / "sanitize_driver")
    _run([hipcc, "-O1", "-g", *ARCH, *SAN, drv, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "sanitized host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
