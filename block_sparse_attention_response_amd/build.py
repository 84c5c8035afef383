"""Build libpark.so (HIP, gfx950) in place, next to this file, and libpark_clocks.so: the same
library with the attention kernel's per-item clock stamps compiled in (PARK_ATTN_CLOCKS), for
measurement only."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpark.so")
CLOCKS_OUT = os.path.join(HERE, "libpark_clocks.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build", "libpark")
SOURCES = ["park_api.hip", "park_noalloc.hip", "k_retrieve.hip", "k_attn.hip", "k_cluster.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 instructions are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-Wall", "-Wno-unused-result"]
# per-source additions: the attention kernel keeps its MFMA accumulators in ordinary VGPRs, so
# the exponentials read the scores directly (the output accumulators fit beside them at one
# wave per SIMD)
EXTRA = {"k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libpark")
    return p


def _compile(job) -> str:
    src, defines, suffix = job
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libpark.so and libpark_clocks.so (always
    rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs_list = [(src, (), "") for src in SOURCES] + [("k_attn.hip", ("PARK_ATTN_CLOCKS",), "_clocks")]
    jobs = min(len(jobs_list), max(1, (os.cpu_count() or 4) // 2))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, jobs_list))
    plain = objs[:len(SOURCES)]
    _link(plain, OUT)
    clocked = [objs[-1] if src == "k_attn.hip" else o for src, o in zip(SOURCES, plain)]
    _link(clocked, CLOCKS_OUT)
    if verbose:
        print("built", OUT, "and", CLOCKS_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
