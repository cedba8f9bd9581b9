"""Builds libqmm.so in place with hipcc for gfx950.

Each HIP source is compiled in its own process (in parallel), then linked
into one shared library next to this file.  Flags: -O3, no fast-math, f32
denormals kept (the E8M0 scale 2^-127 is subnormal), no packed-f32
instructions, hidden visibility except for the C ABI.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libqmm.so")
# The streaming-read probe that measurements compare against (its own
# library; not part of the matmul C ABI).
PROBE_SOURCE = os.path.join(CSRC, "probe", "qmm_stream_read.hip")
PROBE_LIBRARY = os.path.join(HERE, "libqmm_probe.so")
OBJDIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


# Per-source extra flags.  The GEMM keeps its matrix-core accumulators in
# ordinary VGPRs: with accumulation registers the allocator rotates its
# loop-carried accumulators through copies on every iteration.  (The GEMV
# mixes inline assembly with its matrix-core code and keeps the default.)
FILE_FLAGS = {"qmm_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()

    def one(src: str) -> str:
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        cmd = [cc, *compile_flags(), *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, sources()))
    tmp = LIBRARY + ".tmp"
    r = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    build_probe(cc)
    return LIBRARY


def build_probe(cc: str) -> str:
    tmp = PROBE_LIBRARY + ".tmp"
    r = subprocess.run([cc, *compile_flags(), "-shared", PROBE_SOURCE, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SOURCE}:\n{r.stderr}")
    os.replace(tmp, PROBE_LIBRARY)
    return PROBE_LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
