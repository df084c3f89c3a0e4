"""Build libefla.so (the HIP kernels and the C ABI of include/efla.h) in-tree.

hipcc compiles every translation unit for gfx950 in parallel and links one
shared library next to this file.  No GPU is needed to build.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libefla.so")
SOURCES = ["api.hip", "step_kernels.hip", "chunk_bf16.hip", "chunk_bf16_roles.hip", "chunk_bf16_split.hip",
           "chunk_bf16_states.hip", "ut_bf16.hip", "chunk_f32.hip", "bwd.hip", "bwd_bf16_chunk.hip", "seg.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    f"-I{os.path.join(ROOT, 'include')}",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source flags.  The one-role-per-wavefront recurrence and the UT transform
# keep their matrix-core accumulators in ordinary VGPRs, so results feed the
# bf16 conversions that follow every product without a copy out of the
# accumulation registers.
SOURCE_FLAGS = {"chunk_bf16_roles.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "chunk_bf16_split.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "chunk_bf16_states.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "ut_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "bwd_bf16_chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
    sys.exit(0)
