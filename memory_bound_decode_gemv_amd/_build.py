"""Build libdecodegemv.so in-tree with hipcc for gfx950.

Every HIP source under csrc/ is compiled to an object (in parallel), then the
objects are linked into memory_bound_decode_gemv_amd/libdecodegemv.so.  The
packed-FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdecodegemv.so")
ARCH = "gfx950"


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


# Per-source flags.  The matrix-core kernels keep MFMA results in VGPRs (gfx950
# allows it) instead of AGPRs that every result would have to be copied out of.
EXTRA_FLAGS = {"gemv_q4_0_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "gemv_qmfma_res.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "gemv_tiles.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every csrc/*.hip and link libdecodegemv.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def device_asm(src: str, out: str) -> str:
    """gfx950 assembly of one source (device side only), for the assembly audit."""
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(os.path.basename(src), []), "--cuda-device-only", "-S",
           src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build())
