"""Build the gfx950 HIP library in-tree: ``python -m block_scaled_fp4_e2m1_amd.build``.

Each source is compiled to an object under ``_build/`` in parallel, then linked into
``block_scaled_fp4_e2m1_amd/libfp4_e2m1.so``. Flags that matter for exactness:
  * IEEE float32 division (``-fhip-fp32-correctly-rounded-divide-sqrt``) and no denormal
    flushing: the scale computations divide once per block / group and the weights'
    FP16 macro-scales are often subnormal;
  * no fast-math;
  * packed float32 arithmetic is switched off in device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp4_e2m1.so")
SOURCES = ["api.cpp", "quant.hip", "repack.hip", "gemv.hip", "gemm.hip", "gemm_r8.hip", "moe.hip", "attention.hip",
           "mx.hip"]
ARCH = "gfx950"
# measurement probes (copy / read floor, MFMA and LDS rates): a separate library that the
# benchmark loads; nothing in the product path uses it
PROBE_SOURCES = ["probes.hip"]
PROBE_LIB = os.path.join(PKG, "libfp4_probes.so")
# per-source flags: the MFMA probe keeps its accumulators in ordinary VGPRs (with the
# accumulation registers the allocator shuffles its 16x16 accumulators every iteration)
SOURCE_FLAGS = {"probes.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *SOURCE_FLAGS.get(src, []), *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library (and the measurement
    probes' library); returns the library's path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
