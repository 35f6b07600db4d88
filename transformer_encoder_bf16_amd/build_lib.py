"""Builds liblaya_encoder.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Run as ``python -m transformer_encoder_bf16_amd.build_lib``; the library is
written next to this file, in-tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblaya_encoder.so")
PROBE = os.path.join(HERE, "chip_probe")
# diagnostic build: the same library with the GEMMs' per-workgroup phase
# timestamps compiled in (bench.py --gemm-phases); never loaded by the pass
PHASES_LIB = os.path.join(HERE, "liblaya_encoder_phases.so")

SOURCES = ["k_elementwise.hip", "k_gemm.hip", "k_attention.hip", "engine.cpp", "queue.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed float32 instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file additions.  Attention: MFMA accumulators in ordinary VGPRs
# (gfx950 allows it), so the softmax works on them with no copies between
# accumulation and arithmetic registers; and since the kernel never lets a
# NaN into its float arithmetic (masked scores are replaced by -inf with a
# select, values past a row's end are zeroed as bits), its maxima need no NaN
# quieting.  The GEMMs keep their accumulators in AGPRs: the large tiles need
# more than the 256 ordinary VGPRs.
FILE_FLAGS = {"k_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]}


def _compile(src: str, extra: tuple = (), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    if not os.path.exists(HIPCC) and shutil.which(HIPCC) is None:
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        phases = ex.submit(_compile, "k_gemm.hip", ("-DLAYA_GEMM_PHASES",), "_phases")
        objs = list(ex.map(_compile, SOURCES))
        phases_obj = phases.result()
    for lib, lib_objs in ((LIB, objs), (PHASES_LIB, [phases_obj if o.endswith("k_gemm.o") else o
                                                      for o in objs])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    # the chip probe (bench.py --chip-peaks): a program of its own
    tmp = PROBE + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, os.path.join(CSRC, "chip_probe.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for chip_probe.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
