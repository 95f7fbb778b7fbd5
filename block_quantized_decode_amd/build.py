"""Build libqbd.so in-tree with hipcc for gfx950.

    python -m block_quantized_decode_amd.build

Every HIP source is compiled for gfx950 only, at -O3, with packed-FP32
instructions switched off and FP contraction off (each fused multiply-add in
the kernels is written out), then linked into one shared library next to
this file.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libqbd.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "qmv_f32.hip", "qmv_mfma.hip", "quant_act.hip", "qmm_q8act.hip", "qmm_mfma.hip",
           "swiglu.hip"]

# Matrix-core kernels keep MFMA results in VGPRs: their epilogue reads every
# result element on the VALU, which an AGPR result would tax with a copy.
EXTRA_FLAGS = {"qmm_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "qmv_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; ignore that line
    noise = [ln for ln in res.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
