"""Build libqbd.so in-tree with hipcc for gfx950.

    python -m block_quantized_decode_amd.build
    python -m block_quantized_decode_amd.build --resources OUT.md

Also builds libqbd_ceiling.so, the streaming-read reference kernel that the
benchmark measures the memory roofline against (include/qbd_ceiling.h).
Every HIP source is compiled for gfx950 only, at -O3, with packed-FP32
instructions switched off and FP contraction off (each fused multiply-add in
the kernels is written out), then linked into one shared library next to
this file.  --resources also compiles every source with the compiler's
kernel-resource-usage remarks and writes the table of registers, scratch,
static LDS and occupancy of every kernel instantiation.
"""

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libqbd.so")
# the streaming-read reference of the memory roofline, a library of its own
CEILING_LIB = os.path.join(HERE, "libqbd_ceiling.so")
CEILING_SOURCES = ["read_ceiling.hip", "handoff_ceiling.hip"]
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "qmv_f32.hip", "qmv_mfma.hip", "quant_act.hip", "qmm_q8act.hip", "qmm_mfma.hip",
           "qmm_tile16.hip", "swiglu.hip"]

# Matrix-core kernels keep MFMA results in VGPRs: their epilogue reads every
# result element on the VALU, which an AGPR result would tax with a copy.
EXTRA_FLAGS = {"qmm_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "qmv_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "qmm_tile16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

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


def _compile(src, out_dir=None, extra=()):
    obj = os.path.join(out_dir or BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), *extra, "-I", INCLUDE, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; ignore that line
    noise = [ln for ln in res.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
    if extra:
        return res.stderr
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


_REMARK = re.compile(r"^(\S+\.hip):\d+:\d+: remark:\s+(.*?): (.*?) \[-Rpass-analysis")
_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
           "LDS Size [bytes/block]": "lds", "Occupancy [waves/SIMD]": "occupancy"}


def resource_usage():
    """Per kernel instantiation: VGPRs, AGPRs, SGPRs, scratch bytes per lane,
    static LDS bytes and occupancy, from hipcc's kernel-resource-usage
    remarks (a fresh compile of every HIP source)."""
    rows = []
    with tempfile.TemporaryDirectory() as tmp:
        srcs = [s for s in SOURCES + CEILING_SOURCES if s.endswith(".hip")]
        with concurrent.futures.ThreadPoolExecutor(min(len(srcs), 4)) as ex:
            logs = list(ex.map(lambda src: _compile(src, tmp, ("-Rpass-analysis=kernel-resource-usage",)), srcs))
    for src, log in zip(srcs, logs):
        cur = None
        for ln in log.splitlines():
            m = _REMARK.match(ln)
            if not m:
                continue
            key, val = m.group(2).strip(), m.group(3).strip()
            if key == "Function Name":
                cur = {"source": src, "mangled": val}
                rows.append(cur)
            elif cur is not None and key in _FIELDS:
                cur[_FIELDS[key]] = int(val)
    names = subprocess.run(["c++filt"], input="\n".join(r["mangled"] for r in rows), capture_output=True,
                           text=True).stdout.splitlines() if shutil.which("c++filt") else []
    for r, n in zip(rows, names):
        r["kernel"] = n.replace("qbd::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return rows


def _short_name(demangled):
    """'void k<(qbd::Fmt)1, (qbd::Mode)0, 8>(args)' -> 'k<Q4, Plain, 8>'."""
    n = demangled
    if n.endswith(")"):  # drop the parameter list: the last balanced (...)
        depth = 0
        for i in range(len(n) - 1, -1, -1):
            depth += n[i] == ")"
            depth -= n[i] == "("
            if depth == 0:
                n = n[:i]
                break
    n = n[5:] if n.startswith("void ") else n
    for a, b in (("(qbd::Fmt)0", "Q8_0"), ("(qbd::Fmt)1", "Q4"), ("(qbd::Mode)0", "Plain"),
                 ("(qbd::Mode)1", "SwiGLU"), ("qbd::", "")):
        n = n.replace(a, b)
    return n


def write_resource_table(path):
    rows = resource_usage()
    lines = ["# Kernel resources (gfx950)", "",
             "Every kernel instantiation in libqbd.so, from hipcc's kernel-resource-usage remarks.",
             "Command: `python -m block_quantized_decode_amd.build --resources " + os.path.relpath(path, os.path.dirname(HERE)) + "`.",
             "LDS is the static allocation; kernels that size their LDS at launch show 0 here.",
             "Occupancy is the compiler's waves per SIMD from registers alone.", "",
             "| source | kernel | VGPRs | AGPRs | SGPRs | scratch B/lane | static LDS B | waves/SIMD |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        name = _short_name(r.get("kernel", r["mangled"]))
        lines.append(f"| {r['source']} | `{name}` | {r.get('vgpr', '')} | {r.get('agpr', '')} | {r.get('sgpr', '')} | "
                     f"{r.get('scratch', '')} | {r.get('lds', '')} | {r.get('occupancy', '')} |")
    spills = [r for r in rows if r.get("scratch", 0)]
    lines += ["", f"{len(rows)} instantiations; {len(spills)} use scratch."]
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rows


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)


def build(verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    jobs = min(len(srcs), max(1, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--resources":
        write_resource_table(sys.argv[2])
    else:
        build()
