"""Build libkvattn.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m kv_cache_decode_attn_amd.build

Compiles every csrc/*.hip and csrc/*.cpp with hipcc for gfx950 and links
kv_cache_decode_attn_amd/libkvattn.so.  Always rebuilds.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvattn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file extra flags for the MFMA prefill kernel:
#  - it takes maxima of raw matrix results; without NaN-preserving semantics
#    the compiler drops one quieting instruction per score.  NaN can only
#    reach that kernel through padding query rows (whose outputs are written
#    as zeros) and masked keys (whose scores are replaced by -inf before any
#    maximum), so no result changes;
#  - its matrix results live in vector registers (the scores are read by the
#    softmax right away); with no accumulation registers in use the compiler
#    can give each of the two waves per SIMD all 256 registers, and the
#    allocation has no copies between the two register files.
# decode.hip: matrix results in vector registers too.  Its passes hold the
# output accumulator in registers across the whole sweep; without
# accumulation registers the 16-column pass fits three waves per SIMD
# instead of two (150 registers in one file against 148 + 40 in two).
EXTRA = {"prefill_mfma.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
         "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    return obj, msgs


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    objs = []
    with cf.ThreadPoolExecutor(jobs) as ex:
        for obj, msgs in ex.map(_compile, srcs):
            objs.append(obj)
            if verbose and msgs:
                print("\n".join(msgs), file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
