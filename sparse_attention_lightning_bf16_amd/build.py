"""Build liblix.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_attention_lightning_bf16_amd.build

Each translation unit is compiled by hipcc in parallel into _build/, then
linked into sparse_attention_lightning_bf16_amd/liblix.so.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblix.so")
SOURCES = ["api.cpp", "limits.cpp", "score.hip", "topk.hip", "fused.hip", "sparse.hip", "backward.hip"]
# Units whose MFMA accumulators may live in AGPRs (more than 256 registers of
# accumulators and operands at one wave per SIMD).
AGPR_SOURCES = {"backward.hip"}
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblix)")


def common_flags(src=""):
    flags = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             # keep packed fp32 VALU instructions out of the device code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if src not in AGPR_SOURCES:
        # MFMA accumulators in VGPRs: the epilogue reads them directly
        flags += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return flags + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-result"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for (_, warn), src in zip(results, SOURCES):
            if warn:
                print(f"[{src}]\n{warn}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
