"""Build libspa.so (the HIP library behind include/spa.h) for gfx950, in-tree.

Usage: python -m sparse_paged_attention_amd.build   (or build() from Python)
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspa.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["spa_api.cpp", "spa_attention.hip", "spa_pair.hip", "spa_decode.hip", "spa_decode_rows.hip", "spa_merge.hip", "spa_gather.hip", "spa_topk.hip",
           "spa_backward.hip", "spa_latent.hip"]
ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for every HIP source file.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # keep MFMA accumulators in VGPRs: with AGPR accumulators the
                # compiler copies the whole O tile between the register files
                # on every KV tile
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
# The attention kernel's softmax never produces a NaN from valid inputs; without
# NaN semantics the compiler drops the quieting copies it otherwise puts in
# front of every float max.  (A NaN read from the caches still propagates
# through the MFMAs and the exponentials into O.)
SOURCE_FLAGS = {"spa_attention.hip": ["-fno-honor-nans"], "spa_pair.hip": ["-fno-honor-nans"],
                "spa_decode.hip": ["-fno-honor-nans"],
                "spa_latent.hip": ["-fno-honor-nans"],
                "spa_decode_rows.hip": ["-fno-honor-nans"]}
# The backward keeps its MFMA accumulators in AGPRs: the KV-block kernel's
# dK and dV sums (128 registers) leave the VGPRs free for its LDS operands.
AGPR_ACC = {"spa_backward.hip"}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"]


def device_flags(src: str) -> list:
    """DEVICE_FLAGS, without the VGPR accumulator form for AGPR_ACC files."""
    if src not in AGPR_ACC:
        return list(DEVICE_FLAGS)
    f = list(DEVICE_FLAGS)
    i = f.index("-amdgpu-mfma-vgpr-form")
    del f[i - 1:i + 1]
    return f


def _hipcc():
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found")
    return cand


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + COMMON + device_flags(src) + SOURCE_FLAGS.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return obj, out


def build(verbose: bool = False) -> str:
    """Compile every source and link libspa.so; always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, out in results:
        if verbose and out.strip():
            print(out)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
