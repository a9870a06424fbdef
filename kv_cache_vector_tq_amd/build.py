"""Builds libtq.so (HIP kernels for gfx950 + the C ABI) in-tree.

Usage: python -m kv_cache_vector_tq_amd.build   (or build() from Python)
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libtq.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    # packed FP32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
SOURCES = ["tables.cpp", "tq_api.cpp", "encode.hip", "encode_mma.hip", "decode.hip", "decode_mfma.hip", "dequant.hip", "probe.hip"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# matrix-core accumulators stay in ordinary VGPRs (no AGPR round trips in the scan loop)
EXTRA = {"decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "encode_mma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, obj):
    cmd = [_hipcc()] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stderr


def build(verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    objdir = os.path.join(OUT_DIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        futs = [ex.submit(_compile, s, o) for s, o in zip(SOURCES, objs)]
        for f in futs:
            msg = f.result()
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
