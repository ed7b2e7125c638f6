"""Build libmoe.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m sparse_expert_execution_amd.build

Every source is compiled for gfx950 only.  Packed-FP32 instruction
selection is turned off for device code.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
OBJ = os.path.join(ROOT, "_build", "obj")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "host.cpp", "host_expert.cpp", "planner.cpp", "cache.cpp", "stream.cpp", "route.hip",
           "decode.hip", "decode_bf16.hip", "decode_mxfp4.hip", "decode_nvfp4.hip", "prefill.hip",
           "prefill_nvfp4.hip", "formats.hip", "noalloc.hip"]

FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


def _compile(src):
    obj = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that line is noise
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    # librocprofiler-sdk-roctx: the roctx ranges around the C-ABI calls
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs + [
        "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
