"""Build libradixrt.so (host radix tree + gfx950 kernels) in this package
directory with hipcc.  Used by ``__graft_entry__.build()``; also runnable as
``python -m prefix_shared_kv_rt_amd.build``."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libradixrt.so")
BUILD_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
# Device code: no packed-fp32 instructions (compiler-generated v_pk_* fp32
# forms are kept out of every kernel); MFMA accumulators stay in VGPRs so the
# online-softmax rescale never copies them out of AGPRs.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip")))


def _compile(src):
    obj = os.path.join(BUILD_DIR, src + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = ["hipcc", *COMMON, *DEVICE, "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = ["hipcc", *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
