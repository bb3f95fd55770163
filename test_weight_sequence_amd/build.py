"""Build libttt.so (the gfx950 HIP kernels and the C-ABI host layer) in-tree.

    python -m test_weight_sequence_amd.build

Compiles every translation unit under csrc/ with hipcc for gfx950 and links them
into test_weight_sequence_amd/libttt.so. Packed fp32 instructions are disabled for
the device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libttt.so")
BUILD = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]
# MFMA operands and results in ordinary VGPRs (fewer AGPR<->VGPR copies in the forward
# kernels). Not for the backward kernel: it uses more than the 256 VGPRs a wave has, and
# with this option the compiler crashes in its AGPR-copy rewrite pass on that kernel.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"ttt_bwd_mfma.hip"}


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    flags = COMMON + list(extra) + ([] if os.path.basename(src) in NO_VGPR_FORM else VGPR_FORM)
    cmd = [HIPCC, *flags, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *flags, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, lib: str = LIB, build_dir: str = BUILD, extra=()) -> str:
    """Compile every source under csrc/ (with the extra compiler flags) and link `lib`."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
