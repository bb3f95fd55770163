"""Build libttt.so (the gfx950 HIP kernels and the C-ABI host layer) in-tree.

    python -m test_weight_sequence_amd.build [--poison]

Compiles every translation unit under csrc/ with hipcc for gfx950 and links them
into test_weight_sequence_amd/libttt.so (with --poison, also the LDS-poisoning test
build libttt_poison.so). Packed fp32 instructions are disabled for
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
# Test build with every kernel's LDS filled with NaN bit patterns at entry (TTT_LDS_POISON);
# tests/test_lds_poison_gpu.py runs parity cases on it. Never loaded by the product path.
LIB_POISON = os.path.join(PKG, "libttt_poison.so")
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
# The machine scheduler's iterative ILP strategy for the chunk-scan kernels: their time is a
# chain of dependent phases per chunk, and this strategy orders each phase for latency rather
# than register pressure. Interleaved A/Bs of the two builds on one MI355X (kernel ms by
# hipEvents, same outputs to the parity tolerances): paired d=64 1.046 -> 1.020, key output
# 0.996 -> 0.959, one workgroup per head at B=16 1.608 -> 1.580, momentum 2.487 -> 2.455,
# backward 5.244 -> 5.190, split d=128 39.53 -> 37.52, large-chunk layer 0.450 -> 0.445. The
# decode kernel measured no better (11.2 vs 11.3 us) and keeps the default.
ITER_ILP = {"ttt_fwd_mfma_pair.hip", "ttt_fwd_mfma.hip", "ttt_fwd_mfma_mom.hip",
            "ttt_fwd_mfma_split.hip", "ttt_bwd_mfma_split.hip", "ttt_lact.hip"}
ITER_ILP_FLAGS = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]


def source_flags(name: str) -> list:
    """Compiler flags of the product build of csrc/<name> beyond COMMON."""
    return (([] if name in NO_VGPR_FORM else VGPR_FORM) +
            (ITER_ILP_FLAGS if name in ITER_ILP else []))


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    flags = COMMON + list(extra) + source_flags(os.path.basename(src))
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


def build_poison(verbose: bool = True) -> str:
    """The LDS-poisoning test build of the same sources (libttt_poison.so)."""
    return build(verbose, lib=LIB_POISON, build_dir=os.path.join(BUILD, "poison"), extra=("-DTTT_LDS_POISON",))


if __name__ == "__main__":
    build()
    if "--poison" in sys.argv[1:]:
        build_poison()
    sys.exit(0)
