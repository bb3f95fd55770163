"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Builds the library with the host part of every translation unit instrumented (hipcc
-Xarch_host -fsanitize=...; device code is compiled as usual and never launched here) into
_build/asan/, links a C driver (tests/sanitize/abi_host_checks.c) with the same sanitizers and
runs it: every call in the driver is rejected by host validation before anything is enqueued.
The test fails on any sanitizer report or unexpected return code."""
import hashlib
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "test_weight_sequence_amd", "csrc")
OUT = os.path.join(ROOT, "test_weight_sequence_amd", "_build", "asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"  # the sanitizer runtime hipcc's host compiler instruments for
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _build_lib() -> str:
    os.makedirs(OUT, exist_ok=True)
    h = hashlib.sha256()
    for f in _sources() + glob.glob(os.path.join(CSRC, "*.h*")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    lib = os.path.join(OUT, f"libttt_asan_{h.hexdigest()[:12]}.so")
    if os.path.exists(lib):
        return lib
    objs = []
    for src in _sources():
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        x = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "-Xclang",
               "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, *x, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return lib


@pytest.mark.timeout(900)
def test_abi_host_paths_under_asan_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    lib = _build_lib()
    exe = os.path.join(OUT, "abi_host_checks")
    drv = os.path.join(ROOT, "tests", "sanitize", "abi_host_checks.c")
    rt = os.path.dirname(subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                        capture_output=True, text=True).stdout.strip())
    cmd = [CLANG, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-shared-libsan", "-o", exe, drv, lib, f"-Wl,-rpath,{os.path.dirname(lib)}",
           f"-Wl,-rpath,{rt}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "all host ABI checks passed" in out
