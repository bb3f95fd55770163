"""Per-phase clock counts of the paired d = 64 scan kernel (a timing build, not the product).

    python -m test_weight_sequence_amd.phase_clocks build   # on a machine with hipcc
    python -m test_weight_sequence_amd.phase_clocks run     # on the GPU: prints a markdown table

`build` compiles the library with TTT_PHASE_CLOCKS into _build/phase/libttt_phase.so (the
product library libttt.so is untouched). That build stamps the shader clock (s_memtime, with a
wait for the stamp) at the phase boundaries of every 16-token chunk of head 0 and sums each
phase per wave over chunks 16 .. T/16 - 1. `run` times the B=8 H=12 T=8192 d=64 workload with
it and prints the mean clocks per chunk of each phase, for the producer workgroup (the K side
that carries the weights) and the consumer (the Q side). The stamps' own waits add to the
phases, so the sum is a little above the plain kernel's time per chunk.
"""
from __future__ import annotations

import ctypes
import os
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
BUILD_DIR = os.path.join(PKG, "_build", "phase")
LIB = os.path.join(BUILD_DIR, "libttt_phase.so")

PRODUCER = ["start -> GELU/GELU' done", "-> Z^K partial in LDS (look-ahead, conversions)",
            "-> before barrier 1 (W2^T, LN inputs, publish)", "barrier 1",
            "LayerNorm fwd/bwd (waves 0-3), W2^T + staging (waves 4-7)", "barrier 2",
            "E1n = (En2 W2^T) * GELU'", "hand-off stores"]
CONSUMER = ["start -> GELU(H^Q) done", "-> Z^Q partial in LDS", "weight update replay",
            "slot wait + load + staging", "barrier", "output LayerNorm (waves 0-3)"]


def build():
    from test_weight_sequence_amd import build as b
    b.build(lib=LIB, build_dir=BUILD_DIR, extra=("-DTTT_PHASE_CLOCKS",))


def run():
    import torch
    from test_weight_sequence_amd import ops
    from test_weight_sequence_amd.synth import WORKLOADS, make_inputs
    ops._LIB_PATH = LIB
    ops._lib = None
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    d = {k: (tuple(x.to(dev) for x in v) if isinstance(v, tuple) else v.to(dev)) for k, v in inp.items()}
    cfg = ops.Config(kind="mlp", B=w.B, H=w.H, T=w.T, d=w.d, hidden=w.hidden, chunk=w.chunk, io=w.io)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_pair_d64"
    times = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = ops.scan_fwd(cfg, d["Q"], d["K"], d["V"], d["eta"], d["W0"], d["gamma"], d["beta"])
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) * 1e3)
        assert ops.read_status(res["workspace"]) == 0
    L = ctypes.CDLL(LIB)
    buf = (ctypes.c_ulonglong * (2 * 8 * 16))()
    assert L.ttt_phase_clocks_read(buf) == 0
    print(f"stamped launches: {', '.join(f'{t:.3f}' for t in times)} ms (wall, incl. launch)")
    for side, names in ((0, PRODUCER), (1, CONSUMER)):
        print(f"\n{'producer' if side == 0 else 'consumer'} workgroup, clocks per chunk (mean over chunks 16..)")
        print("| wave | " + " | ".join(names) + " | span/chunk |")
        print("|---" * (len(names) + 2) + "|")
        for wv in range(8):
            a = [buf[(side * 8 + wv) * 16 + k] for k in range(16)]
            n = max(a[8], 1)
            row = [f"{a[k] / n:.0f}" for k in range(len(names))]
            print(f"| {wv} | " + " | ".join(row) + f" | {(a[9] - a[10]) / n:.0f} |")


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "build":
        build()
    else:
        sys.path.insert(0, os.path.dirname(PKG))
        run()
