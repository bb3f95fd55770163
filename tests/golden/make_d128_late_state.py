"""Writes d128_late_state.npz: the fp64 oracle's fast weights of two heads of the d = 128,
hidden = 512 long-context workload (AR(1) drifting inputs, B = 1, H = 24, T = 131072) after
the first 126976 tokens, rounded to fp32. A GPU test starts both the split kernel and the
oracle from this state (per-sequence W0) and compares the last 4096 tokens, where the weights
have grown over 7936 chunks. Calls only the oracle and the seeded input generator.

    python tests/golden/make_d128_late_state.py
"""
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import OracleConfig, scan  # noqa: E402
from test_weight_sequence_amd.synth import WORKLOADS, flatten_heads, make_inputs  # noqa: E402

HEADS = [5, 17]
T_START = 126976
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "d128_late_state.npz")


def main():
    torch.set_num_threads(os.cpu_count() or 1)
    w = WORKLOADS["ttt_mlp_bf16_d128_T128k"]
    inp = flatten_heads(make_inputs(w, batch_idx=[0], head_idx=HEADS, T=T_START))
    W = inp["W0"]
    cfg = OracleConfig(kind="mlp", chunk=w.chunk)
    t0 = time.time()
    step = 8192
    for s in range(0, T_START, step):
        sl = slice(s, s + step)
        _, W, _ = scan(inp["Q"][:, sl], inp["K"][:, sl], inp["V"][:, sl], inp["eta"][:, sl], W,
                       inp["gamma"], inp["beta"], cfg)
        print(f"  tokens {min(s + step, T_START)}/{T_START} ({time.time() - t0:.0f} s)", flush=True)
    np.savez(OUT, heads=np.array(HEADS), t_start=np.array(T_START),
             w1=W[0].to(torch.float32).numpy(), w2=W[1].to(torch.float32).numpy())
    print("wrote", OUT)


if __name__ == "__main__":
    main()
