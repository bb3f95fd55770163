"""Benchmark: TTT-MLP forward scan throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: TTT-MLP scan, B=8, H=12, T=8192, d=64, hidden=256, chunk 16, bf16 Q/K/V/Z,
fp32 fast weights (synthetic, seeded inputs resident in HBM before timing starts).
A step is one ttt_scan_fwd call over the whole batch. Prints one JSON line with
token*heads/s, the dominant kernel's achieved fraction of the MI355X dense bf16 MFMA
peak (algorithmic FLOPs / measured kernel time), and the CPU oracle's rate on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3


def flops_per_token_head(d: int, h: int, b: int) -> int:
    # seven d*h-sized products (2 FLOP per MAC) + the four b-sized dual-form products
    return 14 * d * h + 4 * b * (d + h)


def key_flops_per_token_head(d: int, h: int) -> int:
    # the key-side output rule (z_t = f(K_t; W at the chunk start)): the two query-side
    # products and the four dual-form products drop out, five d*h-sized products remain
    return 10 * d * h


def bytes_per_token_head(d: int, io_bytes: int, nW: int, T: int) -> float:
    # Q, K, V in, Z out (io dtype), eta (fp32), W0 read + W_T written, amortised over T
    return 4 * d * io_bytes + 4 + 2 * nW * 4 / T


KERNEL_SOURCES = {
    "ttt_fwd_mfma_pair_d64": ("ttt_fwd_mfma_pair.hip", "ttt_mfma_common.hpp", "ttt_device.hpp", "ttt_gelu.hpp"),
    "ttt_fwd_mfma_key_d64": ("ttt_fwd_mfma_pair.hip", "ttt_mfma_common.hpp", "ttt_device.hpp", "ttt_gelu.hpp"),
    "ttt_fwd_mfma_d64": ("ttt_fwd_mfma.hip", "ttt_mfma_common.hpp", "ttt_device.hpp", "ttt_gelu.hpp"),
    "ttt_fwd_generic": ("ttt_fwd_generic.hip",),
    "ttt_decode_stream_d64": ("ttt_decode_stream.hip", "ttt_device.hpp", "ttt_gelu.hpp"),
    "ttt_decode_split_d64": ("ttt_decode_split.hip", "ttt_device.hpp", "ttt_gelu.hpp"),
    "ttt_fwd_mfma_split_d128": ("ttt_fwd_mfma_split.hip", "ttt_mfma_common.hpp", "ttt_device.hpp",
                                "ttt_gelu.hpp"),
    "ttt_bwd_mfma_d64": ("ttt_bwd_mfma.hip", "ttt_mfma_common.hpp", "ttt_device.hpp", "ttt_gelu.hpp"),
    "ttt_bwd_mfma_split_d64": ("ttt_bwd_mfma_split.hip", "ttt_mfma_common.hpp", "ttt_device.hpp",
                               "ttt_gelu.hpp"),
    "ttt_lact_fwd_d64": ("ttt_lact.hip", "ttt_mfma_common.hpp", "ttt_device.hpp", "ttt_gelu.hpp"),
    "ttt_fwd_mfma_mom_d64": ("ttt_fwd_mfma_mom.hip", "ttt_mfma_common.hpp", "ttt_device.hpp", "ttt_gelu.hpp"),
}


def _source_hash(kernel: str) -> str:
    """Hash of the kernel's product source and of the scheduler flags it is built with beyond
    the common ones. Lines of the LDS-poisoning test instrumentation (those naming TTT_POISON)
    compile to nothing in the product library and are left out."""
    from test_weight_sequence_amd.build import ITER_ILP, ITER_ILP_FLAGS
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "test_weight_sequence_amd", "csrc", name), "rb") as fh:
            h.update(b"".join(l for l in fh.read().splitlines(keepends=True) if b"TTT_POISON" not in l))
    if KERNEL_SOURCES[kernel][0] in ITER_ILP:
        h.update(" ".join(ITER_ILP_FLAGS).encode())
    return h.hexdigest()[:16]


def _traffic(kernel: str, n_launch_units: int, variant: str = ""):
    """HBM bytes per launch from the committed rocprofv3 counter summary (of the launch
    variant named by `variant`, e.g. "_b256"), if it was taken on the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}{variant}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256_16") != _source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "" where it cannot be read."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(w, n_seq: int, T: int, n_heads: int | None = None, grads: bool = False,
                 output: str = "query") -> dict:
    """The fp64 oracle on the first n_seq sequences (the first n_heads heads of each, default
    all), first T tokens; with grads, the oracle's outer-loop gradients (autograd through
    its primal scan) instead of the forward; `output` picks the output rule."""
    import torch
    from oracle import OracleConfig, scan, scan_outer_grads
    from test_weight_sequence_amd.synth import flatten_heads, make_inputs
    torch.set_num_threads(max(1, torch.get_num_threads()))
    cores = torch.get_num_threads()
    nh = w.H if n_heads is None else n_heads
    inp = flatten_heads(make_inputs(w, batch_idx=list(range(n_seq)), head_idx=list(range(nh)),
                                    T=T, with_dz=grads))
    pairs = n_seq * nh
    cfg = OracleConfig(kind=w.kind, chunk=w.chunk, output=output)
    t0 = time.perf_counter()
    if grads:
        scan_outer_grads(inp["Q"], inp["K"], inp["V"], inp["eta"], inp["W0"], inp["gamma"],
                         inp["beta"], cfg, inp["dZ"].double())
    else:
        scan(inp["Q"], inp["K"], inp["V"], inp["eta"], inp["W0"], inp["gamma"], inp["beta"], cfg)
    dt = time.perf_counter() - t0
    what = "outer-loop gradients (autograd through the primal scan)" if grads else "forward scan"
    if output != "query":
        what += f" ({output}-side output rule)"
    return {"value": pairs * T / dt, "unit": "token*heads/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"fp64 oracle {what} on sequences 0..{n_seq - 1} x heads 0..{nh - 1} "
                      f"({pairs} (batch, head) pairs) x first T={T} tokens of the same workload "
                      f"({dt:.1f} s wall, torch intra-op threads={cores})"}


def _time_calls(call, steps: int, warmup: int, calls_per_step: int = 1):
    """Run `warmup` untimed steps, then `steps` timed steps of `calls_per_step` library calls
    each. Every call is bracketed by hipEvents on the launch stream (torch's current stream,
    which is the stream handed to the library). Returns (wall ms per step, per-call ms list)."""
    import torch
    from test_weight_sequence_amd import ops
    for i in range(warmup * calls_per_step):
        rc = call(i % calls_per_step)
        if rc != 0:
            raise ops.TTTError(rc, "warm-up call")
    torch.cuda.synchronize()
    n = steps * calls_per_step
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        starts[i].record()
        call(i % calls_per_step)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, [s.elapsed_time(e) for s, e in zip(starts, ends)]


DATA = "synthetic (seeded N(0,1/d) Q/K/V, N(0,0.02^2) W0, eta=0.1*sigmoid(N(0,1)))"

# The source pages' own figures near this path, restated (other hardware, models and
# precisions; none is this metric, so vs_baseline stays null).
CONTEXT_SCAN = ("pages, for context only: earlier TTT implementations were reported below 5% of "
                "peak FLOPS on recent GPUs; TTT-E2E prefill was 2.7x faster than full attention at "
                "128K tokens on one H100 and its training 3.4x slower at 8K on H200")
CONTEXT_LACT = ("pages, for context only: the large-chunk layer was reported at up to 70% of peak "
                "on A100 with chunks of 2K to 1M tokens")


def _base_record(args, metric, value, ms_step, w, kernel, dtype, extra_cfg=None):
    cfg = {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "hidden": w.hidden,
           "chunk": w.chunk, "io": w.io, "state": "fp32", "kernel": kernel}
    cfg.update(extra_cfg or {})
    return {"metric": metric, "value": value, "unit": "token*heads/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": DATA + (" (AR(1) drift 0.999 along tokens)" if w.drift > 0 else ""),
            "config": cfg}


def _device_inputs(w, dev, with_dz=False):
    from test_weight_sequence_amd.synth import make_inputs
    inp = make_inputs(w, with_dz=with_dz)
    return {k: (tuple(x.to(dev) for x in v) if isinstance(v, tuple) else v.to(dev))
            for k, v in inp.items()}


def bench_scan_fwd(args, wid: str, output_key: bool = False) -> dict:
    """One step = one ttt_scan_fwd over the whole batch (with the key-side output rule of
    Eq. 9 in the E2E paper review, section 2.4.2, when output_key)."""
    import ctypes
    import torch
    from test_weight_sequence_amd import ops
    from test_weight_sequence_amd.synth import WORKLOADS
    w = WORKLOADS[wid]
    headline = wid == "ttt_mlp_bf16_d64_T8k" and not output_key
    cfg = ops.Config(kind=w.kind, B=w.B, H=w.H, T=w.T, d=w.d, hidden=w.hidden, chunk=w.chunk,
                     io=w.io, force_generic=args.force_generic, one_wg_per_head=args.one_wg,
                     output_key=output_key)
    kernel = ops.fwd_kernel_name(cfg)
    dev = torch.device("cuda:0")
    d = _device_inputs(w, dev)
    ws = ops.new_workspace(cfg, ops.TTT_OP_FWD, dev)
    Z = torch.empty(w.B, w.H, w.T, w.d, dtype=cfg.io_dtype, device=dev)
    WT = tuple(torch.empty(s, device=dev) for s in cfg.weight_shapes((w.B, w.H)))
    # arguments are marshalled once, outside the timed region
    cfg_struct = cfg.c()
    cfg_c = ctypes.byref(cfg_struct)
    P = ctypes.c_void_p
    ptrs = [P(d[k].data_ptr()) for k in ("Q", "K", "V", "eta", "gamma", "beta")]
    ptrs.append(ctypes.byref(ops.CWeights(d["W0"][0].data_ptr(), d["W0"][1].data_ptr())))
    ptrs.append(P(Z.data_ptr()))
    wt_arg = ctypes.byref(ops.CWeights(WT[0].data_ptr(), WT[1].data_ptr()))
    ws_ptr = P(ws.data_ptr())
    stream = P(torch.cuda.current_stream().cuda_stream)
    fwd = ops.lib().ttt_scan_fwd
    ms_step, kms = _time_calls(
        lambda i: fwd(cfg_c, *ptrs, wt_arg, None, None, ws_ptr, ws.numel(), stream),
        args.steps, args.warmup)
    if ops.read_status(ws) != 0:
        raise RuntimeError("kernel reported non-finite values")
    k_avg = statistics.fmean(kms)
    units = w.B * w.H * w.T
    # A mini-batch larger than 16 tokens is evaluated in 16-token blocks (the dual-form tril
    # products inside a block, the earlier blocks through the running weights), so the work per
    # token is that of b = 16 however large the mini-batch is.
    flop = units * (key_flops_per_token_head(w.d, w.hidden) if output_key else
                    flops_per_token_head(w.d, w.hidden, min(w.chunk, 16)))
    achieved = flop / (k_avg * 1e-3) / 1e12
    mfma = kernel != "ttt_fwd_generic"
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_FP32_VALU_TFLOPS
    io_bytes = 2 if w.io == "bf16" else 4
    metric = ("TTT-MLP scan token*heads/s at d=64, T=8K (+ fraction of MI355X dense bf16 MFMA peak)"
              if headline else f"TTT-MLP scan token*heads/s at d={w.d}, T={w.T}" +
              (f", mini-batch {w.chunk}" if w.chunk != 16 else "") +
              (", key-side output rule (z_t = f(K_t; W at the chunk start))" if output_key else ""))
    out = _base_record(args, metric, units / (ms_step * 1e-3), ms_step, w, kernel,
                       "bf16" if mfma else "f32", {"output": "key"} if output_key else None)
    if headline:
        out["context"] = CONTEXT_SCAN
    # counter summaries are per launch variant: larger mini-batches move different bytes
    # from the 16-token launch of the same kernel
    variant = "" if w.chunk == 16 else f"_b{w.chunk}"
    out["roofline"] = {
        "bound": "mfma" if mfma else "alu", "achieved": achieved, "peak": peak,
        "unit": "TFLOP/s", "frac": achieved / peak,
        "traffic": _traffic(kernel, units, variant) if kernel in KERNEL_SOURCES else None,
        "kernel_ms": k_avg, "kernel_ms_min": min(kms), "flop_per_launch": flop,
        # (Q is not read under the key-side rule)
        "algorithmic_bytes_per_launch": units * (bytes_per_token_head(
            w.d, io_bytes, 2 * w.d * w.hidden, w.T) - (w.d * io_bytes if output_key else 0))}
    if not args.no_cpu_baseline:
        if headline:
            out["cpu_baseline"] = cpu_baseline(w, args.cpu_seqs, args.cpu_T)
        else:
            # about 10-15 s of oracle work: up to 8 sequences x 4096 tokens
            out["cpu_baseline"] = cpu_baseline(w, min(w.B, 8), 4096,
                                               output="key" if output_key else "query")
    return out


def bench_scan_fwd_momentum(args) -> dict:
    """One step = one ttt_scan_fwd_momentum over the whole batch (the tuned kernel; the portable
    fp32 one with --force-generic), d=64 T=8192 head shape at B=8, H=12, gates
    mom = 0.9 sigmoid(u), alpha = 0.01 sigmoid(u')."""
    import torch
    from test_weight_sequence_amd import ops
    from test_weight_sequence_amd.synth import WORKLOADS, momentum_gates
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    cfg = ops.Config(kind=w.kind, B=w.B, H=w.H, T=w.T, d=w.d, hidden=w.hidden, chunk=w.chunk, io=w.io,
                     force_generic=args.force_generic)
    dev = torch.device("cuda:0")
    d = _device_inputs(w, dev)
    gates = {k: v.to(dev) for k, v in momentum_gates(w).items()}
    ws = ops.new_workspace(cfg, ops.TTT_OP_FWD_MOMENTUM, dev)

    def call(i):
        ops.scan_fwd_momentum(cfg, d["Q"], d["K"], d["V"], d["eta"], gates["mom"], gates["alpha"],
                              d["W0"], d["gamma"], d["beta"], workspace=ws)
        return 0

    ms_step, kms = _time_calls(call, args.steps, args.warmup)
    if ops.read_status(ws) != 0:
        raise RuntimeError("kernel reported non-finite values")
    k_avg = statistics.fmean(kms)
    units = w.B * w.H * w.T
    # the plain scan's products, plus Q S1 and A^Q S2 and the momentum's own update
    flop = units * (flops_per_token_head(w.d, w.hidden, w.chunk) + 8 * w.d * w.hidden)
    achieved = flop / (k_avg * 1e-3) / 1e12
    kernel = ops.fwd_momentum_kernel_name(cfg)
    mfma = kernel != "ttt_fwd_generic"
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_FP32_VALU_TFLOPS
    out = _base_record(args, f"TTT-MLP momentum/forget-gate scan token*heads/s at d={w.d}, T={w.T}",
                       units / (ms_step * 1e-3), ms_step, w, kernel, "bf16" if mfma else "f32")
    out["roofline"] = {
        "bound": "mfma" if mfma else "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
        "frac": achieved / peak, "traffic": _traffic(kernel, units) if kernel in KERNEL_SOURCES else None,
        "kernel_ms": k_avg,
        "kernel_ms_min": min(kms), "flop_per_launch": flop,
        # the plain scan's streams and W0 / W_T, the two gates (fp32) and the final momentum S_T
        "algorithmic_bytes_per_launch": units * (bytes_per_token_head(w.d, 2, 2 * w.d * w.hidden, w.T) + 8)
                                        + w.B * w.H * 2 * w.d * w.hidden * 4}
    return out


def lact_flops_per_token_head(d: int, h: int) -> int:
    # nine d*h-sized products per token: K W1, K W3, V W2^T, the three gradient sums
    # (K^T gA, K^T gC, u~^T V) and the read-out Q W1, Q W3, U W2
    return 18 * d * h


def bench_lact(args) -> dict:
    """One step = one ttt_lact_fwd (the large-chunk SwiGLU layer) over the whole batch:
    B=8, H=12, T=8192, d=64, hidden=256, chunks of 2048 tokens."""
    import torch
    from test_weight_sequence_amd import ops
    from test_weight_sequence_amd.synth import WORKLOADS
    w = WORKLOADS["lact_swiglu_bf16_d64_T8k_b2048"]
    cfg = ops.Config(kind="swiglu", B=w.B, H=w.H, T=w.T, d=w.d, hidden=w.hidden, chunk=w.chunk, io=w.io)
    dev = torch.device("cuda:0")
    d = _device_inputs(w, dev)
    ws = ops.new_workspace(cfg, ops.TTT_OP_LACT, dev)
    Z = torch.empty(w.B, w.H, w.T, w.d, dtype=torch.bfloat16, device=dev)

    def call(i):
        ops.lact_fwd(cfg, d["Q"], d["K"], d["V"], d["eta"], d["W0"], workspace=ws, out=Z)
        return 0

    ms_step, kms = _time_calls(call, args.steps, args.warmup)
    if ops.read_status(ws) != 0:
        raise RuntimeError("kernel reported non-finite values")
    k_avg = statistics.fmean(kms)
    units = w.B * w.H * w.T
    flop = units * lact_flops_per_token_head(w.d, w.hidden)
    achieved = flop / (k_avg * 1e-3) / 1e12
    kernel = "ttt_lact_fwd_d64"
    out = _base_record(args, f"LaCT SwiGLU layer token*heads/s at d={w.d}, T={w.T}, chunk {w.chunk}",
                       units / (ms_step * 1e-3), ms_step, w, kernel, "bf16")
    out["context"] = CONTEXT_LACT
    out["data"] = ("synthetic (seeded N(0,1/d) Q/K/V, W1, W3 ~ N(0,1/d), W2 ~ N(0,1/hidden), "
                   "eta=1.0*sigmoid(N(0,1)))")
    nW = 3 * w.d * w.hidden
    out["roofline"] = {
        "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": achieved / PEAK_BF16_TFLOPS, "traffic": _traffic(kernel, units),
        # one call = T/chunk + 1 launches of the step kernel and the W_T copy-out; the
        # duration is the whole call's, bracketed by events on the launch stream
        "kernel_ms": k_avg, "kernel_ms_min": min(kms), "flop_per_launch": flop,
        # Q, K, V in and Z out (bf16), eta in, W0 in and W_T out (fp32, three matrices)
        "algorithmic_bytes_per_launch": units * (4 * w.d * 2 + 4) + w.H * nW * 4 + w.B * w.H * nW * 4}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_lact(w, 1, 4096)
    return out


def cpu_baseline_lact(w, n_seq: int, T: int) -> dict:
    """The fp64 oracle's large-chunk layer (scan_lact) on the first n_seq sequences, all heads,
    first T tokens."""
    import torch
    from oracle import scan_lact
    from test_weight_sequence_amd.synth import flatten_heads, make_inputs
    torch.set_num_threads(max(1, torch.get_num_threads()))
    cores = torch.get_num_threads()
    inp = flatten_heads(make_inputs(w, batch_idx=list(range(n_seq)), T=T))
    t0 = time.perf_counter()
    scan_lact(inp["Q"], inp["K"], inp["V"], inp["eta"], inp["W0"], w.chunk)
    dt = time.perf_counter() - t0
    pairs = n_seq * w.H
    return {"value": pairs * T / dt, "unit": "token*heads/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"fp64 oracle scan_lact on sequences 0..{n_seq - 1} x heads 0..{w.H - 1} "
                      f"({pairs} (batch, head) pairs) x first T={T} tokens of the same workload "
                      f"({dt:.1f} s wall, torch intra-op threads={cores})"}


def bwd_flops_per_token_head(d: int, h: int, b: int) -> int:
    # The chunk's forward recomputed from its saved start weights (the five forward products:
    # K W1, A^K W2, E2 W2^T, Q W1, A^Q W2, and the four dual terms), then two adjoint
    # products for each of the seven d*h products (the five above and the two weight
    # updates) and for each of the four dual terms.
    return 5 * 2 * d * h + 4 * b * (d + h) + 2 * (7 * 2 * d * h + 4 * b * (d + h))


def bench_scan_bwd(args) -> dict:
    """One step = one ttt_scan_bwd over the whole batch (saved chunk-start weights from one
    forward before the timed region)."""
    import torch
    from test_weight_sequence_amd import ops
    from test_weight_sequence_amd.synth import WORKLOADS
    w = WORKLOADS["ttt_mlp_bf16_d64_fwd_bwd"]
    cfg = ops.Config(kind=w.kind, B=w.B, H=w.H, T=w.T, d=w.d, hidden=w.hidden, chunk=w.chunk,
                     io=w.io, force_generic=args.force_generic, one_wg_per_head=args.one_wg)
    kernel = ops.bwd_kernel_name(cfg)
    dev = torch.device("cuda:0")
    d = _device_inputs(w, dev, with_dz=True)
    fwd = ops.scan_fwd(cfg, d["Q"], d["K"], d["V"], d["eta"], d["W0"], d["gamma"], d["beta"],
                       want_saved=True)
    ws = ops.new_workspace(cfg, ops.TTT_OP_BWD, dev)
    res = {}

    def call(i):
        res.update(ops.scan_bwd(cfg, d["Q"], d["K"], d["V"], d["eta"], d["gamma"], d["beta"],
                                fwd["saved"], d["dZ"], workspace=ws))
        return 0

    ms_step, kms = _time_calls(call, args.steps, args.warmup)
    if ops.read_status(ws) != 0:
        raise RuntimeError("kernel reported non-finite values")
    k_avg = statistics.fmean(kms)
    units = w.B * w.H * w.T
    flop = units * bwd_flops_per_token_head(w.d, w.hidden, w.chunk)
    achieved = flop / (k_avg * 1e-3) / 1e12
    mfma = kernel != "ttt_bwd_generic"
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_FP32_VALU_TFLOPS
    out = _base_record(args, f"TTT-MLP outer-loop backward token*heads/s at d={w.d}, T={w.T}",
                       units / (ms_step * 1e-3), ms_step, w, kernel, "bf16" if mfma else "f32")
    saved_bytes = w.B * w.H * (w.T // w.chunk) * 2 * w.d * w.hidden * 4
    out["roofline"] = {
        "bound": "mfma" if mfma else "alu", "achieved": achieved, "peak": peak,
        "unit": "TFLOP/s", "frac": achieved / peak,
        "traffic": _traffic(kernel, units) if kernel in KERNEL_SOURCES else None,
        "kernel_ms": k_avg, "kernel_ms_min": min(kms), "flop_per_launch": flop,
        # Q, K, V, dZ in and dQ, dK, dV out (bf16), eta in and deta out, the saved weights
        "algorithmic_bytes_per_launch": units * (7 * w.d * 2 + 8) + saved_bytes}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, 1, 1024, n_heads=4, grads=True)
    return out


def bench_decode(args) -> dict:
    """One step = one full chunk of decode calls (16 tokens for every (batch, head) of the
    d = 64 bf16 MLP shape), so every step includes one commit. The chunk's 16 calls are
    captured once into a HIP graph (through torch.cuda.graph) and the graph is replayed, as a
    serving loop would run them: a call through the Python binding costs more host time than
    the kernel takes on the GPU. The eager per-call wall time is reported beside it."""
    import ctypes
    import torch
    from test_weight_sequence_amd import ops
    from test_weight_sequence_amd.synth import WORKLOADS
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    if args.decode_batch:
        w = w.with_(B=args.decode_batch)
    b = w.chunk
    cfg = ops.Config(kind=w.kind, B=w.B, H=w.H, T=b, d=w.d, hidden=w.hidden, chunk=b, io=w.io,
                     force_generic=args.force_generic, decode_split=args.decode_split)
    dev = torch.device("cuda:0")
    d = _device_inputs(w.with_(T=b), dev)
    Ws = tuple(x.unsqueeze(0).expand(w.B, *x.shape).contiguous() for x in d["W0"])
    acc = tuple(torch.zeros_like(x) for x in Ws)
    qkv = [d[k].permute(2, 0, 1, 3).contiguous() for k in ("Q", "K", "V")]  # [b, B, H, d]
    eta = d["eta"].permute(2, 0, 1).contiguous()
    z = torch.empty(w.B, w.H, w.d, dtype=cfg.io_dtype, device=dev)
    ws = ops.new_workspace(cfg, ops.TTT_OP_DECODE, dev)
    cfg_struct = cfg.c()
    cfg_c = ctypes.byref(cfg_struct)
    P = ctypes.c_void_p
    wsw = ctypes.byref(ops.CWeights(Ws[0].data_ptr(), Ws[1].data_ptr()))
    wacc = ctypes.byref(ops.CWeights(acc[0].data_ptr(), acc[1].data_ptr()))
    gam, bet = P(d["gamma"].data_ptr()), P(d["beta"].data_ptr())
    per_tok = [[P(qkv[0][t].data_ptr()), P(qkv[1][t].data_ptr()), P(qkv[2][t].data_ptr()),
                P(eta[t].data_ptr())] for t in range(b)]
    zp, ws_ptr = P(z.data_ptr()), P(ws.data_ptr())
    dec = ops.lib().ttt_decode_step

    def call(t, stream):
        q, k, v, e = per_tok[t]
        return dec(cfg_c, q, k, v, e, gam, bet, wsw, wacc, t, zp, ws_ptr, ws.numel(), stream)

    eager_stream = P(torch.cuda.current_stream().cuda_stream)
    eager_ms_step, _ = _time_calls(lambda t: call(t, eager_stream), max(2, args.steps // 4), 1,
                                   calls_per_step=b)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cap = P(torch.cuda.current_stream().cuda_stream)
        for t in range(b):
            rc = call(t, cap)
            if rc != 0:
                raise ops.TTTError(rc, "ttt_decode_step (capture)")

    def replay(i):
        graph.replay()
        return 0

    ms_step, kms = _time_calls(replay, args.steps, args.warmup)
    if ops.read_status(ws) != 0:
        raise RuntimeError("kernel reported non-finite values")
    heads = w.B * w.H
    nW = 2 * w.d * w.hidden * 4
    # per head: every call reads W_start and acc; b - 1 calls write acc, the commit writes
    # W_start and clears acc
    bytes_step = heads * nW * (2 * b + (b - 1) + 2)
    k_sum_step = statistics.fmean(kms)
    achieved = bytes_step / (k_sum_step * 1e-3) / 1e9
    kernel = ops.decode_kernel_name(cfg)
    out = _base_record(args, f"TTT-MLP decode token*heads/s at d={w.d} ({heads} heads, one token "
                             "per head per call)", heads * b / (ms_step * 1e-3), ms_step,
                       w.with_(T=b), kernel, "f32", extra_cfg={"launch": f"HIP graph of {b} calls"})
    out["roofline"] = {
        "bound": "hbm", "achieved": achieved, "peak": 8000.0, "unit": "GB/s",
        "frac": achieved / 8000.0,
        "traffic": _traffic(kernel, heads) if kernel in KERNEL_SOURCES else None,
        # GPU time of one replayed chunk (16 kernels back to back) / 16
        "kernel_ms": k_sum_step / b, "kernel_ms_min": min(kms) / b,
        "algorithmic_bytes_per_launch": bytes_step / b}
    out["eager_ms_per_call"] = eager_ms_step / b
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, w.B, 4096)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 2 for the d=128 workload)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default 5; 1 for the d=128 workload)")
    ap.add_argument("--workload", default="scan_fwd",
                    choices=["scan_fwd", "scan_fwd_b16", "scan_fwd_d128", "scan_bwd", "decode",
                             "scan_fwd_momentum", "scan_fwd_bigchunk", "scan_fwd_key", "lact"],
                    help="scan_fwd: B=8 H=12 T=8192 d=64 forward (the headline); "
                         "scan_fwd_b16: the same head shape at B=16 (192 heads, 131,072 tokens "
                         "per batch); "
                         "scan_fwd_d128: B=1 H=24 T=131072 d=128 forward; "
                         "scan_fwd_momentum: the B=8 forward with momentum and forget gate; "
                         "scan_fwd_bigchunk: the B=8 forward with mini-batches of --chunk "
                         "tokens (256 or 1024); "
                         "scan_fwd_key: the B=8 forward with the key-side output rule; "
                         "lact: the large-chunk SwiGLU layer, B=8 H=12 T=8192, chunks of 2048; "
                         "scan_bwd: B=4 H=16 T=8192 d=64 outer-loop backward; "
                         "decode: one chunk of decode steps at the B=8 H=12 d=64 shape")
    ap.add_argument("--chunk", type=int, default=256, choices=[256, 1024],
                    help="mini-batch size of the scan_fwd_bigchunk workload")
    ap.add_argument("--decode-batch", type=int, default=0, metavar="B",
                    help="decode workload only: B sequences of 12 heads instead of 8")
    ap.add_argument("--decode-split", action="store_true",
                    help="decode workload only: four workgroups per head (TTT_DECODE_SPLIT)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=8)
    ap.add_argument("--cpu-T", type=int, default=8192)
    ap.add_argument("--force-generic", action="store_true")
    ap.add_argument("--one-wg", action="store_true",
                    help="tuned kernel with one workgroup per head (no producer/consumer pair)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the scan, time a plain device-to-device copy of MIB MiB "
                         "(the known-size reference for scaling the HBM byte counters)")
    args = ap.parse_args()
    long_run = args.workload == "scan_fwd_d128" or (args.workload == "scan_fwd_momentum" and args.force_generic)
    if args.steps is None:
        args.steps = 2 if long_run else 20
    if args.warmup is None:
        args.warmup = 1 if long_run else 5
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on exactly one GPU; the scan's heads would be "
              "sharded across GPUs with no communication, which is not built here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(torch.device("cuda:0"))

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.randn(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                          "ms_per_copy": dt * 1e3, "GB_per_s": 8 * n / dt / 1e9}), flush=True)
        return

    if args.workload == "scan_fwd":
        out = bench_scan_fwd(args, "ttt_mlp_bf16_d64_T8k")
    elif args.workload == "scan_fwd_b16":
        out = bench_scan_fwd(args, "ttt_mlp_bf16_d64_T8k_B16")
    elif args.workload == "scan_fwd_d128":
        out = bench_scan_fwd(args, "ttt_mlp_bf16_d128_T128k")
    elif args.workload == "scan_fwd_bigchunk":
        out = bench_scan_fwd(args, f"ttt_mlp_bf16_d64_T8k_b{args.chunk}")
    elif args.workload == "lact":
        out = bench_lact(args)
    elif args.workload == "scan_fwd_key":
        out = bench_scan_fwd(args, "ttt_mlp_bf16_d64_T8k", output_key=True)
    elif args.workload == "scan_bwd":
        out = bench_scan_bwd(args)
    elif args.workload == "scan_fwd_momentum":
        out = bench_scan_fwd_momentum(args)
    else:
        out = bench_decode(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
