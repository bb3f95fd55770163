"""Shared helpers for the GPU parity tests (inputs from the seeded generator, the
oracle on selected heads, relative L2 error)."""
from __future__ import annotations

import sys

import torch

from oracle import OracleConfig, scan as oracle_scan
from test_weight_sequence_amd import ops
from test_weight_sequence_amd.synth import flatten_heads, make_inputs

TOL = {"f32": 1e-4, "bf16": 2e-2}


def note(msg: str):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, file=sys.stderr, flush=True)


def rel_l2(a: torch.Tensor, b: torch.Tensor) -> float:
    a = a.detach().to("cpu", torch.float64)
    b = b.detach().to("cpu", torch.float64)
    return ((a - b).norm() / b.norm()).item()


def to_dev(inp: dict, device="cuda") -> dict:
    out = {}
    for k, v in inp.items():
        if isinstance(v, tuple):
            out[k] = tuple(x.to(device).contiguous() for x in v)
        else:
            out[k] = v.to(device).contiguous()
    return out


def ops_config(w, T=None, B=None, H=None, **kw) -> ops.Config:
    return ops.Config(kind=w.kind, B=B or w.B, H=H or w.H, T=T or w.T, d=w.d,
                      hidden=w.hidden, chunk=w.chunk, io=w.io, **kw)


def oracle_heads(inp: dict, pairs, kind, chunk, **cfg_kw):
    """Run the oracle on the listed (batch, head) pairs of a make_inputs() dict."""
    sub = {}
    for k in ("Q", "K", "V", "eta"):
        sub[k] = torch.stack([inp[k][b, h] for b, h in pairs])[None]
    sub["W0"] = tuple(torch.stack([w[h] for _, h in pairs]) for w in inp["W0"])
    sub["gamma"] = torch.stack([inp["gamma"][h] for _, h in pairs])
    sub["beta"] = torch.stack([inp["beta"][h] for _, h in pairs])
    # flatten_heads expects [nb, nh, ...]; pairs are laid out as one batch row
    flat = flatten_heads(sub)
    cfg = OracleConfig(kind=kind, chunk=chunk, **cfg_kw)
    torch.set_num_threads(max(1, torch.get_num_threads()))
    Z, WT, L = oracle_scan(flat["Q"], flat["K"], flat["V"], flat["eta"], flat["W0"],
                           flat["gamma"], flat["beta"], cfg)
    return Z, WT, L


def fresh_inputs(w, **kw):
    return make_inputs(w, **kw)
