"""Seeded synthetic inputs for the TTT scan workloads.

This module holds only input recipes (shapes, distributions, seeds, rounding to the
I/O dtype). It contains none of the scan's arithmetic, so both the HIP path and the
CPU oracle can be fed from it.

Every random stream is keyed by (seed, tensor, batch index, head index), so any
subset of heads, and any prefix of the token axis, is generated identically to the
corresponding slice of the full workload.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

_TENSOR_CODE = {"Q": 0, "K": 1, "V": 2, "u": 3, "W0": 4, "dZ": 5, "u_mom": 6, "u_alpha": 7}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "mlp", "linear" or "swiglu" (the large-chunk SwiGLU layer)
    B: int
    H: int
    T: int
    d: int
    hidden: int        # 4d for the MLP; equals d for the linear map
    chunk: int
    io: str            # "f32" or "bf16" for Q, K, V, Z
    eta_base: float    # eta_t = eta_base * sigmoid(u_t), u_t ~ N(0, 1)
    w0: str            # "normal": N(0, 0.02^2); "identity_plus": I + N(0, 0.02^2);
                       # "fan_in": entries N(0, 1/inputs) (the SwiGLU layer's W1, W2, W3)
    drift: float = 0.0  # AR(1) coefficient along tokens (0 = i.i.d.)
    seed: int = 0

    @property
    def heads(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The seeded workloads of the scan, keyed by name (shapes, dtypes and value
# distributions).
WORKLOADS = {
    "ttt_mlp_fp32_d16": Workload("ttt_mlp_fp32_d16", "mlp", 1, 1, 256, 16, 64, 16, "f32", 0.1, "normal", seed=1001),
    "ttt_linear_fp32_d64": Workload("ttt_linear_fp32_d64", "linear", 4, 12, 2048, 64, 64, 16, "f32", 1.0,
                "identity_plus", seed=1002),
    "ttt_mlp_bf16_d64_T8k": Workload("ttt_mlp_bf16_d64_T8k", "mlp", 8, 12, 8192, 64, 256, 16, "bf16", 0.1, "normal",
                seed=1003),
    "ttt_mlp_bf16_d128_T128k": Workload("ttt_mlp_bf16_d128_T128k", "mlp", 1, 24, 131072, 128, 512, 16, "bf16", 0.1,
                "normal", drift=0.999, seed=1004),
    "ttt_mlp_bf16_d64_fwd_bwd": Workload("ttt_mlp_bf16_d64_fwd_bwd", "mlp", 4, 16, 8192, 64, 256, 16, "bf16", 0.1,
                "normal", seed=1005),
    # the d=64 T=8192 head shape at 131,072 tokens per batch (B=16, 192 heads): the same
    # seed as the B=8 workload, so its first eight sequences are that workload's inputs
    "ttt_mlp_bf16_d64_T8k_B16": Workload("ttt_mlp_bf16_d64_T8k_B16", "mlp", 16, 12, 8192, 64, 256, 16, "bf16", 0.1,
                "normal", seed=1003),
    # the B=8 d=64 T=8192 inputs (same seed) with large mini-batches of 256 and 1024 tokens
    "ttt_mlp_bf16_d64_T8k_b256": Workload("ttt_mlp_bf16_d64_T8k_b256", "mlp", 8, 12, 8192, 64, 256, 256, "bf16", 0.1,
                "normal", seed=1003),
    "ttt_mlp_bf16_d64_T8k_b1024": Workload("ttt_mlp_bf16_d64_T8k_b1024", "mlp", 8, 12, 8192, 64, 256, 1024, "bf16",
                0.1, "normal", seed=1003),
    # the large-chunk SwiGLU layer at the same head shape and token count, chunks of 2048
    "lact_swiglu_bf16_d64_T8k_b2048": Workload("lact_swiglu_bf16_d64_T8k_b2048", "swiglu", 8, 12, 8192, 64, 256,
                2048, "bf16", 1.0, "fan_in", seed=1006),
}


def _rng(seed: int, tensor: str, *idx: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, _TENSOR_CODE[tensor], *idx]))


def _token_stream(w: Workload, tensor: str, b: int, h: int, T: int, d: int) -> np.ndarray:
    """[T, d] fp64 with N(0, 1/d) marginals; AR(1) along tokens when drift > 0."""
    e = _rng(w.seed, tensor, b, h).standard_normal((T, d)) * math.sqrt(1.0 / d)
    if w.drift <= 0.0:
        return e
    from scipy.signal import lfilter
    rho = w.drift
    c = math.sqrt(1.0 - rho * rho)
    # x_0 = e_0 ; x_t = rho x_{t-1} + c e_t  (keeps the marginal at N(0, 1/d))
    zi = ((1.0 - c) * e[0])[None, :]
    return lfilter([c], [1.0, -rho], e, axis=0, zi=zi)[0]


def _round_io(x: np.ndarray, io: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32)
    return t.to(torch.bfloat16) if io == "bf16" else t


def make_inputs(w: Workload, batch_idx=None, head_idx=None, T: int | None = None,
                with_dz: bool = False) -> dict:
    """Build one workload's inputs (CPU tensors, already in their I/O dtypes).

    batch_idx / head_idx select a sub-grid of (batch, head) pairs (default: all);
    T selects a token prefix (default: w.T). Returns
      Q, K, V, [dZ]: [nb, nh, T, d] in the I/O dtype
      eta:           [nb, nh, T] fp32
      W0:            tuple of fp32 [nh, ...] (shared across the batch axis)
                     MLP: (W1 [nh, d, hidden], W2 [nh, hidden, d]); linear: (W [nh, d, d],)
      gamma, beta:   [nh, d] fp32 (ones / zeros)
    """
    bi = list(range(w.B)) if batch_idx is None else list(batch_idx)
    hi = list(range(w.H)) if head_idx is None else list(head_idx)
    T = w.T if T is None else int(T)
    if T % w.chunk != 0:
        raise ValueError("T must be a multiple of the chunk size")
    d, hid = w.d, w.hidden
    out = {}
    names = ["Q", "K", "V"] + (["dZ"] if with_dz else [])
    for name in names:
        arr = np.empty((len(bi), len(hi), T, d))
        for i, b in enumerate(bi):
            for j, h in enumerate(hi):
                if name == "dZ":
                    arr[i, j] = _rng(w.seed, "dZ", b, h).standard_normal((T, d))
                else:
                    arr[i, j] = _token_stream(w, name, b, h, T, d)
        out[name] = _round_io(arr, w.io)
    eta = np.empty((len(bi), len(hi), T))
    for i, b in enumerate(bi):
        for j, h in enumerate(hi):
            u = _rng(w.seed, "u", b, h).standard_normal(T)
            eta[i, j] = w.eta_base / (1.0 + np.exp(-u))
    out["eta"] = torch.from_numpy(eta).to(torch.float32)
    if w.kind == "swiglu":
        # W1, W3 [d, hidden] with N(0, 1/d) entries, W2 [hidden, d] with N(0, 1/hidden)
        Ws = [np.empty((len(hi), d, hid)), np.empty((len(hi), hid, d)), np.empty((len(hi), d, hid))]
        for j, h in enumerate(hi):
            for k, (shape, fan) in enumerate((((d, hid), d), ((hid, d), hid), ((d, hid), d))):
                Ws[k][j] = _rng(w.seed, "W0", h, k).standard_normal(shape) * math.sqrt(1.0 / fan)
        out["W0"] = tuple(torch.from_numpy(x).float() for x in Ws)
    elif w.kind == "mlp":
        W1 = np.empty((len(hi), d, hid))
        W2 = np.empty((len(hi), hid, d))
        for j, h in enumerate(hi):
            r = _rng(w.seed, "W0", h)
            W1[j] = r.standard_normal((d, hid)) * 0.02
            W2[j] = r.standard_normal((hid, d)) * 0.02
        out["W0"] = (torch.from_numpy(W1).float(), torch.from_numpy(W2).float())
    else:
        Wl = np.empty((len(hi), d, d))
        for j, h in enumerate(hi):
            Wl[j] = _rng(w.seed, "W0", h).standard_normal((d, d)) * 0.02
            if w.w0 == "identity_plus":
                Wl[j] += np.eye(d)
        out["W0"] = (torch.from_numpy(Wl).float(),)
    out["gamma"] = torch.ones(len(hi), d, dtype=torch.float32)
    out["beta"] = torch.zeros(len(hi), d, dtype=torch.float32)
    return out


def flatten_heads(inp: dict) -> dict:
    """Reshape a make_inputs() dict to per-(batch, head) rows in fp64:
    Q/K/V/dZ -> [N, T, d], eta -> [N, T], W0 -> per-row copies, gamma/beta -> [N, d]."""
    nb, nh = inp["Q"].shape[:2]
    out = {}
    for name in ("Q", "K", "V", "dZ"):
        if name in inp:
            x = inp[name]
            out[name] = x.to(torch.float64).reshape(nb * nh, *x.shape[2:])
    out["eta"] = inp["eta"].to(torch.float64).reshape(nb * nh, -1)
    out["W0"] = tuple(w.to(torch.float64).unsqueeze(0).expand(nb, *w.shape)
                      .reshape(nb * nh, *w.shape[1:]).clone() for w in inp["W0"])
    for name in ("gamma", "beta"):
        g = inp[name].to(torch.float64)
        out[name] = g.unsqueeze(0).expand(nb, *g.shape).reshape(nb * nh, -1).clone()
    return out


def momentum_gates(w: Workload, batch_idx=None, head_idx=None, T: int | None = None,
                   mom_max: float = 0.9, alpha_max: float = 0.01) -> dict:
    """Per-token gates for the momentum / forget-gate scan, fp32 [nb, nh, T]:
    mom_t = mom_max * sigmoid(u_t), alpha_t = alpha_max * sigmoid(u'_t), u, u' ~ N(0, 1),
    keyed like the other streams (a slice is generated exactly as the full workload).
    The forget gate stays small: with alpha up to 0.1 the memory of the d=64 MLP decays into
    the LayerNorm's eps regime and the scan's output moves by O(1) under 1e-7 input noise."""
    bi = list(range(w.B)) if batch_idx is None else list(batch_idx)
    hi = list(range(w.H)) if head_idx is None else list(head_idx)
    T = w.T if T is None else T
    out = {}
    for name, code, top in (("mom", "u_mom", mom_max), ("alpha", "u_alpha", alpha_max)):
        arr = np.empty((len(bi), len(hi), T))
        for i, b in enumerate(bi):
            for j, h in enumerate(hi):
                u = _rng(w.seed, code, b, h).standard_normal(w.T)[:T]
                arr[i, j] = top / (1.0 + np.exp(-u))
        out[name] = torch.from_numpy(arr).to(torch.float32)
    return out
