"""Thin ctypes binding over libttt.so (argument marshalling only).

Every step of the scan runs in the HIP library; torch is used here only to allocate
device memory and to obtain the current HIP stream. If libttt.so is missing or
cannot be loaded, every entry point raises: there is no fallback path.

Names mirror include/ttt.h: scan_fwd, scan_fwd_momentum, scan_bwd, decode_step, lact_fwd, validate,
workspace_size, saved_size, read_status, reset_status, fwd_kernel_name, bwd_kernel_name,
decode_kernel_name.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttt.so")

TTT_LINEAR, TTT_MLP, TTT_SWIGLU = 0, 1, 2
TTT_F32, TTT_BF16 = 0, 1
TTT_GELU_ERF, TTT_GELU_TANH = 0, 1
TTT_W0_PER_SEQ, TTT_FORCE_GENERIC, TTT_ONE_WG_PER_HEAD, TTT_OUTPUT_KEY = 1, 2, 4, 8
TTT_FORCE_DEVICE_SCOPE = 16
TTT_DECODE_SPLIT = 32
TTT_LACT_READ_BEFORE = 64
TTT_OP_FWD, TTT_OP_BWD, TTT_OP_DECODE, TTT_OP_FWD_MOMENTUM, TTT_OP_LACT = 0, 1, 2, 3, 4

STATUS = {0: "TTT_OK", 1: "TTT_ERR_NULL", 2: "TTT_ERR_SHAPE", 3: "TTT_ERR_DTYPE",
          4: "TTT_ERR_UNSUPPORTED", 5: "TTT_ERR_ALIGN", 6: "TTT_ERR_WORKSPACE",
          7: "TTT_ERR_HIP", 8: "TTT_ERR_NONFINITE", 9: "TTT_ERR_ARG",
          10: "TTT_ERR_TIMEOUT"}

EXPORTS = ("ttt_validate", "ttt_workspace_size", "ttt_saved_size", "ttt_scan_fwd", "ttt_scan_fwd_static",
           "ttt_scan_fwd_momentum",
           "ttt_scan_bwd", "ttt_decode_step", "ttt_lact_fwd", "ttt_read_status", "ttt_reset_status",
           "ttt_fwd_kernel_name", "ttt_fwd_momentum_kernel_name", "ttt_bwd_kernel_name",
           "ttt_decode_kernel_name", "ttt_status_str",
           "ttt_abi_version")


class TTTError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, code)}")
        self.code = code


class CConfig(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("T", ctypes.c_int32), ("d", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("gelu", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("eta_scale", ctypes.c_float)]


class CWeights(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w2", ctypes.c_void_p)]


class CSwiGLUWeights(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("w3", ctypes.c_void_p)]


_lib = None
_loaded = {}


def _load(path: str) -> ctypes.CDLL:
    """Load a build of the library at `path` and declare its entry points (raises if the
    file has not been built)."""
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m test_weight_sequence_amd.build`")
    L = ctypes.CDLL(path)
    P, S, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    cfgp = ctypes.POINTER(CConfig)
    wp = ctypes.POINTER(CWeights)
    L.ttt_validate.argtypes = [cfgp]
    L.ttt_workspace_size.argtypes = [cfgp, I32, ctypes.POINTER(S)]
    L.ttt_saved_size.argtypes = [cfgp, ctypes.POINTER(S)]
    L.ttt_scan_fwd.argtypes = [cfgp, P, P, P, P, P, P, wp, P, wp, P, P, P, S, P]
    L.ttt_scan_fwd_static.argtypes = [cfgp, P, P, P, P, P, P, wp, P, wp, P, P, P, P]
    L.ttt_scan_fwd_momentum.argtypes = [cfgp, P, P, P, P, P, P, P, P, wp, wp, P, wp, wp, P, P, S, P]
    L.ttt_scan_bwd.argtypes = [cfgp, P, P, P, P, P, P, P, P, wp, P, P, P, P, wp, P, P, P, S, P]
    L.ttt_decode_step.argtypes = [cfgp, P, P, P, P, P, P, wp, wp, I32, P, P, S, P]
    sp = ctypes.POINTER(CSwiGLUWeights)
    L.ttt_lact_fwd.argtypes = [cfgp, P, P, P, P, sp, P, sp, P, S, P]
    L.ttt_read_status.argtypes = [P, P]
    L.ttt_reset_status.argtypes = [P, P]
    L.ttt_fwd_kernel_name.argtypes = [cfgp]
    L.ttt_fwd_kernel_name.restype = ctypes.c_char_p
    L.ttt_fwd_momentum_kernel_name.argtypes = [cfgp]
    L.ttt_fwd_momentum_kernel_name.restype = ctypes.c_char_p
    L.ttt_bwd_kernel_name.argtypes = [cfgp]
    L.ttt_bwd_kernel_name.restype = ctypes.c_char_p
    L.ttt_decode_kernel_name.argtypes = [cfgp]
    L.ttt_decode_kernel_name.restype = ctypes.c_char_p
    L.ttt_status_str.argtypes = [I32]
    L.ttt_status_str.restype = ctypes.c_char_p
    for name in ("ttt_validate", "ttt_workspace_size", "ttt_saved_size", "ttt_scan_fwd",
                 "ttt_scan_fwd_static", "ttt_scan_fwd_momentum",
                 "ttt_scan_bwd", "ttt_decode_step", "ttt_lact_fwd", "ttt_read_status",
                 "ttt_reset_status", "ttt_abi_version"):
        getattr(L, name).restype = I32
    _loaded[path] = L
    return L


def lib() -> ctypes.CDLL:
    """Load libttt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Inside the with-block every call of this module goes to the build of the library at
    `path` (tests use it for the LDS-poisoning test build); afterwards to libttt.so again."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


@dataclass(frozen=True)
class Config:
    kind: str = "mlp"          # "mlp" | "linear" | "swiglu" (the large-chunk layer, lact_fwd)
    B: int = 1
    H: int = 1
    T: int = 16
    d: int = 64
    hidden: int = 256
    chunk: int = 16
    io: str = "bf16"           # "bf16" | "f32"
    gelu: str = "erf"          # "erf" | "tanh"
    w0_per_seq: bool = False
    force_generic: bool = False
    one_wg_per_head: bool = False  # tuned forward without the producer/consumer pairing
    output_key: bool = False       # Eq. 9 output rule: z_t = f(K_t; W at the chunk start)
    device_scope: bool = False     # tuned forward: device-scope hand-offs between workgroups
    decode_split: bool = False     # decode: four workgroups per head (MLP d = 64)
    read_before: bool = False      # lact_fwd: read a chunk out with its start weights
    ln_eps: float = 1e-6
    eta_scale: float = 1.0

    def c(self) -> CConfig:
        flags = (TTT_W0_PER_SEQ if self.w0_per_seq else 0) | \
                (TTT_FORCE_GENERIC if self.force_generic else 0) | \
                (TTT_ONE_WG_PER_HEAD if self.one_wg_per_head else 0) | \
                (TTT_OUTPUT_KEY if self.output_key else 0) | \
                (TTT_FORCE_DEVICE_SCOPE if self.device_scope else 0) | \
                (TTT_DECODE_SPLIT if self.decode_split else 0) | \
                (TTT_LACT_READ_BEFORE if self.read_before else 0)
        kind = {"mlp": TTT_MLP, "linear": TTT_LINEAR, "swiglu": TTT_SWIGLU}[self.kind]
        return CConfig(kind, self.B, self.H, self.T,
                       self.d, self.d if self.kind == "linear" else self.hidden, self.chunk,
                       TTT_BF16 if self.io == "bf16" else TTT_F32,
                       TTT_GELU_TANH if self.gelu == "tanh" else TTT_GELU_ERF, flags,
                       float(self.ln_eps), float(self.eta_scale))

    @property
    def io_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.io == "bf16" else torch.float32

    def weight_shapes(self, lead: tuple) -> list:
        if self.kind == "swiglu":
            return [(*lead, self.d, self.hidden), (*lead, self.hidden, self.d), (*lead, self.d, self.hidden)]
        if self.kind == "mlp":
            return [(*lead, self.d, self.hidden), (*lead, self.hidden, self.d)]
        return [(*lead, self.d, self.d)]


def _check(code: int, where: str):
    if code != 0:
        raise TTTError(code, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _weights(ws):
    if ws is None:
        return None
    w1 = ws[0].data_ptr()
    w2 = ws[1].data_ptr() if len(ws) > 1 and ws[1] is not None else None
    return ctypes.byref(CWeights(w1, w2))


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def validate(cfg: Config) -> int:
    return int(lib().ttt_validate(ctypes.byref(cfg.c())))


def workspace_size(cfg: Config, op: int = TTT_OP_FWD) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ttt_workspace_size(ctypes.byref(cfg.c()), op, ctypes.byref(n)),
           "ttt_workspace_size")
    return int(n.value)


def saved_size(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ttt_saved_size(ctypes.byref(cfg.c()), ctypes.byref(n)), "ttt_saved_size")
    return int(n.value)


def fwd_kernel_name(cfg: Config) -> str:
    return lib().ttt_fwd_kernel_name(ctypes.byref(cfg.c())).decode()


def fwd_momentum_kernel_name(cfg: Config) -> str:
    return lib().ttt_fwd_momentum_kernel_name(ctypes.byref(cfg.c())).decode()


def bwd_kernel_name(cfg: Config) -> str:
    return lib().ttt_bwd_kernel_name(ctypes.byref(cfg.c())).decode()


def decode_kernel_name(cfg: Config) -> str:
    return lib().ttt_decode_kernel_name(ctypes.byref(cfg.c())).decode()


def new_workspace(cfg: Config, op: int = TTT_OP_FWD, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (status word cleared) for `op`."""
    return torch.zeros(max(workspace_size(cfg, op), 256), dtype=torch.uint8, device=device)


def read_status(workspace: torch.Tensor, stream=None) -> int:
    return int(lib().ttt_read_status(_ptr(workspace), _stream(stream)))


def reset_status(workspace: torch.Tensor, stream=None):
    _check(lib().ttt_reset_status(_ptr(workspace), _stream(stream)), "ttt_reset_status")


def scan_fwd(cfg: Config, Q, K, V, eta, W0, gamma, beta, *, want_wt=True, want_loss=False,
             want_saved=False, workspace=None, out=None, stream=None) -> dict:
    """Forward scan. Device tensors: Q, K, V [B,H,T,d] (io dtype), eta [B,H,T] fp32,
    W0 tuple of fp32 ([H,...] or [B,H,...] with w0_per_seq), gamma/beta [H,d] fp32.
    Returns dict with Z and, when asked, W_T, loss, saved."""
    dev = Q.device
    lead = (cfg.B, cfg.H)
    Z = out if out is not None else torch.empty(*lead, cfg.T, cfg.d, dtype=cfg.io_dtype, device=dev)
    WT = [torch.empty(s, dtype=torch.float32, device=dev) for s in cfg.weight_shapes(lead)] \
        if want_wt else None
    loss = torch.empty(*lead, cfg.T, dtype=torch.float32, device=dev) if want_loss else None
    saved = torch.empty(saved_size(cfg) // 4, dtype=torch.float32, device=dev) \
        if want_saved else None
    ws = workspace if workspace is not None else new_workspace(cfg, TTT_OP_FWD, dev)
    code = lib().ttt_scan_fwd(ctypes.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(eta),
                              _ptr(gamma), _ptr(beta), _weights(W0), _ptr(Z), _weights(WT),
                              _ptr(loss), _ptr(saved), _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "ttt_scan_fwd")
    return {"Z": Z, "W_T": tuple(WT) if WT else None, "loss": loss, "saved": saved,
            "workspace": ws}


def scan_fwd_static(cfg: Config, Q, K, V, eta, W0, gamma, beta, *, want_wt=True,
                    want_loss=False, want_saved=False, want_status=True, out=None,
                    stream=None) -> dict:
    """ttt_scan_fwd_static: the forward scan with the library's own device workspace (no
    workspace argument). Outputs are allocated here as for scan_fwd; the call itself
    allocates nothing. "status" is a one-element int32 device tensor holding the call's
    status word (0 = clean)."""
    dev = Q.device
    lead = (cfg.B, cfg.H)
    Z = out if out is not None else torch.empty(*lead, cfg.T, cfg.d, dtype=cfg.io_dtype, device=dev)
    WT = [torch.empty(s, dtype=torch.float32, device=dev) for s in cfg.weight_shapes(lead)] \
        if want_wt else None
    loss = torch.empty(*lead, cfg.T, dtype=torch.float32, device=dev) if want_loss else None
    saved = torch.empty(saved_size(cfg) // 4, dtype=torch.float32, device=dev) \
        if want_saved else None
    status = torch.full((1,), -1, dtype=torch.int32, device=dev) if want_status else None
    code = lib().ttt_scan_fwd_static(ctypes.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(eta),
                                     _ptr(gamma), _ptr(beta), _weights(W0), _ptr(Z), _weights(WT),
                                     _ptr(loss), _ptr(saved), _ptr(status), _stream(stream))
    _check(code, "ttt_scan_fwd_static")
    return {"Z": Z, "W_T": tuple(WT) if WT else None, "loss": loss, "saved": saved,
            "status": status}


def scan_fwd_momentum(cfg: Config, Q, K, V, theta, mom, alpha, W0, gamma, beta, S0=None, *,
                      want_loss=False, workspace=None, stream=None) -> dict:
    """Forward scan with momentum and a forget gate (ttt_scan_fwd_momentum). theta, mom,
    alpha [B,H,T] fp32; S0 (optional) tuple of fp32 [B,H,...]. Returns Z, W_T, S_T (and
    loss when asked)."""
    dev = Q.device
    lead = (cfg.B, cfg.H)
    Z = torch.empty(*lead, cfg.T, cfg.d, dtype=cfg.io_dtype, device=dev)
    WT = [torch.empty(s, dtype=torch.float32, device=dev) for s in cfg.weight_shapes(lead)]
    ST = [torch.empty(s, dtype=torch.float32, device=dev) for s in cfg.weight_shapes(lead)]
    loss = torch.empty(*lead, cfg.T, dtype=torch.float32, device=dev) if want_loss else None
    ws = workspace if workspace is not None else new_workspace(cfg, TTT_OP_FWD_MOMENTUM, dev)
    code = lib().ttt_scan_fwd_momentum(
        ctypes.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(theta), _ptr(mom), _ptr(alpha),
        _ptr(gamma), _ptr(beta), _weights(W0), _weights(S0), _ptr(Z), _weights(WT), _weights(ST),
        _ptr(loss), _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "ttt_scan_fwd_momentum")
    return {"Z": Z, "W_T": tuple(WT), "S_T": tuple(ST), "loss": loss, "workspace": ws}


def scan_bwd(cfg: Config, Q, K, V, eta, gamma, beta, saved, dZ, dW_T=None, *,
             want_dgb=True, workspace=None, stream=None) -> dict:
    """Outer-loop backward. Returns dQ, dK, dV (io dtype), deta, dW0 (tuple, shaped like
    W0) and, when asked, dgamma, dbeta ([H,d])."""
    dev = Q.device
    lead = (cfg.B, cfg.H)
    dQ, dK, dV = (torch.empty_like(x) for x in (Q, K, V))
    deta = torch.empty_like(eta)
    w_lead = lead if cfg.w0_per_seq else (cfg.H,)
    dW0 = [torch.empty(s, dtype=torch.float32, device=dev) for s in cfg.weight_shapes(w_lead)]
    dg = torch.empty(cfg.H, cfg.d, dtype=torch.float32, device=dev) if want_dgb else None
    db = torch.empty(cfg.H, cfg.d, dtype=torch.float32, device=dev) if want_dgb else None
    ws = workspace if workspace is not None else new_workspace(cfg, TTT_OP_BWD, dev)
    code = lib().ttt_scan_bwd(ctypes.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(eta),
                              _ptr(gamma), _ptr(beta), _ptr(saved), _ptr(dZ), _weights(dW_T),
                              _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(deta), _weights(dW0),
                              _ptr(dg), _ptr(db), _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "ttt_scan_bwd")
    return {"dQ": dQ, "dK": dK, "dV": dV, "deta": deta, "dW0": tuple(dW0), "dgamma": dg,
            "dbeta": db, "workspace": ws}


def decode_step(cfg: Config, q, k, v, eta, gamma, beta, W_start, acc, pos_in_chunk, *,
                z=None, workspace=None, stream=None):
    """One decode token per (batch, head); W_start / acc ([B,H,...] fp32 tuples) are
    updated in place. Returns z [B,H,d]."""
    dev = q.device
    z = z if z is not None else torch.empty(cfg.B, cfg.H, cfg.d, dtype=cfg.io_dtype, device=dev)
    ws = workspace if workspace is not None else new_workspace(cfg, TTT_OP_DECODE, dev)
    code = lib().ttt_decode_step(ctypes.byref(cfg.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                 _ptr(gamma), _ptr(beta), _weights(W_start), _weights(acc),
                                 int(pos_in_chunk), _ptr(z), _ptr(ws), ws.numel(),
                                 _stream(stream))
    _check(code, "ttt_decode_step")
    return z


def lact_fwd(cfg: Config, Q, K, V, eta, W0, *, want_wt=True, workspace=None, out=None,
             stream=None) -> dict:
    """The large-chunk SwiGLU layer (ttt_lact_fwd). Q, K, V [B,H,T,d] bf16, eta [B,H,T] fp32,
    W0 = (W1, W2, W3) fp32 ([H,...] or [B,H,...] with w0_per_seq). Returns Z and W_T."""
    lead = (cfg.B, cfg.H)
    dev = Q.device
    Z = out if out is not None else torch.empty(*lead, cfg.T, cfg.d, dtype=cfg.io_dtype, device=dev)
    WT = tuple(torch.empty(s, dtype=torch.float32, device=dev) for s in cfg.weight_shapes(lead)) \
        if want_wt else None
    ws = workspace if workspace is not None else new_workspace(cfg, TTT_OP_LACT, dev)
    w0 = CSwiGLUWeights(W0[0].data_ptr(), W0[1].data_ptr(), W0[2].data_ptr())
    wt = CSwiGLUWeights(WT[0].data_ptr(), WT[1].data_ptr(), WT[2].data_ptr()) if WT else None
    code = lib().ttt_lact_fwd(ctypes.byref(cfg.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(eta),
                              ctypes.byref(w0), _ptr(Z), ctypes.byref(wt) if wt else None,
                              _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "ttt_lact_fwd")
    return {"Z": Z, "W_T": WT, "workspace": ws}
