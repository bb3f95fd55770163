"""GPU parity of ttt_scan_fwd_momentum (momentum and forget gate, "Titans와 Miras" Eq. 13/14
of the TTT-memory page, on the mini-batch scan) against the fp64 oracle's primal scan."""
from __future__ import annotations

import pytest
import torch

from helpers import BF16_STEP, TOL, assert_parity, note, ops_config, rel_l2, to_dev
from oracle import OracleConfig, scan_momentum
from test_weight_sequence_amd import ops
from test_weight_sequence_amd.synth import WORKLOADS, flatten_heads, make_inputs, momentum_gates

pytestmark = pytest.mark.gpu


def _case(wid, B, H, T, seed_s0=None, mom_max=0.9, alpha_max=0.01):
    w = WORKLOADS[wid]
    inp = make_inputs(w, batch_idx=range(B), head_idx=range(H), T=T)
    inp.update(momentum_gates(w, batch_idx=range(B), head_idx=range(H), T=T, mom_max=mom_max,
                              alpha_max=alpha_max))
    cfg = ops_config(w, B=B, H=H, T=T)
    S0 = None
    if seed_s0 is not None:
        g = torch.Generator().manual_seed(seed_s0)
        S0 = tuple(1e-3 * torch.randn((B, H) + s[2:], generator=g) for s in cfg.weight_shapes((B, H)))
    return w, cfg, inp, S0


def _oracle(w, cfg, inp, S0):
    flat = flatten_heads(inp)
    n = cfg.B * cfg.H
    mom = inp["mom"].to(torch.float64).reshape(n, -1)
    alpha = inp["alpha"].to(torch.float64).reshape(n, -1)
    s0 = None if S0 is None else tuple(s.to(torch.float64).reshape(n, *s.shape[2:]) for s in S0)
    ocfg = OracleConfig(kind=w.kind, chunk=w.chunk)
    return scan_momentum(flat["Q"], flat["K"], flat["V"], flat["eta"], mom, alpha, flat["W0"], s0,
                         flat["gamma"], flat["beta"], ocfg)


def _oracle_perturbed(w, cfg, inp, S0, seeds=(0, 1, 2, 3)):
    """The momentum oracle on inputs (Q, K, V, W0) perturbed at the bf16 rounding scale, one run
    per seed (see helpers.oracle_perturbed)."""
    out = []
    for sd in seeds:
        g = torch.Generator().manual_seed(1000 + sd)
        pert = lambda x: x.double() * (1.0 + BF16_STEP * torch.randn(x.shape, generator=g, dtype=torch.float64))
        pi = dict(inp)
        for k in ("Q", "K", "V"):
            pi[k] = pert(inp[k])
        pi["W0"] = tuple(pert(x) for x in inp["W0"])
        out.append(_oracle(w, cfg, pi, S0))
    return out


def _run(cfg, inp, S0):
    d = to_dev(inp)
    s0 = None if S0 is None else tuple(s.cuda().contiguous() for s in S0)
    res = ops.scan_fwd_momentum(cfg, d["Q"], d["K"], d["V"], d["eta"], d["mom"], d["alpha"], d["W0"],
                                d["gamma"], d["beta"], S0=s0, want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    return res


@pytest.mark.parametrize("wid,B,H,T,s0", [
    ("ttt_mlp_fp32_d16", 1, 1, 256, None),
    ("ttt_mlp_fp32_d16", 1, 1, 256, 5),
    ("ttt_linear_fp32_d64", 2, 3, 512, 6),
    ("ttt_mlp_bf16_d64_T8k", 1, 3, 1024, 7),
    ("ttt_mlp_bf16_d128_T128k", 1, 2, 256, None),
])
def test_momentum_scan_matches_oracle(wid, B, H, T, s0):
    w, cfg, inp, S0 = _case(wid, B, H, T, seed_s0=s0)
    note(f"momentum {wid} B={B} H={H} T={T} s0={s0}")
    res = _run(cfg, inp, S0)
    Z, MT, ST, L = _oracle(w, cfg, inp, S0)
    tol = TOL["bf16" if w.io == "bf16" else "f32"]
    n = cfg.B * cfg.H
    P = _oracle_perturbed(w, cfg, inp, S0) if w.d >= 128 else None
    assert_parity(res["Z"].reshape(n, T, -1), Z, tol, "Z", perturbed=P and [p[0] for p in P])
    assert_parity(res["loss"].reshape(n, T), L, tol, "loss", per_token=False,
                  perturbed=P and [p[3] for p in P])
    for g, o in zip(res["W_T"] + res["S_T"], MT + ST):
        assert_parity(g.reshape(o.shape), o, tol, "M_T/S_T", time_axis=False)


def test_momentum_without_gates_equals_plain_scan():
    """mom = 0 and alpha = 0 reduce the variant to ttt_scan_fwd (portable kernel, same inputs)."""
    w, cfg, inp, _ = _case("ttt_mlp_fp32_d16", 1, 1, 256, mom_max=0.0, alpha_max=0.0)
    note("momentum gates off vs plain scan")
    res = _run(cfg, inp, None)
    d = to_dev(inp)
    gcfg = ops_config(w, B=1, H=1, T=256, force_generic=True)
    ref = ops.scan_fwd(gcfg, d["Q"], d["K"], d["V"], d["eta"], d["W0"], d["gamma"], d["beta"])
    torch.cuda.synchronize()
    assert rel_l2(res["Z"], ref["Z"]) <= 1e-6
    for a, b in zip(res["W_T"], ref["W_T"]):
        assert rel_l2(a, b) <= 1e-6


def test_momentum_state_carries_across_calls():
    """Two calls of T/2 tokens, the second started from the first's (W_T, S_T), equal one call."""
    w, cfg, inp, _ = _case("ttt_linear_fp32_d64", 1, 2, 256)
    note("momentum carry across calls")
    full = _run(cfg, inp, None)
    half = ops_config(w, B=1, H=2, T=128, w0_per_seq=True)
    cut = lambda x, sl: x[:, :, sl].contiguous() if x.dim() >= 3 else x
    a_inp = {k: (cut(v, slice(0, 128)) if k in ("Q", "K", "V", "eta", "mom", "alpha") else v) for k, v in inp.items()}
    a_inp["W0"] = tuple(x.unsqueeze(0).expand(1, *x.shape).contiguous() for x in inp["W0"])
    a = _run(half, a_inp, None)
    b_inp = {k: (cut(v, slice(128, 256)) if k in ("Q", "K", "V", "eta", "mom", "alpha") else v) for k, v in inp.items()}
    b_inp["W0"] = tuple(x.cpu() for x in a["W_T"])
    b = _run(half, b_inp, tuple(x.cpu() for x in a["S_T"]))
    assert rel_l2(torch.cat([a["Z"], b["Z"]], dim=2), full["Z"]) <= 1e-6
    for x, y in zip(b["W_T"] + b["S_T"], full["W_T"] + full["S_T"]):
        assert rel_l2(x, y) <= 1e-6


@pytest.mark.parametrize("wid,H", [("ttt_mlp_fp32_d16", 1), ("ttt_mlp_bf16_d64_T8k", 3)])
def test_momentum_full_forget_one_chunk_closed_form(wid, H):
    """alpha = 1 (the forget gate at the top of its range) and mom = 0 over one chunk: the
    memory after token t is its own step alone, M_t = S_t = -theta_t grad l_t(W0), so
    z_t = f(Q_t; -theta_t grad l_t(W0)) with the gradient from the oracle's hand-derived
    token gradient. This case is well conditioned at any alpha, unlike long scans with a
    strong forget gate."""
    from oracle import f_apply, token_loss_and_grad
    w, cfg, inp, _ = _case(wid, 1, H, 16, mom_max=0.0, alpha_max=0.0)
    inp["mom"] = torch.zeros_like(inp["mom"])
    inp["alpha"] = torch.ones_like(inp["alpha"])
    note(f"momentum full forget one chunk {wid} H={H}")
    res = _run(cfg, inp, None)
    flat = flatten_heads(inp)
    ocfg = OracleConfig(kind=w.kind, chunk=w.chunk)
    zs = []
    for t in range(16):
        _, grads = token_loss_and_grad(flat["K"][:, t], flat["V"][:, t], flat["W0"], flat["gamma"],
                                       flat["beta"], ocfg)
        th = flat["eta"][:, t].reshape(-1, 1, 1)
        Mt = tuple(-th * g for g in grads)
        zs.append(f_apply(flat["Q"][:, t], Mt, flat["gamma"], flat["beta"], ocfg))
    Zc = torch.stack(zs, dim=1)
    tol = TOL["bf16" if w.io == "bf16" else "f32"]
    assert_parity(res["Z"].reshape(H, 16, -1), Zc, tol, "Z vs closed form")
    # the carried memory and momentum are the last token's step
    for g, m in zip(res["W_T"] + res["S_T"], Mt + Mt):
        assert_parity(g.reshape(m.shape), m, tol, "M_T/S_T", time_axis=False)
