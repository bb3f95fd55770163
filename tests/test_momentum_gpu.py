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


def _case(wid, B, H, T, seed_s0=None, mom_max=0.9, alpha_max=0.01, **cfg_kw):
    w = WORKLOADS[wid]
    inp = make_inputs(w, batch_idx=range(B), head_idx=range(H), T=T)
    inp.update(momentum_gates(w, batch_idx=range(B), head_idx=range(H), T=T, mom_max=mom_max,
                              alpha_max=alpha_max))
    cfg = ops_config(w, B=B, H=H, T=T, **cfg_kw)
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


MOM_KERNELS = {"mfma": ({}, "ttt_fwd_mfma_mom_d64"), "generic": (dict(force_generic=True), "ttt_fwd_generic")}


@pytest.mark.parametrize("wid,B,H,T,s0,kernel", [
    ("ttt_mlp_fp32_d16", 1, 1, 256, None, "generic"),
    ("ttt_mlp_fp32_d16", 1, 1, 256, 5, "generic"),
    ("ttt_linear_fp32_d64", 2, 3, 512, 6, "generic"),
    ("ttt_mlp_bf16_d64_T8k", 1, 3, 1024, 7, "mfma"),
    ("ttt_mlp_bf16_d64_T8k", 1, 3, 1024, 7, "generic"),
    ("ttt_mlp_bf16_d64_T8k", 2, 5, 256, None, "mfma"),
    ("ttt_mlp_bf16_d128_T128k", 1, 2, 256, None, "generic"),
])
def test_momentum_scan_matches_oracle(wid, B, H, T, s0, kernel):
    flags, name = MOM_KERNELS[kernel]
    w, cfg, inp, S0 = _case(wid, B, H, T, seed_s0=s0, **flags)
    assert ops.fwd_momentum_kernel_name(cfg) == name
    note(f"momentum {wid} B={B} H={H} T={T} s0={s0} {name}")
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


def test_momentum_mfma_full_size_sampled_heads():
    """The tuned momentum kernel on the full B=8 H=12 T=8192 launch (the shape the benchmark
    times); the oracle checks three heads at full length.

    Over 8192 tokens with momentum up to 0.9 the scan's final memory and momentum are chaotic:
    perturbing Q, K, V and W0 by the bf16 rounding step moves the oracle's own M_T and S_T by
    7-9% (relative L2) and Z by 1%. Z and the loss keep the plain bf16 bound; the final states
    are bounded by twice the oracle-to-oracle change under that perturbation."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    inp = make_inputs(w)
    inp.update(momentum_gates(w))
    cfg = ops_config(w)
    assert ops.fwd_momentum_kernel_name(cfg) == "ttt_fwd_mfma_mom_d64"
    note("momentum mfma full size")
    res = _run(cfg, inp, None)
    pairs = [(0, 0), (3, 7), (7, 11)]
    sub = {k: torch.stack([inp[k][b, h] for b, h in pairs])[None] for k in ("Q", "K", "V", "eta", "mom", "alpha")}
    sub["W0"] = tuple(torch.stack([x[h] for _, h in pairs]) for x in inp["W0"])
    sub["gamma"] = torch.stack([inp["gamma"][h] for _, h in pairs])
    sub["beta"] = torch.stack([inp["beta"][h] for _, h in pairs])
    scfg = ops_config(w, B=1, H=3)
    Z, MT, ST, L = _oracle(w, scfg, sub, None)
    P = _oracle_perturbed(w, scfg, sub, None, seeds=(0, 1, 2))
    tol = TOL["bf16"]
    assert_parity(torch.stack([res["Z"][b, h] for b, h in pairs]).cpu(), Z, tol, "Z",
                  perturbed=[p[0] for p in P])
    assert_parity(torch.stack([res["loss"][b, h] for b, h in pairs]).cpu(), L, tol, "loss", per_token=False,
                  perturbed=[p[3] for p in P])
    for k in range(2):
        g = torch.stack([res["W_T"][k][b, h] for b, h in pairs]).cpu()
        assert_parity(g, MT[k], tol, f"M_T[{k}]", time_axis=False, perturbed=[p[1][k] for p in P],
                      whole_from_perturbed=True)
        g = torch.stack([res["S_T"][k][b, h] for b, h in pairs]).cpu()
        assert_parity(g, ST[k], tol, f"S_T[{k}]", time_axis=False, perturbed=[p[2][k] for p in P],
                      whole_from_perturbed=True)


@pytest.mark.parametrize("device_scope", [False, True])
def test_momentum_mfma_tanh_per_seq_scaled(device_scope):
    """The tuned momentum kernel with tanh GELU, per-sequence W0, a carried-in momentum,
    eta_scale = 0.5 and a head count that leaves most of the last group of eight empty; with
    device_scope the two workgroups of a head exchange their partial sums through the
    device-scope path (counters and fences), as when they sit on different XCDs."""
    from oracle import OracleConfig, scan_momentum
    B, H, T = 2, 3, 192
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    inp = make_inputs(w, batch_idx=range(B), head_idx=range(H), T=T)
    inp.update(momentum_gates(w, batch_idx=range(B), head_idx=range(H), T=T))
    g = torch.Generator().manual_seed(41)
    inp["W0"] = tuple(x.unsqueeze(0).expand(B, *x.shape) + 0.01 * torch.randn((B,) + x.shape, generator=g)
                      for x in inp["W0"])
    cfg = ops.Config(kind="mlp", B=B, H=H, T=T, d=64, hidden=256, chunk=16, io="bf16", gelu="tanh",
                     w0_per_seq=True, eta_scale=0.5, device_scope=device_scope)
    assert ops.fwd_momentum_kernel_name(cfg) == "ttt_fwd_mfma_mom_d64"
    S0 = tuple(1e-3 * torch.randn((B, H) + s[2:], generator=g) for s in cfg.weight_shapes((B, H)))
    note(f"momentum mfma tanh per-seq device_scope={device_scope}")
    res = _run(cfg, inp, S0)
    n = B * H
    flat = flatten_heads({**inp, "W0": tuple(x[0] for x in inp["W0"])})
    flat["W0"] = tuple(x.double().reshape(n, *x.shape[2:]) for x in inp["W0"])
    Z, MT, ST, _ = scan_momentum(flat["Q"], flat["K"], flat["V"], flat["eta"],
                                 inp["mom"].double().reshape(n, -1), inp["alpha"].double().reshape(n, -1),
                                 flat["W0"], tuple(s.double().reshape(n, *s.shape[2:]) for s in S0),
                                 flat["gamma"], flat["beta"], OracleConfig(kind="mlp", chunk=16, gelu="tanh",
                                                                           eta_scale=0.5))
    assert_parity(res["Z"].reshape(n, T, -1), Z, TOL["bf16"], "Z")
    for x, o in zip(res["W_T"] + res["S_T"], MT + ST):
        assert_parity(x.reshape(o.shape), o, TOL["bf16"], "M_T/S_T", time_axis=False)


def test_momentum_mfma_gates_off_matches_plain_scan():
    """mom = 0 and alpha = 0 reduce the tuned momentum kernel to the plain scan: against the
    paired forward kernel on the same inputs (different kernels, so within the bf16 bound)."""
    w, cfg, inp, _ = _case("ttt_mlp_bf16_d64_T8k", 2, 3, 512, mom_max=0.0, alpha_max=0.0)
    assert ops.fwd_momentum_kernel_name(cfg) == "ttt_fwd_mfma_mom_d64"
    note("momentum mfma gates off vs paired scan")
    res = _run(cfg, inp, None)
    d = to_dev(inp)
    ref = ops.scan_fwd(cfg, d["Q"], d["K"], d["V"], d["eta"], d["W0"], d["gamma"], d["beta"])
    torch.cuda.synchronize()
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_pair_d64"
    assert_parity(res["Z"].reshape(6, 512, -1).cpu(), ref["Z"].reshape(6, 512, -1).cpu(), TOL["bf16"], "Z")
    for a, b in zip(res["W_T"], ref["W_T"]):
        assert_parity(a.reshape(6, -1).cpu(), b.reshape(6, -1).cpu(), TOL["bf16"], "W_T", time_axis=False)


def test_momentum_mfma_state_carries_across_calls():
    """Two calls of T/2 tokens of the tuned kernel, the second started from the first's
    (M_T, S_T), equal one call (bitwise: the same kernel, the same order of operations)."""
    w, cfg, inp, _ = _case("ttt_mlp_bf16_d64_T8k", 1, 2, 256)
    note("momentum mfma carry across calls")
    full = _run(cfg, inp, None)
    half = ops_config(w, B=1, H=2, T=128, w0_per_seq=True)
    cut = lambda x, sl: x[:, :, sl].contiguous() if x.dim() >= 3 else x
    a_inp = {k: (cut(v, slice(0, 128)) if k in ("Q", "K", "V", "eta", "mom", "alpha") else v) for k, v in inp.items()}
    a_inp["W0"] = tuple(x.unsqueeze(0).expand(1, *x.shape).contiguous() for x in inp["W0"])
    a = _run(half, a_inp, None)
    b_inp = {k: (cut(v, slice(128, 256)) if k in ("Q", "K", "V", "eta", "mom", "alpha") else v) for k, v in inp.items()}
    b_inp["W0"] = tuple(x.cpu() for x in a["W_T"])
    b = _run(half, b_inp, tuple(x.cpu() for x in a["S_T"]))
    assert torch.equal(torch.cat([a["Z"], b["Z"]], dim=2), full["Z"])
    for x, y in zip(b["W_T"] + b["S_T"], full["W_T"] + full["S_T"]):
        assert torch.equal(x, y)
