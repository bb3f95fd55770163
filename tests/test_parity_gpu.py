"""GPU parity: the HIP scan (through the C ABI) against the fp64 CPU oracle on the
same seeded inputs. Tolerances (relative L2): 1e-4 for fp32 I/O, 2e-2 for bf16 I/O (fp32
state in both), over the whole tensor and over each head; outputs with a token axis are also
bounded per 16-token chunk and per token (helpers.assert_parity)."""
import math

import pytest
import torch

from helpers import (TOL, assert_parity, note, oracle_heads, oracle_perturbed, ops_config, rel_l2,
                     to_dev)
from oracle import OracleConfig, f_apply
from test_weight_sequence_amd import ops
from test_weight_sequence_amd.synth import WORKLOADS, flatten_heads, make_inputs

pytestmark = pytest.mark.gpu


def _run(cfg, d, **kw):
    return ops.scan_fwd(cfg, d["Q"], d["K"], d["V"], d["eta"], d["W0"], d["gamma"], d["beta"],
                        **kw)


def _sensitive(w) -> bool:
    """The d = 128 head shape (drifting inputs in its workload): a few tokens are far more
    sensitive to rounding than the average, so its chunk and token bounds take the oracle's
    own response to bf16-scale perturbations into account."""
    return w.d >= 128 or w.drift > 0


def _check_heads(res, inp, pairs, w, tol, cfg_kw=None, B_axis=True):
    out = oracle_heads(inp, pairs, w.kind, w.chunk, perturbed=_sensitive(w), **(cfg_kw or {}))
    Z, WT, L = out[:3]
    pz = [p[0] for p in out[3]] if len(out) > 3 else None
    pl = [p[2] for p in out[3]] if len(out) > 3 else None
    gz = torch.stack([res["Z"][b, h] for b, h in pairs]).cpu()
    err = assert_parity(gz, Z, tol, "Z", perturbed=pz)
    for k, wt in enumerate(WT):
        g = torch.stack([res["W_T"][k][b, h] for b, h in pairs]).cpu()
        assert_parity(g, wt, tol, f"W_T[{k}]", time_axis=False)
    if res.get("loss") is not None:
        gl = torch.stack([res["loss"][b, h] for b, h in pairs]).cpu()
        assert_parity(gl, L, tol, "loss", per_token=False, perturbed=pl)
    return err


# forward variants: the portable kernel, the tuned kernel with a producer/consumer pair of
# workgroups per head (the default where it applies), and the tuned kernel with one
# workgroup per head
KERNEL_FLAGS = {"generic": dict(force_generic=True), "pair": {}, "one_wg": dict(one_wg_per_head=True)}
KERNEL_NAMES = {"generic": "ttt_fwd_generic", "pair": "ttt_fwd_mfma_pair_d64",
                "one_wg": "ttt_fwd_mfma_d64"}


def _variant_config(w, kernel, **kw):
    cfg = ops_config(w, **kw, **KERNEL_FLAGS[kernel])
    assert ops.fwd_kernel_name(cfg) == KERNEL_NAMES[kernel], ops.fwd_kernel_name(cfg)
    return cfg


def test_mlp_fp32_d16_full():
    w = WORKLOADS["ttt_mlp_fp32_d16"]
    note(f"mlp fp32 d16 full {w}")
    inp = make_inputs(w)
    res = _run(ops_config(w), to_dev(inp), want_loss=True)
    _check_heads(res, inp, [(0, 0)], w, TOL["f32"])


def test_linear_fp32_d64_full():
    w = WORKLOADS["ttt_linear_fp32_d64"]
    note(f"linear fp32 d64 full {w}")
    inp = make_inputs(w)
    res = _run(ops_config(w), to_dev(inp), want_loss=True)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    _check_heads(res, inp, pairs, w, TOL["f32"])


@pytest.mark.parametrize("kernel", ["generic", "pair", "one_wg"])
def test_mlp_bf16_d64_T8k_sampled_heads(kernel):
    """Full launch at B=8, H=12, T=8192; the oracle checks three heads at full T."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    cfg = _variant_config(w, kernel)
    note(f"mlp bf16 d64 T8k full {kernel} -> {ops.fwd_kernel_name(cfg)}")
    inp = make_inputs(w)
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    _check_heads(res, inp, [(0, 0), (3, 7), (7, 11)], w, TOL["bf16"])


def test_mlp_bf16_d64_T8k_B16_sampled_heads():
    """Full launch at B=16, H=12, T=8192 (192 heads: one workgroup per head, the launch that
    the wider-batch measurement times); the oracle checks three heads at full T."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k_B16"]
    cfg = ops_config(w)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_d64"
    note("mlp bf16 d64 T8k B=16 full")
    inp = make_inputs(w)
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    _check_heads(res, inp, [(0, 5), (9, 2), (15, 11)], w, TOL["bf16"])


@pytest.mark.parametrize("kernel", ["generic", "pair", "one_wg"])
def test_mlp_bf16_d64_all_heads_short(kernel):
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    cfg = _variant_config(w, kernel, T=256)
    note(f"mlp bf16 d64 T=256 all heads {kernel}")
    inp = make_inputs(w, T=256)
    res = _run(cfg, to_dev(inp), want_loss=True)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    _check_heads(res, inp, pairs, w, TOL["bf16"])


D128_KERNELS = {"split": ({}, "ttt_fwd_mfma_split_d128"),
                "generic": (dict(force_generic=True), "ttt_fwd_generic")}


@pytest.mark.parametrize("kernel", ["split", "generic"])
def test_mlp_bf16_d128_reduced_T(kernel):
    """The d=128, hidden=512 head shape (AR(1) drifting inputs) on two heads, T=512,
    through the split kernel (four workgroups per head) and the portable one."""
    w = WORKLOADS["ttt_mlp_bf16_d128_T128k"]
    inp = make_inputs(w, head_idx=[0, 23], T=512)
    flags, name = D128_KERNELS[kernel]
    cfg = ops_config(w, T=512, H=2, **flags)
    assert ops.fwd_kernel_name(cfg) == name
    note(f"mlp bf16 d=128 T=512 heads 0,23 {name}")
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    _check_heads(res, inp, [(0, 0), (0, 1)], w, TOL["bf16"])


def test_mlp_bf16_d128_T128k_sampled_heads_prefix():
    """Full launch at B=1, H=24, T=131072 of the split kernel: the end state of every
    head is finite, and for two heads z and the per-token loss of the first 4096 tokens
    (which depend only on that prefix) match the oracle."""
    w = WORKLOADS["ttt_mlp_bf16_d128_T128k"]
    inp = make_inputs(w)
    cfg = ops_config(w)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_split_d128"
    note("mlp bf16 d128 T128k full size, split kernel")
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    for x in res["W_T"]:
        assert torch.isfinite(x).all()
    Tp = 4096
    pairs = [(0, 5), (0, 17)]
    pre = {k: (v[:, :, :Tp] if k in ("Q", "K", "V", "eta") else v) for k, v in inp.items()}
    Z, _, L, P = oracle_heads(pre, pairs, w.kind, w.chunk, perturbed=True)
    gz = torch.stack([res["Z"][b, h, :Tp] for b, h in pairs]).cpu()
    gl = torch.stack([res["loss"][b, h, :Tp] for b, h in pairs]).cpu()
    assert_parity(gz, Z, TOL["bf16"], "Z prefix", perturbed=[p[0] for p in P])
    assert_parity(gl, L, TOL["bf16"], "loss prefix", per_token=False, perturbed=[p[2] for p in P])


def test_mlp_bf16_d128_late_window():
    """The last 4096 tokens of the 131072-token d=128 workload on two heads, started from the
    fp64 oracle's weights after token 126976 (rounded to fp32, tests/golden/d128_late_state.npz,
    written by make_d128_late_state.py from the oracle alone). Both the split kernel (per-
    sequence W0) and the oracle start from that state, so the check covers the regime where the
    weights have grown over 7936 chunks, which the prefix check does not reach."""
    import os
    import numpy as np
    w = WORKLOADS["ttt_mlp_bf16_d128_T128k"]
    st = np.load(os.path.join(os.path.dirname(__file__), "golden", "d128_late_state.npz"))
    heads = [int(h) for h in st["heads"]]
    t0 = int(st["t_start"])
    Tw = w.T - t0
    full = make_inputs(w, head_idx=heads)
    inp = {k: (v[:, :, t0:].contiguous() if k in ("Q", "K", "V", "eta") else v) for k, v in full.items()}
    inp["W0"] = (torch.from_numpy(st["w1"]).unsqueeze(0), torch.from_numpy(st["w2"]).unsqueeze(0))
    cfg = ops_config(w, T=Tw, H=2, w0_per_seq=True)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_split_d128"
    note(f"mlp bf16 d128 late window heads {heads} tokens {t0}..{w.T}")
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    flat, ocfg = _oracle_all(inp, "mlp", w.chunk, per_seq=True)
    from oracle import scan as oracle_scan
    Z, WT, L = oracle_scan(flat["Q"], flat["K"], flat["V"], flat["eta"], flat["W0"],
                           flat["gamma"], flat["beta"], ocfg)
    P = oracle_perturbed(flat, ocfg)
    assert_parity(res["Z"].reshape(2, Tw, 128), Z, TOL["bf16"], "Z late window",
                  perturbed=[p[0] for p in P])
    assert_parity(res["loss"].reshape(2, Tw), L, TOL["bf16"], "loss late window", per_token=False,
                  perturbed=[p[2] for p in P])
    for g, o in zip(res["W_T"], WT):
        assert_parity(g.reshape(o.shape), o, TOL["bf16"], "W_T late window", time_axis=False)


def test_split_partial_group_tanh_per_seq():
    """The split kernel with per-sequence W0, tanh GELU and a head count that leaves most of
    the last group of eight empty (B=2, H=3), all heads against the oracle."""
    B, H, T = 2, 3, 96
    inp = _rand_case("mlp", B, H, T, 128, 16, "bf16", seed=13, per_seq=True)
    cfg = ops.Config(kind="mlp", B=B, H=H, T=T, d=128, hidden=512, chunk=16, io="bf16",
                     gelu="tanh", w0_per_seq=True, eta_scale=0.5)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_split_d128"
    note("split tanh per-seq B=2 H=3")
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    flat, ocfg = _oracle_all(inp, "mlp", 16, per_seq=True, gelu="tanh", eta_scale=0.5)
    from oracle import scan as oracle_scan
    Z, WT, L = oracle_scan(flat["Q"], flat["K"], flat["V"], flat["eta"], flat["W0"],
                           flat["gamma"], flat["beta"], ocfg)
    P = oracle_perturbed(flat, ocfg)
    assert_parity(res["Z"].reshape(B * H, T, 128), Z, TOL["bf16"], "Z", perturbed=[p[0] for p in P])
    assert_parity(res["loss"].reshape(B * H, T), L, TOL["bf16"], "loss", per_token=False,
                  perturbed=[p[2] for p in P])
    for g, o in zip(res["W_T"], WT):
        assert_parity(g.reshape(o.shape), o, TOL["bf16"], "W_T", time_axis=False)


def test_split_more_heads_than_one_launch():
    """72 heads of the d=128 shape: more than one launch of the split kernel holds on a
    256-CU device (64 heads); heads from both launches against the oracle."""
    w = WORKLOADS["ttt_mlp_bf16_d128_T128k"]
    B, H, T = 9, 8, 32
    inp = make_inputs(w.with_(B=9, H=8), T=T)
    cfg = ops_config(w, T=T, B=B, H=H)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_split_d128"
    note("split 72 heads")
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    _check_heads(res, inp, [(0, 0), (3, 5), (7, 7), (8, 0), (8, 7)], w, TOL["bf16"])


@pytest.mark.parametrize("B,H", [(4, 8), (5, 8)])
def test_split_forms_at_the_launch_boundary(B, H):
    """The d=128 kernel takes its producer/consumer form (eight workgroups per head) while all
    heads fit in one launch of it (32 heads on 256 CUs) and the form with both sides in every
    workgroup above that: 32 heads fill a whole launch of the first, 40 heads take the second.
    Heads from the first and the last group of eight against the oracle. The inputs are this
    head shape's without the AR(1) drift: over the first chunks of the drifting inputs the
    oracle itself moves by 5-24% on some heads when they are perturbed at the bf16 scale, which
    would leave a whole-tensor bound nothing to decide; here it moves by about 0.5%."""
    w = WORKLOADS["ttt_mlp_bf16_d128_T128k"].with_(drift=0.0)
    T = 48
    inp = make_inputs(w.with_(B=B, H=H), T=T)
    cfg = ops_config(w, T=T, B=B, H=H)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_split_d128"
    note(f"split {B * H} heads")
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    _check_heads(res, inp, [(0, 0), (1, 7), (B - 1, 0), (B - 1, H - 1)], w, TOL["bf16"])


def test_split_saved_chunk_start_weights():
    """The split kernel's saved buffer: W0 exactly at chunk 0, and at chunk 2 the W_T of a
    scan over the first two chunks."""
    w = WORKLOADS["ttt_mlp_bf16_d128_T128k"]
    T = 64
    inp = make_inputs(w, head_idx=[3, 4, 9], T=T)
    cfg = ops_config(w, T=T, H=3)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_split_d128"
    d = to_dev(inp)
    note("split saved weights")
    res = _run(cfg, d, want_saved=True)
    nW1 = w.d * w.hidden
    sv = res["saved"].view(1, 3, T // w.chunk, 2 * nW1).cpu()
    for h in range(3):
        assert torch.equal(sv[0, h, 0, :nW1], inp["W0"][0][h].reshape(-1))
        assert torch.equal(sv[0, h, 0, nW1:], inp["W0"][1][h].reshape(-1))
    pre = _run(ops_config(w, T=32, H=3), {**d, **{k: d[k][:, :, :32].contiguous()
                                                  for k in ("Q", "K", "V", "eta")}})
    torch.cuda.synchronize()
    assert torch.equal(sv[:, :, 2, :nW1], pre["W_T"][0].reshape(1, 3, -1).cpu())
    assert torch.equal(sv[:, :, 2, nW1:], pre["W_T"][1].reshape(1, 3, -1).cpu())


@pytest.mark.parametrize("kernel", ["generic", "pair", "one_wg"])
def test_mlp_bf16_d64_B4H16_fwd_sampled_heads(kernel):
    w = WORKLOADS["ttt_mlp_bf16_d64_fwd_bwd"]
    cfg = _variant_config(w, kernel)
    note(f"mlp bf16 d64 B=4 H=16 fwd full {kernel}")
    inp = make_inputs(w)
    res = _run(cfg, to_dev(inp))
    _check_heads(res, inp, [(1, 2), (3, 15)], w, TOL["bf16"])


@pytest.mark.parametrize("B,H,T", [(1, 5, 128), (2, 3, 16), (3, 1, 48)])
def test_pair_partial_groups_all_heads(B, H, T):
    """Head counts that leave part of the last group of 8 pairs empty, single-chunk and
    few-chunk scans (fewer chunks than ring slots): every head against the oracle."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    cfg = _variant_config(w, "pair", B=B, H=H, T=T)
    note(f"pair partial groups B={B} H={H} T={T}")
    inp = make_inputs(w, batch_idx=list(range(B)), head_idx=list(range(H)), T=T)
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    _check_heads(res, inp, [(b, h) for b in range(B) for h in range(H)], w, TOL["bf16"])


def test_pair_not_used_above_128_heads():
    """More than 128 (batch, head) pairs: the host picks one workgroup per head."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    cfg = ops_config(w, B=9, H=16, T=64)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_d64"
    note("144 heads T=64")
    inp = make_inputs(w, batch_idx=list(range(9)), head_idx=list(range(16)), T=64)
    res = _run(cfg, to_dev(inp))
    _check_heads(res, inp, [(0, 0), (4, 9), (8, 15)], w, TOL["bf16"])


def test_pair_tanh_per_seq():
    """The paired kernel with tanh GELU and per-sequence W0, all heads."""
    B, H, T = 2, 3, 160
    inp = _rand_case("mlp", B, H, T, 64, 16, "bf16", seed=11, per_seq=True)
    cfg = ops.Config(kind="mlp", B=B, H=H, T=T, d=64, hidden=256, chunk=16, io="bf16",
                     gelu="tanh", w0_per_seq=True, eta_scale=0.5)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_pair_d64"
    note("pair tanh per-seq")
    res = _run(cfg, to_dev(inp))
    flat, ocfg = _oracle_all(inp, "mlp", 16, per_seq=True, gelu="tanh", eta_scale=0.5)
    from oracle import scan as oracle_scan
    Z, WT, _ = oracle_scan(flat["Q"], flat["K"], flat["V"], flat["eta"], flat["W0"],
                           flat["gamma"], flat["beta"], ocfg)
    assert_parity(res["Z"].reshape(B * H, T, 64), Z, TOL["bf16"], "Z")
    for g, o in zip(res["W_T"], WT):
        assert_parity(g.reshape(o.shape), o, TOL["bf16"], "W_T", time_axis=False)


@pytest.mark.parametrize("B,H,T,gelu,per_seq", [(2, 3, 160, "tanh", True), (9, 16, 48, "erf", False)])
def test_key_output_tuned_variants(B, H, T, gelu, per_seq):
    """The tuned key-output forward with tanh GELU and per-sequence W0, and with 144 heads
    (above the paired kernel's head limit), all heads, Z, W_T and the loss."""
    inp = _rand_case("mlp", B, H, T, 64, 16, "bf16", seed=B * 100 + T, per_seq=per_seq)
    cfg = ops.Config(kind="mlp", B=B, H=H, T=T, d=64, hidden=256, chunk=16, io="bf16",
                     gelu=gelu, w0_per_seq=per_seq, eta_scale=0.5, output_key=True)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_key_d64"
    note(f"key output tuned B={B} H={H} T={T} {gelu} per_seq={per_seq}")
    res = _run(cfg, to_dev(inp), want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    flat, ocfg = _oracle_all(inp, "mlp", 16, per_seq=per_seq, gelu=gelu, eta_scale=0.5,
                             output="key")
    from oracle import scan as oracle_scan
    Z, WT, L = oracle_scan(flat["Q"], flat["K"], flat["V"], flat["eta"], flat["W0"],
                           flat["gamma"], flat["beta"], ocfg)
    assert_parity(res["Z"].reshape(B * H, T, 64), Z, TOL["bf16"], "Z")
    assert_parity(res["loss"].reshape(B * H, T), L, TOL["bf16"], "loss", per_token=False)
    for g, o in zip(res["W_T"], WT):
        assert_parity(g.reshape(o.shape), o, TOL["bf16"], "W_T", time_axis=False)


def _rand_case(kind, B, H, T, d, chunk, io, seed, per_seq=False):
    g = torch.Generator().manual_seed(seed)
    hid = 4 * d if kind == "mlp" else d
    sc = math.sqrt(1.0 / d)
    mk = lambda *s: torch.randn(*s, generator=g) * sc
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    inp = {"Q": mk(B, H, T, d).to(dt), "K": mk(B, H, T, d).to(dt), "V": mk(B, H, T, d).to(dt),
           "eta": 0.2 * torch.sigmoid(torch.randn(B, H, T, generator=g))}
    lead = (B, H) if per_seq else (H,)
    if kind == "mlp":
        inp["W0"] = (0.2 * torch.randn(*lead, d, hid, generator=g),
                     0.2 * torch.randn(*lead, hid, d, generator=g))
    else:
        inp["W0"] = (torch.eye(d) + 0.1 * torch.randn(*lead, d, d, generator=g),)
    inp["gamma"] = 1.0 + 0.2 * torch.randn(H, d, generator=g)
    inp["beta"] = 0.1 * torch.randn(H, d, generator=g)
    return inp


def _oracle_all(inp, kind, chunk, per_seq=False, **kw):
    B, H = inp["Q"].shape[:2]
    if per_seq:
        flat = flatten_heads({**inp, "W0": tuple(w[0] for w in inp["W0"])})
        flat["W0"] = tuple(w.to(torch.float64).reshape(B * H, *w.shape[2:]) for w in inp["W0"])
    else:
        flat = flatten_heads(inp)
    cfg = OracleConfig(kind=kind, chunk=chunk, **kw)
    return flat, cfg


@pytest.mark.parametrize("kind,d,chunk,T,gelu,eta_scale,per_seq", [
    ("mlp", 16, 1, 24, "erf", 1.0, False),
    ("mlp", 48, 4, 44, "tanh", 0.25, True),
    ("mlp", 64, 16, 48, "erf", 1.0 / 16, False),
    ("mlp", 128, 8, 40, "erf", 1.0, True),
    ("linear", 32, 3, 33, "erf", 1.0, False),
    ("linear", 128, 16, 32, "erf", 0.5, True),
])
def test_edge_shapes_fp32(kind, d, chunk, T, gelu, eta_scale, per_seq):
    B, H = 2, 3
    inp = _rand_case(kind, B, H, T, d, chunk, "f32", seed=d * 7 + chunk, per_seq=per_seq)
    cfg = ops.Config(kind=kind, B=B, H=H, T=T, d=d, hidden=4 * d, chunk=chunk, io="f32",
                     gelu=gelu, eta_scale=eta_scale, w0_per_seq=per_seq)
    note(f"edge {cfg}")
    res = _run(cfg, to_dev(inp), want_loss=True)
    flat, ocfg = _oracle_all(inp, kind, chunk, per_seq, gelu=gelu, eta_scale=eta_scale)
    from oracle import scan
    Z, WT, L = scan(flat["Q"], flat["K"], flat["V"], flat["eta"], flat["W0"], flat["gamma"],
                    flat["beta"], ocfg)
    assert_parity(res["Z"].reshape(B * H, T, d), Z, TOL["f32"], "Z")
    assert_parity(res["loss"].reshape(B * H, T), L, TOL["f32"], "loss", per_token=False)
    for g, o in zip(res["W_T"], WT):
        assert_parity(g.reshape(o.shape), o, TOL["f32"], "W_T", time_axis=False)


def test_eta_zero_gives_initial_map():
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    inp = make_inputs(w, batch_idx=[0, 1], head_idx=[0, 1, 2], T=64)
    inp["eta"] = torch.zeros_like(inp["eta"])
    cfg = ops_config(w, T=64, B=2, H=3)
    note("eta=0")
    res = _run(cfg, to_dev(inp))
    flat = flatten_heads(inp)
    ref = torch.stack([f_apply(flat["Q"][n], tuple(x[n:n + 1].expand(64, *x.shape[1:])
                                                   for x in flat["W0"]),
                               flat["gamma"][n], flat["beta"][n], OracleConfig())
                       for n in range(6)])
    assert_parity(res["Z"].reshape(6, 64, 64), ref, TOL["bf16"], "Z")
    for g, w0 in zip(res["W_T"], inp["W0"]):
        assert torch.equal(g.cpu(), w0.unsqueeze(0).expand(2, *w0.shape))


def test_split_scan_equals_unsplit():
    w = WORKLOADS["ttt_mlp_fp32_d16"]
    inp = make_inputs(w)
    d = to_dev(inp)
    cfg = ops_config(w)
    note("split scan")
    full = _run(cfg, d)
    half = w.T // 2
    cut = lambda x, a, b: x[:, :, a:b].contiguous()
    c2 = ops_config(w, T=half)
    r1 = _run(c2, {**d, "Q": cut(d["Q"], 0, half), "K": cut(d["K"], 0, half),
                   "V": cut(d["V"], 0, half), "eta": cut(d["eta"], 0, half)})
    c3 = ops.Config(**{**c2.__dict__, "w0_per_seq": True})
    r2 = _run(c3, {**d, "Q": cut(d["Q"], half, w.T), "K": cut(d["K"], half, w.T),
                   "V": cut(d["V"], half, w.T), "eta": cut(d["eta"], half, w.T),
                   "W0": r1["W_T"]})
    joined = torch.cat([r1["Z"], r2["Z"]], dim=2)
    assert torch.equal(joined, full["Z"])
    for a, b in zip(r2["W_T"], full["W_T"]):
        assert torch.equal(a, b)


def _tok(x, t):
    """Token t of a [B, H, T, ...] tensor in a fresh (16-byte aligned) allocation."""
    return x[:, :, t].clone()


@pytest.mark.parametrize("wid", ["ttt_mlp_fp32_d16", "ttt_linear_fp32_d64"])
def test_decode_loop_equals_scan(wid):
    w = WORKLOADS[wid]
    T = 64
    inp = make_inputs(w, batch_idx=[0], head_idx=[0, 1] if w.H > 1 else [0], T=T)
    B, H = inp["Q"].shape[:2]
    cfg = ops_config(w, T=T, B=B, H=H)
    d = to_dev(inp)
    note(f"decode loop {wid}")
    scan_res = _run(cfg, d)
    Ws = tuple(x.unsqueeze(0).expand(B, *x.shape).contiguous().clone() for x in d["W0"])
    acc = tuple(torch.zeros_like(x) for x in Ws)
    zs = []
    for t in range(T):
        zs.append(ops.decode_step(cfg, _tok(d["Q"], t), _tok(d["K"], t), _tok(d["V"], t),
                                  _tok(d["eta"], t), d["gamma"], d["beta"], Ws, acc,
                                  t % w.chunk))
    Zd = torch.stack(zs, dim=2)
    assert_parity(Zd.reshape(B * H, T, -1), scan_res["Z"].reshape(B * H, T, -1), TOL[w.io],
                  "decode loop vs scan")
    for a, b in zip(Ws, scan_res["W_T"]):
        assert rel_l2(a, b) <= TOL[w.io]
    for a in acc:
        assert torch.count_nonzero(a).item() == 0


DECODE_KERNELS = {
    "split": (dict(decode_split=True), "ttt_decode_split_d64"),
    "split_device_scope": (dict(decode_split=True, device_scope=True), "ttt_decode_split_d64"),
    "stream": (dict(), "ttt_decode_stream_d64"),
    "generic": (dict(force_generic=True), "ttt_decode_generic"),
}


@pytest.mark.parametrize("io,gelu", [("bf16", "erf"), ("f32", "tanh")])
@pytest.mark.parametrize("kernel", list(DECODE_KERNELS))
def test_decode_stream_equals_oracle(io, gelu, kernel):
    """The tuned decode kernels (MLP, d=64: one workgroup per head, and four workgroups per
    head on either exchange path) and the portable one: 48 decode steps (three commits) over
    2 x 3 heads of the d = 64 bf16 MLP workload's distributions, against the oracle scan of the
    same tokens (z of every token, the committed weights). All 48 calls share one workspace;
    the four-workgroup kernel leaves its exchange area zero after every call."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"].with_(io=io)
    T, bi, hi = 48, [0, 5], [1, 6, 11]
    inp = make_inputs(w, batch_idx=bi, head_idx=hi, T=T)
    B, H = len(bi), len(hi)
    inp["W0"] = tuple(x.unsqueeze(0).expand(B, *x.shape).contiguous() for x in inp["W0"])
    pairs = [(b, h) for b in range(B) for h in range(H)]
    sub = {**inp, "W0": tuple(x[0] for x in inp["W0"])}
    Zo, WTo, _ = oracle_heads(sub, pairs, "mlp", w.chunk, gelu=gelu)
    d = to_dev(inp)
    flags, name = DECODE_KERNELS[kernel]
    cfg = ops.Config(kind="mlp", B=B, H=H, T=T, d=64, hidden=256, chunk=16, io=io, gelu=gelu,
                     w0_per_seq=True, **flags)
    assert ops.decode_kernel_name(cfg) == name
    note(f"decode {name} ({kernel}) io={io} gelu={gelu}")
    ws = ops.new_workspace(cfg, ops.TTT_OP_DECODE, "cuda")
    Ws = tuple(x.clone() for x in d["W0"])
    acc = tuple(torch.zeros_like(x) for x in Ws)
    zs = [ops.decode_step(cfg, _tok(d["Q"], t), _tok(d["K"], t), _tok(d["V"], t),
                          _tok(d["eta"], t), d["gamma"], d["beta"], Ws, acc, t % 16, workspace=ws)
          for t in range(T)]
    assert ops.read_status(ws) == 0
    Z = torch.stack(zs, dim=2).cpu().reshape(B * H, T, 64)
    tol = TOL[io]
    assert_parity(Z, Zo, tol, f"decode Z {kernel}")
    for a, b in zip(Ws, WTo):
        assert rel_l2(a.cpu().reshape(b.shape), b) <= TOL["f32"], kernel
    for a in acc:
        assert torch.count_nonzero(a).item() == 0
    assert torch.count_nonzero(ws[256:]).item() == 0


def test_decode_full_size_both_tuned_kernels():
    """Both tuned decode kernels on all 96 heads of the d = 64 workload (the launch the
    benchmark times), one chunk of 16 calls on one workspace: each against the oracle on three
    heads, and the two against each other on every head (the partial sums are added in another
    order: fp32 rounding apart)."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    T = 16
    inp = make_inputs(w, T=T)
    d = to_dev(inp)
    pairs = [(0, 0), (3, 7), (7, 11)]
    Zo, WTo, _ = oracle_heads(inp, pairs, "mlp", w.chunk)
    out = {}
    for kernel in ("stream", "split"):
        flags, name = DECODE_KERNELS[kernel]
        cfg = ops_config(w, T=T, **flags)
        assert ops.decode_kernel_name(cfg) == name
        note(f"decode full size {name}")
        ws = ops.new_workspace(cfg, ops.TTT_OP_DECODE, "cuda")
        Ws = tuple(x.unsqueeze(0).expand(w.B, *x.shape).contiguous().clone() for x in d["W0"])
        acc = tuple(torch.zeros_like(x) for x in Ws)
        zs = [ops.decode_step(cfg, _tok(d["Q"], t), _tok(d["K"], t), _tok(d["V"], t),
                              _tok(d["eta"], t), d["gamma"], d["beta"], Ws, acc, t, workspace=ws)
              for t in range(T)]
        assert ops.read_status(ws) == 0
        Z, W = torch.stack(zs, dim=2).cpu(), tuple(x.cpu() for x in Ws)
        out[kernel] = (Z, W)
        assert_parity(torch.stack([Z[b, h] for b, h in pairs]), Zo, TOL["bf16"], f"decode Z {kernel} full size")
        for k in range(2):
            g = torch.stack([W[k][b, h] for b, h in pairs])
            assert rel_l2(g.reshape(WTo[k].shape), WTo[k]) <= TOL["f32"], kernel
    assert rel_l2(out["split"][0].float(), out["stream"][0].float()) <= 1e-2
    for a, b in zip(out["split"][1], out["stream"][1]):
        assert rel_l2(a, b) <= 1e-5


@pytest.mark.parametrize("kernel", ["split", "stream"])
def test_decode_chunk_replayed_as_graph(kernel):
    """One chunk of 16 decode calls captured into a HIP graph (through torch.cuda.graph, on the
    capture stream) and replayed three times, each replay after eager copies that reset the
    weights and the accumulator and a synchronisation: every replay equals the eager run bit
    for bit (the same kernels on the same inputs), and the exchange area stays zero."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    T, bi, hi = 16, [0, 5], [1, 6, 11]
    inp = make_inputs(w, batch_idx=bi, head_idx=hi, T=T)
    B, H = len(bi), len(hi)
    flags, name = DECODE_KERNELS[kernel]
    cfg = ops_config(w, T=T, B=B, H=H, **flags)
    assert ops.decode_kernel_name(cfg) == name
    note(f"decode graph replay {name}")
    d = to_dev(inp)
    toks = [[_tok(d[k], t) for k in ("Q", "K", "V", "eta")] for t in range(T)]
    W0 = tuple(x.unsqueeze(0).expand(B, *x.shape).contiguous() for x in d["W0"])
    ws = ops.new_workspace(cfg, ops.TTT_OP_DECODE, "cuda")
    Ws = tuple(x.clone() for x in W0)
    acc = tuple(torch.zeros_like(x) for x in Ws)
    zs = [torch.empty(B, H, 64, dtype=cfg.io_dtype, device="cuda") for _ in range(T)]

    def chunk(stream=None):
        for t in range(T):
            ops.decode_step(cfg, *toks[t][:3], toks[t][3], d["gamma"], d["beta"], Ws, acc, t,
                            z=zs[t], workspace=ws, stream=stream)

    chunk()
    torch.cuda.synchronize()
    ref_z = [z.clone() for z in zs]
    ref_w = tuple(x.clone() for x in Ws)
    g = torch.cuda.CUDAGraph()
    for x, x0 in zip(Ws, W0):
        x.copy_(x0)
    for a in acc:
        a.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        chunk(torch.cuda.current_stream())
    for rep in range(3):
        for x, x0 in zip(Ws, W0):
            x.copy_(x0)
        for a in acc:
            a.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert ops.read_status(ws) == 0
        for t in range(T):
            assert torch.equal(zs[t], ref_z[t]), (rep, t)
        for x, r in zip(Ws, ref_w):
            assert torch.equal(x, r), rep
        assert torch.count_nonzero(ws[256:]).item() == 0


@pytest.mark.parametrize("wid,kind", [("ttt_mlp_fp32_d16", "mlp"), ("ttt_linear_fp32_d64", "linear"),
                                      ("ttt_mlp_bf16_d64_T8k", "mlp")])
def test_key_output_forward_and_decode(wid, kind):
    """The Eq. 9 output rule (z_t = f(K_t; W at the chunk start)) through the forward (the
    tuned kernel for the bf16 d = 64 shape, the portable one otherwise) and the portable
    decode, against the oracle with the same rule."""
    w = WORKLOADS[wid]
    T = 64
    bi, hi = [0], ([0, 1] if w.H > 1 else [0])
    inp = make_inputs(w, batch_idx=bi, head_idx=hi, T=T)
    B, H = len(bi), len(hi)
    cfg = ops_config(w, T=T, B=B, H=H, output_key=True)
    want = "ttt_fwd_mfma_key_d64" if wid == "ttt_mlp_bf16_d64_T8k" else "ttt_fwd_generic"
    assert ops.fwd_kernel_name(cfg) == want
    note(f"key output {wid}")
    d = to_dev(inp)
    res = _run(cfg, d, want_loss=True)
    torch.cuda.synchronize()
    pairs = [(0, h) for h in range(H)]
    _check_heads(res, inp, pairs, w, TOL[w.io], cfg_kw=dict(output="key"))
    Ws = tuple(x.unsqueeze(0).expand(B, *x.shape).contiguous().clone() for x in d["W0"])
    acc = tuple(torch.zeros_like(x) for x in Ws)
    zs = [ops.decode_step(cfg, _tok(d["Q"], t), _tok(d["K"], t), _tok(d["V"], t),
                          _tok(d["eta"], t), d["gamma"], d["beta"], Ws, acc, t % w.chunk)
          for t in range(T)]
    assert_parity(torch.stack(zs, dim=2).reshape(B * H, T, -1), res["Z"].reshape(B * H, T, -1),
                  TOL[w.io], "key-output decode vs scan")
    # the decode's final memory against the oracle's, and against the scan's (the tuned bf16
    # forward rounds its update operands to bf16, the portable kernels do not)
    WTo = oracle_heads(inp, pairs, w.kind, w.chunk, output="key")[1]
    for a, b, o in zip(Ws, res["W_T"], WTo):
        assert_parity(a.reshape(o.shape), o, TOL[w.io], "key-output decode W_T", time_axis=False)
        assert rel_l2(a, b) <= TOL[w.io]


@pytest.mark.parametrize("kernel", ["tuned", "generic"])
def test_key_output_bf16_d64_T8k_sampled_heads(kernel):
    """The Eq. 9 output rule over the full launch at B=8, H=12, T=8192 (the tuned kernel: the
    paired kernel's producer alone; or the portable kernel); the oracle with the same rule checks three heads
    at full T. Under this rule the per-token loss is ||z_t - V_t||^2, which every head's device
    output must reproduce up to the bf16 rounding of z."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    cfg = ops_config(w, output_key=True, force_generic=kernel == "generic")
    want = "ttt_fwd_mfma_key_d64" if kernel == "tuned" else "ttt_fwd_generic"
    assert ops.fwd_kernel_name(cfg) == want
    note(f"key output bf16 d64 T8k full {kernel}")
    inp = make_inputs(w)
    d = to_dev(inp)
    res = _run(cfg, d, want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    _check_heads(res, inp, [(0, 0), (3, 7), (7, 11)], w, TOL["bf16"], cfg_kw=dict(output="key"))
    # the loss is the squared distance of the (unrounded) output to V
    zl = ((res["Z"].float() - d["V"].float()) ** 2).sum(-1)
    assert rel_l2(zl, res["loss"]) <= TOL["bf16"]


def test_scan_then_decode_continues_the_sequence():
    """Prefill T0 tokens with the scan, decode the rest: equals the oracle on all T."""
    w = WORKLOADS["ttt_mlp_fp32_d16"]
    T0, T = 64, 96
    inp = make_inputs(w, T=T)
    d = to_dev(inp)
    note("scan then decode")
    pre = _run(ops_config(w, T=T0), {**d, **{k: d[k][:, :, :T0].contiguous()
                                             for k in ("Q", "K", "V", "eta")}})
    cfg = ops_config(w, T=T)
    Ws = tuple(x.clone() for x in pre["W_T"])
    acc = tuple(torch.zeros_like(x) for x in Ws)
    zs = [ops.decode_step(cfg, _tok(d["Q"], t), _tok(d["K"], t), _tok(d["V"], t),
                          _tok(d["eta"], t), d["gamma"], d["beta"], Ws, acc, (t - T0) % w.chunk)
          for t in range(T0, T)]
    Z = torch.cat([pre["Z"], torch.stack(zs, dim=2)], dim=2)
    Zo, WTo, _ = oracle_heads(inp, [(0, 0)], w.kind, w.chunk)
    assert_parity(Z[0], Zo, TOL["f32"], "scan+decode Z")
    for a, b in zip(Ws, WTo):
        assert rel_l2(a[0], b) <= TOL["f32"]


@pytest.mark.parametrize("wid", ["ttt_mlp_fp32_d16", "ttt_mlp_bf16_d64_T8k"])
def test_runs_are_bitwise_deterministic(wid):
    w = WORKLOADS[wid]
    T = min(w.T, 512)
    inp = to_dev(make_inputs(w, T=T))
    cfg = ops_config(w, T=T)
    note(f"determinism {wid}")
    a = _run(cfg, inp, want_loss=True)
    b = _run(cfg, inp, want_loss=True)
    assert torch.equal(a["Z"], b["Z"]) and torch.equal(a["loss"], b["loss"])
    for x, y in zip(a["W_T"], b["W_T"]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("force_generic", [True, False])
def test_nonfinite_input_sets_status(force_generic):
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    inp = make_inputs(w, batch_idx=[0], head_idx=[0, 1], T=64)
    inp["K"][0, 1, 37, 5] = float("nan")
    cfg = ops_config(w, T=64, B=1, H=2, force_generic=force_generic)
    note(f"nan injection generic={force_generic}")
    res = _run(cfg, to_dev(inp))
    ws = res["workspace"]
    assert ops.read_status(ws) == 8
    ops.reset_status(ws)
    assert ops.read_status(ws) == 0
    clean = make_inputs(w, batch_idx=[0], head_idx=[0, 1], T=64)
    _run(cfg, to_dev(clean), workspace=ws)
    assert ops.read_status(ws) == 0


def test_debug_mode_returns_device_status(monkeypatch):
    """With TTT_DEBUG set, an entry point waits for its kernels and returns the status word's
    outcome itself: the NaN-injected forward fails with TTT_ERR_NONFINITE at the call, a clean
    one returns TTT_OK; without it the call returns TTT_OK and the status word holds the error."""
    w = WORKLOADS["ttt_mlp_bf16_d64_T8k"]
    bad = make_inputs(w, batch_idx=[0], head_idx=[0, 1], T=64)
    bad["K"][0, 0, 21, 9] = float("nan")
    clean = make_inputs(w, batch_idx=[0], head_idx=[0, 1], T=64)
    cfg = ops_config(w, T=64, B=1, H=2)
    note("TTT_DEBUG on the paired forward")
    monkeypatch.setenv("TTT_DEBUG", "1")
    with pytest.raises(ops.TTTError) as err:
        _run(cfg, to_dev(bad))
    assert err.value.code == 8
    res = _run(cfg, to_dev(clean))
    assert ops.read_status(res["workspace"]) == 0
    monkeypatch.setenv("TTT_DEBUG", "0")
    res = _run(cfg, to_dev(bad))
    assert ops.read_status(res["workspace"]) == 8


@pytest.mark.parametrize("kernel", ["pair", "split", "split_wide"])
def test_device_scope_handoff(kernel):
    """The tuned forwards with their cross-workgroup hand-offs forced onto the device-scope
    path (atomics and fences, as when the workgroups of a head sit on different XCDs): same
    kernel, status clean, every head against the oracle, and the same result as the default
    same-XCD path up to bf16 noise."""
    # split: the d = 128 kernel's producer/consumer form (3 heads); split_wide: its form with
    # both sides in every workgroup (40 heads, more than one launch of the other form holds;
    # drift-free inputs, see test_split_forms_at_the_launch_boundary)
    if kernel == "pair":
        w, (B, H, T) = WORKLOADS["ttt_mlp_bf16_d64_T8k"], (2, 5, 96)
    elif kernel == "split":
        w, (B, H, T) = WORKLOADS["ttt_mlp_bf16_d128_T128k"], (1, 3, 64)
    else:
        w, (B, H, T) = WORKLOADS["ttt_mlp_bf16_d128_T128k"].with_(drift=0.0, B=5, H=8), (5, 8, 32)
    inp = make_inputs(w, batch_idx=list(range(B)), head_idx=list(range(H)), T=T)
    cfg = ops_config(w, B=B, H=H, T=T, device_scope=True)
    name = "ttt_fwd_mfma_pair_d64" if kernel == "pair" else "ttt_fwd_mfma_split_d128"
    assert ops.fwd_kernel_name(cfg) == name
    note(f"device-scope hand-off {name} B={B} H={H} T={T}")
    d = to_dev(inp)
    res = _run(cfg, d, want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    pairs = [(b, h) for b in range(B) for h in range(H)]
    _check_heads(res, inp, pairs if kernel != "split_wide" else [(0, 0), (2, 3), (4, 7)], w, TOL["bf16"])
    ref = _run(ops_config(w, B=B, H=H, T=T), d)
    torch.cuda.synchronize()
    # the two paths move the same values; only the hand-off mechanism differs
    assert torch.equal(res["Z"], ref["Z"])
