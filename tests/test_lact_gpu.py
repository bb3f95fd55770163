"""GPU parity of the large-chunk SwiGLU layer (ttt_lact_fwd: "Test-Time Training(TTT)과 LLM
메모리", section "LaCT", Eq. 6/7/4/8/2) against the fp64 oracle scan_lact on the same seeded
inputs: Z over the whole tensor, each head, each 16 tokens and each token, and W_T, at the
bf16 tolerance (2e-2 relative L2; the kernel's products take bf16 operands)."""
import pytest
import torch

from helpers import TOL, assert_parity, note, rel_l2, to_dev
from oracle import scan_lact
from test_weight_sequence_amd import ops
from test_weight_sequence_amd.synth import WORKLOADS, flatten_heads, make_inputs

pytestmark = pytest.mark.gpu

W = WORKLOADS["lact_swiglu_bf16_d64_T8k_b2048"]


def _config(B, H, T, chunk, **kw):
    return ops.Config(kind="swiglu", B=B, H=H, T=T, d=64, hidden=256, chunk=chunk, io="bf16", **kw)


def _per_seq(inp):
    """W0 [H, ...] -> [B, H, ...] with every sequence's own copy perturbed differently, so a
    kernel that read the shared copy would fail."""
    B = inp["Q"].shape[0]
    g = torch.Generator().manual_seed(7)
    return tuple((w.unsqueeze(0).expand(B, *w.shape) *
                  (1.0 + 0.1 * torch.randn(B, *w.shape, generator=g))).contiguous() for w in inp["W0"])


def _oracle(inp, chunk, eta_scale=1.0, read_before=False, W0=None):
    flat = flatten_heads(inp)
    if W0 is not None:
        flat["W0"] = tuple(w.to(torch.float64).reshape(-1, *w.shape[2:]) for w in W0)
    return scan_lact(flat["Q"], flat["K"], flat["V"], flat["eta"], flat["W0"], chunk,
                     eta_scale=eta_scale, apply="before" if read_before else "after")


def _run(cfg, d, W0=None):
    return ops.lact_fwd(cfg, d["Q"], d["K"], d["V"], d["eta"], W0 if W0 is not None else d["W0"])


def _check(res, Zo, WTo, N):
    Z = res["Z"].reshape(N, -1, 64).cpu()
    assert_parity(Z, Zo, TOL["bf16"], "Z")
    for k, (g, o) in enumerate(zip(res["W_T"], WTo)):
        assert_parity(g.reshape(o.shape).cpu(), o, TOL["bf16"], f"W_T[{k}]", time_axis=False)


@pytest.mark.parametrize("chunk,T,read_before,per_seq,eta_scale", [
    (64, 256, False, False, 1.0),
    (128, 256, True, False, 1.0),
    (64, 192, False, True, 0.5),
    (256, 256, True, True, 1.0),
    (1024, 2048, False, False, 1.0),
])
def test_lact_small(chunk, T, read_before, per_seq, eta_scale):
    """Several heads, several chunks (or one), both read-out orders, shared or per-sequence W0."""
    B, H = 2, 3
    inp = make_inputs(W.with_(chunk=chunk), batch_idx=[0, 5], head_idx=[1, 4, 9], T=T)
    cfg = _config(B, H, T, chunk, read_before=read_before, w0_per_seq=per_seq, eta_scale=eta_scale)
    note(f"lact chunk={chunk} T={T} before={read_before} per_seq={per_seq}")
    W0 = _per_seq(inp) if per_seq else None
    d = to_dev(inp)
    res = _run(cfg, d, None if W0 is None else tuple(w.cuda() for w in W0))
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    Zo, WTo = _oracle(inp, chunk, eta_scale, read_before, W0)
    _check(res, Zo, WTo, B * H)


def test_lact_one_chunk_spans_the_sequence():
    """chunk = T = 4096: one gradient over the whole sequence (32 staging rounds per gradient
    block), then the read-out of every token with the updated weights."""
    inp = make_inputs(W.with_(chunk=4096), batch_idx=[1], head_idx=[0, 6], T=4096)
    cfg = _config(1, 2, 4096, 4096)
    note("lact chunk = T = 4096")
    res = _run(cfg, to_dev(inp))
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    Zo, WTo = _oracle(inp, 4096)
    _check(res, Zo, WTo, 2)


def test_lact_many_heads_sampled():
    """192 (batch, head) pairs (B = 16, H = 12; more than the 128 a paired launch may hold, and
    not a multiple of the block grouping per XCD in the last group), T = 512, chunks of 256;
    the oracle checks four heads spread over the grid."""
    B, H, T, chunk = 16, 12, 512, 256
    inp = make_inputs(W.with_(chunk=chunk, B=B), batch_idx=list(range(B)), T=T)
    cfg = _config(B, H, T, chunk)
    note("lact 192 heads")
    res = _run(cfg, to_dev(inp))
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    pairs = [(0, 0), (5, 11), (10, 3), (15, 7)]
    Zs, WTs = [], []
    for b, h in pairs:
        sub = make_inputs(W.with_(chunk=chunk, B=B), batch_idx=[b], head_idx=[h], T=T)
        Zo, WTo = _oracle(sub, chunk)
        Zs.append(Zo[0])
        WTs.append(WTo)
    gz = torch.stack([res["Z"][b, h] for b, h in pairs]).cpu()
    assert_parity(gz, torch.stack(Zs), TOL["bf16"], "Z")
    for k in range(3):
        g = torch.stack([res["W_T"][k][b, h] for b, h in pairs]).cpu()
        assert_parity(g, torch.stack([wt[k][0] for wt in WTs]), TOL["bf16"], f"W_T[{k}]", time_axis=False)


def test_lact_full_size_sampled_heads():
    """The full launch at B=8, H=12, T=8192, chunks of 2048; the oracle checks three heads at
    full T (heads are independent)."""
    inp = make_inputs(W)
    cfg = _config(W.B, W.H, W.T, W.chunk)
    note("lact full size")
    res = _run(cfg, to_dev(inp))
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    pairs = [(0, 0), (3, 7), (7, 11)]
    Zs, WTs = [], []
    for b, h in pairs:
        sub = make_inputs(W, batch_idx=[b], head_idx=[h])
        Zo, WTo = _oracle(sub, W.chunk)
        Zs.append(Zo[0])
        WTs.append(WTo)
    Zo = torch.stack(Zs)
    gz = torch.stack([res["Z"][b, h] for b, h in pairs]).cpu()
    assert_parity(gz, Zo, TOL["bf16"], "Z")
    for k in range(3):
        g = torch.stack([res["W_T"][k][b, h] for b, h in pairs]).cpu()
        o = torch.stack([wt[k][0] for wt in WTs])
        assert_parity(g, o, TOL["bf16"], f"W_T[{k}]", time_axis=False)


def test_lact_deterministic_and_workspace_reuse():
    """Two calls on one workspace give the same bits; the W2 column sums left in the workspace
    by the first call do not leak into the second."""
    inp = to_dev(make_inputs(W.with_(chunk=128), batch_idx=[0, 1], head_idx=list(range(12)), T=512))
    cfg = _config(2, 12, 512, 128)
    ws = ops.new_workspace(cfg, ops.TTT_OP_LACT)
    a = ops.lact_fwd(cfg, inp["Q"], inp["K"], inp["V"], inp["eta"], inp["W0"], workspace=ws)
    b = ops.lact_fwd(cfg, inp["Q"], inp["K"], inp["V"], inp["eta"], inp["W0"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a["Z"], b["Z"])
    for x, y in zip(a["W_T"], b["W_T"]):
        assert torch.equal(x, y)


def test_lact_zero_eta_keeps_w0_and_reads_it_out():
    """eta = 0: no gradient, so W_T is W0 with its units normalised, and reading before the
    update gives f_{W0}(Q) on the first chunk."""
    inp = make_inputs(W.with_(chunk=64), batch_idx=[0], head_idx=[2, 3], T=128)
    inp["eta"].zero_()
    cfg = _config(1, 2, 128, 64, read_before=True)
    res = _run(cfg, to_dev(inp))
    torch.cuda.synchronize()
    Zo, WTo = _oracle(inp, 64, read_before=True)
    _check(res, Zo, WTo, 2)
    n1 = res["W_T"][0].norm(dim=-2)
    assert rel_l2(n1, torch.ones_like(n1)) <= 1e-5

