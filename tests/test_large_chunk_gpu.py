"""GPU parity of the scan with mini-batches larger than 16 tokens (b = 32 ... 1024; the
large-chunk regime of the page "Test-Time Training(TTT)과 LLM 메모리", section "LaCT", applied
to the same TTT-MLP layer and loss): the paired d = 64 kernel against the fp64 oracle with the
same mini-batch size, on the d = 64 bf16 workload's inputs."""
import pytest
import torch

from helpers import TOL, assert_parity, note, oracle_heads, ops_config, to_dev
from oracle import OracleConfig, scan as oracle_scan
from test_weight_sequence_amd import ops
from test_weight_sequence_amd.synth import WORKLOADS, flatten_heads, make_inputs

pytestmark = pytest.mark.gpu

W = WORKLOADS["ttt_mlp_bf16_d64_T8k"]


def _run(cfg, d, **kw):
    res = ops.scan_fwd(cfg, d["Q"], d["K"], d["V"], d["eta"], d["W0"], d["gamma"], d["beta"], **kw)
    torch.cuda.synchronize()
    assert ops.read_status(res["workspace"]) == 0
    return res


def _check(res, inp, pairs, chunk, tol=TOL["bf16"], **cfg_kw):
    Z, WT, L = oracle_heads(inp, pairs, "mlp", chunk, **cfg_kw)
    gz = torch.stack([res["Z"][b, h] for b, h in pairs]).cpu()
    assert_parity(gz, Z, tol, f"Z b={chunk}")
    for k, wt in enumerate(WT):
        g = torch.stack([res["W_T"][k][b, h] for b, h in pairs]).cpu()
        assert_parity(g, wt, tol, f"W_T[{k}] b={chunk}", time_axis=False)
    if res.get("loss") is not None:
        gl = torch.stack([res["loss"][b, h] for b, h in pairs]).cpu()
        assert_parity(gl, L, tol, f"loss b={chunk}", per_token=False)


@pytest.mark.parametrize("chunk", [32, 64, 256, 1024])
def test_large_chunk_all_heads(chunk):
    """Two sequences x three heads of the workload, T = 2048 (two to 64 mini-batches), every
    head against the oracle at the same mini-batch size."""
    B, H, T = 2, 3, 2048
    inp = make_inputs(W, batch_idx=[0, 5], head_idx=[1, 4, 10], T=T)
    cfg = ops_config(W, B=B, H=H, T=T, chunk=chunk)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_pair_d64"
    note(f"large chunk b={chunk} B={B} H={H} T={T}")
    res = _run(cfg, to_dev(inp), want_loss=True)
    _check(res, inp, [(b, h) for b in range(B) for h in range(H)], chunk)


@pytest.mark.parametrize("wid", ["ttt_mlp_bf16_d64_T8k_b256", "ttt_mlp_bf16_d64_T8k_b1024"])
def test_large_chunk_full_size_sampled_heads(wid):
    """The full B=8 H=12 T=8192 launch at b = 256 and 1024 (the configuration the benchmark
    times); the oracle checks three heads at full length."""
    w = WORKLOADS[wid]
    cfg = ops_config(w)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_pair_d64"
    note(f"large chunk full size {wid}")
    inp = make_inputs(w)
    res = _run(cfg, to_dev(inp), want_loss=True)
    _check(res, inp, [(0, 0), (3, 7), (7, 11)], w.chunk)


def test_large_chunk_tanh_per_seq_scaled():
    """tanh GELU, per-sequence W0, eta_scale = 1/b and a head count that leaves most of the last
    group of eight pairs empty, every head against the oracle."""
    B, H, T, b = 1, 3, 512, 128
    g = torch.Generator().manual_seed(21)
    inp = make_inputs(W, batch_idx=[2], head_idx=[0, 3, 6], T=T)
    inp["W0"] = tuple(x.unsqueeze(0) + 0.05 * torch.randn((1,) + x.shape, generator=g) for x in inp["W0"])
    cfg = ops.Config(kind="mlp", B=B, H=H, T=T, d=64, hidden=256, chunk=b, io="bf16", gelu="tanh",
                     w0_per_seq=True, eta_scale=1.0 / b)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_pair_d64"
    note("large chunk tanh per-seq eta_scale=1/b")
    res = _run(cfg, to_dev(inp))
    flat = flatten_heads({**inp, "W0": tuple(x[0] for x in inp["W0"])})
    flat["W0"] = tuple(x.double().reshape(B * H, *x.shape[2:]) for x in inp["W0"])
    Z, WT, _ = oracle_scan(flat["Q"], flat["K"], flat["V"], flat["eta"], flat["W0"], flat["gamma"],
                           flat["beta"], OracleConfig(kind="mlp", chunk=b, gelu="tanh", eta_scale=1.0 / b))
    assert_parity(res["Z"].reshape(B * H, T, 64), Z, TOL["bf16"], "Z")
    for x, o in zip(res["W_T"], WT):
        assert_parity(x.reshape(o.shape), o, TOL["bf16"], "W_T", time_axis=False)


def test_large_chunk_saved_weights_and_split():
    """The saved buffer holds W0 at mini-batch 0 and, at mini-batch 2, the W_T of a scan over
    the first two mini-batches (bitwise: the same kernel and update order); a scan split at a
    mini-batch boundary equals the whole scan up to bf16 rounding (not bitwise: the whole scan
    enters the third mini-batch through the look-ahead and its correction, the split one
    converts the carried weights directly)."""
    b, T = 64, 256
    inp = to_dev(make_inputs(W, batch_idx=[0, 1], head_idx=[3, 9], T=T))
    cfg = ops_config(W, B=2, H=2, T=T, chunk=b)
    note("large chunk saved weights")
    full = _run(cfg, inp, want_saved=True)
    nW1 = 64 * 256
    sv = full["saved"].view(2, 2, T // b, 2 * nW1).cpu()
    for bb in range(2):
        for h in range(2):
            assert torch.equal(sv[bb, h, 0, :nW1], inp["W0"][0][h].cpu().reshape(-1))
    cut = lambda a, z: {**inp, **{k: inp[k][:, :, a:z].contiguous() for k in ("Q", "K", "V", "eta")}}
    pre = _run(ops_config(W, B=2, H=2, T=2 * b, chunk=b), cut(0, 2 * b))
    assert torch.equal(sv[:, :, 2, :nW1], pre["W_T"][0].reshape(2, 2, -1).cpu())
    assert torch.equal(sv[:, :, 2, nW1:], pre["W_T"][1].reshape(2, 2, -1).cpu())
    rest = _run(ops_config(W, B=2, H=2, T=T - 2 * b, chunk=b, w0_per_seq=True),
                {**cut(2 * b, T), "W0": pre["W_T"]})
    joined = torch.cat([pre["Z"], rest["Z"]], dim=2)
    assert_parity(joined.reshape(4, T, 64), full["Z"].reshape(4, T, 64), TOL["bf16"], "split vs whole")
    assert torch.equal(joined[:, :, :2 * b], full["Z"][:, :, :2 * b])
    for x, y in zip(rest["W_T"], full["W_T"]):
        assert_parity(x.reshape(4, -1), y.reshape(4, -1), TOL["bf16"], "W_T split vs whole", time_axis=False)


def test_large_chunk_scan_then_decode():
    """Prefill with the scan at b = 64, then decode the next 64 tokens one at a time (the
    streaming decode kernel, committing at the mini-batch end): equals the oracle on all
    tokens."""
    b, T0, T = 64, 128, 192
    inp = make_inputs(W, batch_idx=[4], head_idx=[2, 8], T=T)
    d = to_dev(inp)
    pre = _run(ops_config(W, B=1, H=2, T=T0, chunk=b),
               {**d, **{k: d[k][:, :, :T0].contiguous() for k in ("Q", "K", "V", "eta")}})
    cfg = ops_config(W, B=1, H=2, T=T, chunk=b)
    assert ops.decode_kernel_name(cfg) == "ttt_decode_stream_d64"
    note("large chunk scan then decode")
    Ws = tuple(x.clone() for x in pre["W_T"])
    acc = tuple(torch.zeros_like(x) for x in Ws)
    zs = [ops.decode_step(cfg, d["Q"][:, :, t].clone(), d["K"][:, :, t].clone(), d["V"][:, :, t].clone(),
                          d["eta"][:, :, t].clone(), d["gamma"], d["beta"], Ws, acc, (t - T0) % b)
          for t in range(T0, T)]
    torch.cuda.synchronize()
    Z = torch.cat([pre["Z"], torch.stack(zs, dim=2)], dim=2)
    Zo, WTo, _ = oracle_heads(inp, [(0, 0), (0, 1)], "mlp", b)
    assert_parity(Z[0].cpu(), Zo, TOL["bf16"], "scan+decode Z")
    for a, o in zip(Ws, WTo):
        assert_parity(a[0].cpu(), o, TOL["bf16"], "W", time_axis=False)


def test_large_chunk_bitwise_deterministic():
    inp = to_dev(make_inputs(W, batch_idx=[0], head_idx=[0, 1, 2], T=1024))
    cfg = ops_config(W, B=1, H=3, T=1024, chunk=256)
    note("large chunk determinism")
    a = _run(cfg, inp, want_loss=True)
    b = _run(cfg, inp, want_loss=True)
    assert torch.equal(a["Z"], b["Z"]) and torch.equal(a["loss"], b["loss"])


@pytest.mark.parametrize("chunk,T", [(32, 512), (256, 1024), (1024, 2048)])
def test_large_chunk_key_output(chunk, T):
    """The key-side output rule (z_t = f(K_t; W at the mini-batch start)) with large
    mini-batches on the key-output kernel (the producer alone), 144 heads (above the paired
    kernel's head limit) of which six are checked at full T."""
    B, H = 9, 16
    inp = make_inputs(W, batch_idx=list(range(B)), head_idx=list(range(H)), T=T)
    cfg = ops_config(W, B=B, H=H, T=T, chunk=chunk, output_key=True)
    assert ops.fwd_kernel_name(cfg) == "ttt_fwd_mfma_key_d64"
    note(f"large chunk key output b={chunk} B={B} H={H} T={T}")
    res = _run(cfg, to_dev(inp), want_loss=True)
    _check(res, inp, [(0, 0), (2, 5), (4, 9), (6, 13), (8, 15), (8, 0)], chunk, output="key")
