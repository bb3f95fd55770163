"""ttt_scan_fwd_static (the forward with the library's own device workspace, for callers that
cannot allocate) against ttt_scan_fwd on the same inputs: the two run the same kernels, so the
outputs must agree bit for bit. Two calls in a row, the second smaller, for each kernel family
(paired d = 64, split d = 128, portable), and the size limit."""
import pytest
import torch

from helpers import note, ops_config, to_dev
from test_weight_sequence_amd import ops
from test_weight_sequence_amd.synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _pair(w, B, H, T):
    inp = make_inputs(w, batch_idx=list(range(B)), head_idx=list(range(H)), T=T)
    return ops_config(w, B=B, H=H, T=T), to_dev(inp)


def _both(cfg, d):
    args = (d["Q"], d["K"], d["V"], d["eta"], d["W0"], d["gamma"], d["beta"])
    ref = ops.scan_fwd(cfg, *args, want_loss=True)
    got = ops.scan_fwd_static(cfg, *args, want_loss=True)
    torch.cuda.synchronize()
    assert ops.read_status(ref["workspace"]) == 0
    assert int(got["status"].item()) == 0
    assert torch.equal(got["Z"], ref["Z"])
    assert torch.equal(got["loss"], ref["loss"])
    for a, b in zip(got["W_T"], ref["W_T"]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("wid,kernel,shapes", [
    ("ttt_mlp_bf16_d64_T8k", "ttt_fwd_mfma_pair_d64", [(2, 3, 256), (1, 2, 64)]),
    ("ttt_mlp_bf16_d128_T128k", "ttt_fwd_mfma_split_d128", [(1, 3, 96), (1, 1, 32)]),
    ("ttt_linear_fp32_d64", "ttt_fwd_generic", [(2, 3, 128), (1, 1, 48)]),
])
def test_static_fwd_equals_fwd(wid, kernel, shapes):
    w = WORKLOADS[wid]
    for B, H, T in shapes:
        cfg, d = _pair(w, B, H, T)
        assert ops.fwd_kernel_name(cfg) == kernel
        note(f"static fwd {kernel} B={B} H={H} T={T}")
        _both(cfg, d)


def test_static_fwd_rejects_oversized_workspace():
    w = WORKLOADS["ttt_mlp_bf16_d128_T128k"]
    cfg, d = _pair(w, 1, 32, 32)
    note("static fwd oversized")
    with pytest.raises(ops.TTTError) as e:
        ops.scan_fwd_static(cfg, d["Q"], d["K"], d["V"], d["eta"], d["W0"], d["gamma"], d["beta"])
    assert e.value.code == 6
