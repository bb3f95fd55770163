"""C-ABI tests that need no GPU: the library loads, exports every function that
include/ttt.h declares, and its host-side validation rejects bad arguments before
anything is enqueued (no HIP call is made on these paths)."""
import ctypes
import os
import re

import pytest

from test_weight_sequence_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "ttt.h")) as fh:
        src = fh.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = ops.lib()
    names = _declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(ops.EXPORTS) <= set(names)


def test_abi_version_and_status_strings():
    L = ops.lib()
    assert L.ttt_abi_version() == 1
    for code in range(11):
        assert L.ttt_status_str(code).decode() != "unknown status"
    assert L.ttt_status_str(99).decode() == "unknown status"


def mlp_d64(**kw):
    base = dict(kind="mlp", B=8, H=12, T=8192, d=64, hidden=256, chunk=16, io="bf16")
    base.update(kw)
    return ops.Config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(kind="linear", io="f32"), 0),
    (dict(d=16, hidden=64, io="f32"), 0),
    (dict(d=128, hidden=512), 0),
    (dict(T=8200), 2),               # T not a multiple of the chunk
    (dict(B=0), 2),
    (dict(T=0), 2),
    (dict(hidden=128), 4),           # MLP hidden must be 4d
    (dict(d=8, hidden=32), 4),
    (dict(d=144, hidden=576), 4),
    (dict(d=40, hidden=160), 4),     # not a multiple of 16
    (dict(chunk=32), 0),             # larger mini-batches: the paired d=64 bf16 kernel
    (dict(chunk=1024, T=8192), 0),
    (dict(chunk=24), 4),             # above 16 only multiples of 16
    (dict(chunk=2048), 4),           # at most 1024
    (dict(chunk=32, io="f32"), 4),   # no other kernel takes mini-batches above 16
    (dict(chunk=32, B=16), 4),       # more heads than the paired kernel's 128
    (dict(chunk=32, force_generic=True), 4),
    (dict(chunk=32, one_wg_per_head=True), 4),
    (dict(chunk=0), 2),
    (dict(ln_eps=-1.0), 9),
    (dict(ln_eps=float("nan")), 9),
    (dict(eta_scale=float("inf")), 9),
])
def test_validate(kw, code):
    assert ops.validate(mlp_d64(**kw)) == code


def test_validate_bad_enums_and_flags():
    L = ops.lib()
    c = mlp_d64().c()
    c.io_dtype = 7
    assert L.ttt_validate(ctypes.byref(c)) == 3
    c = mlp_d64().c()
    c.kind = 5
    assert L.ttt_validate(ctypes.byref(c)) == 4
    c = mlp_d64().c()
    c.gelu = 3
    assert L.ttt_validate(ctypes.byref(c)) == 4
    c = mlp_d64().c()
    c.flags = 1 << 7
    assert L.ttt_validate(ctypes.byref(c)) == 9
    assert L.ttt_validate(None) == 1


def test_workspace_and_saved_sizes():
    c = mlp_d64()
    # decode: the status word, plus the exchange area of the four-workgroup kernel (4352 B per
    # head, heads rounded up to a multiple of 8) where it runs
    assert ops.workspace_size(c, ops.TTT_OP_DECODE) == 256
    assert ops.workspace_size(mlp_d64(decode_split=True), ops.TTT_OP_DECODE) == 256 + 96 * 4352
    assert ops.workspace_size(mlp_d64(B=1, H=3, decode_split=True), ops.TTT_OP_DECODE) == 256 + 8 * 4352
    assert ops.workspace_size(mlp_d64(B=16, decode_split=True), ops.TTT_OP_DECODE) == 256
    gen = ops.workspace_size(ops.Config(**{**c.__dict__, "force_generic": True}))
    assert gen == 256 + 8 * 12 * 2 * 64 * 256 * 4
    # key-side output rule: the tuned kernel needs the status word only
    assert ops.workspace_size(mlp_d64(output_key=True)) == 256
    assert ops.workspace_size(c, ops.TTT_OP_BWD) > 256
    assert ops.saved_size(c) == 8 * 12 * 512 * 2 * 64 * 256 * 4
    lin = ops.Config(kind="linear", B=4, H=12, T=2048, d=64, io="f32", force_generic=True)
    assert ops.workspace_size(lin) == 256 + 48 * 64 * 64 * 4
    with pytest.raises(ops.TTTError):
        ops.workspace_size(c, 17)
    with pytest.raises(ops.TTTError):
        ops.workspace_size(mlp_d64(T=3))


def test_kernel_selection_names():
    assert ops.fwd_kernel_name(mlp_d64(force_generic=True)) == "ttt_fwd_generic"
    assert ops.fwd_kernel_name(mlp_d64(io="f32")) == "ttt_fwd_generic"
    assert ops.fwd_kernel_name(mlp_d64(T=7)) == ""
    assert ops.bwd_kernel_name(mlp_d64(io="f32")) == "ttt_bwd_generic"
    assert ops.bwd_kernel_name(mlp_d64(T=7)) == ""
    assert ops.bwd_kernel_name(mlp_d64()) == "ttt_bwd_mfma_split_d64"
    assert ops.bwd_kernel_name(mlp_d64(one_wg_per_head=True)) == "ttt_bwd_mfma_d64"
    assert ops.decode_kernel_name(mlp_d64()) == "ttt_decode_stream_d64"
    assert ops.decode_kernel_name(mlp_d64(decode_split=True)) == "ttt_decode_split_d64"
    assert ops.decode_kernel_name(mlp_d64(B=16, decode_split=True)) == "ttt_decode_stream_d64"  # 192 heads
    assert ops.decode_kernel_name(mlp_d64(io="f32", decode_split=True)) == "ttt_decode_split_d64"
    assert ops.decode_kernel_name(mlp_d64(force_generic=True)) == "ttt_decode_generic"
    # the Eq. 9 output rule: a tuned forward (the paired kernel's producer alone, one
    # workgroup per head, any head count), the rest on the portable kernels
    assert ops.fwd_kernel_name(mlp_d64(output_key=True)) == "ttt_fwd_mfma_key_d64"
    assert ops.fwd_kernel_name(mlp_d64(output_key=True, one_wg_per_head=True)) == "ttt_fwd_mfma_key_d64"
    assert ops.fwd_kernel_name(mlp_d64(output_key=True, B=64)) == "ttt_fwd_mfma_key_d64"
    assert ops.fwd_kernel_name(mlp_d64(output_key=True, io="f32")) == "ttt_fwd_generic"
    assert ops.fwd_kernel_name(mlp_d64(output_key=True, force_generic=True)) == "ttt_fwd_generic"
    # ... and with mini-batches above 16 tokens (any head count); no decode or backward there
    assert ops.fwd_kernel_name(mlp_d64(output_key=True, chunk=256)) == "ttt_fwd_mfma_key_d64"
    assert ops.fwd_kernel_name(mlp_d64(output_key=True, chunk=1024, B=64)) == "ttt_fwd_mfma_key_d64"
    assert ops.fwd_kernel_name(mlp_d64(output_key=True, chunk=256, one_wg_per_head=True)) == "ttt_fwd_mfma_key_d64"
    assert ops.workspace_size(mlp_d64(output_key=True, chunk=256)) == 256
    assert ops.decode_kernel_name(mlp_d64(output_key=True, chunk=256)) == ""
    assert ops.bwd_kernel_name(mlp_d64(output_key=True, chunk=256)) == ""
    assert ops.fwd_kernel_name(mlp_d64(output_key=True, chunk=256, force_generic=True)) == ""
    assert ops.bwd_kernel_name(mlp_d64(output_key=True)) == "ttt_bwd_generic"
    assert ops.decode_kernel_name(mlp_d64(output_key=True)) == "ttt_decode_generic"
    assert ops.validate(mlp_d64(output_key=True)) == 0
    # the momentum variant: the tuned kernel for the d=64 bf16 shape, the portable one otherwise
    assert ops.fwd_momentum_kernel_name(mlp_d64()) == "ttt_fwd_mfma_mom_d64"
    assert ops.fwd_momentum_kernel_name(mlp_d64(force_generic=True)) == "ttt_fwd_generic"
    assert ops.fwd_momentum_kernel_name(mlp_d64(io="f32")) == "ttt_fwd_generic"
    assert ops.fwd_momentum_kernel_name(mlp_d64(d=128, hidden=512)) == "ttt_fwd_generic"
    assert ops.fwd_momentum_kernel_name(mlp_d64(output_key=True)) == ""
    assert ops.fwd_momentum_kernel_name(mlp_d64(chunk=256)) == ""
    # mini-batches above 16 tokens: forward on the paired kernel, decode on the tuned decode
    # kernels, no backward
    assert ops.fwd_kernel_name(mlp_d64(chunk=256)) == "ttt_fwd_mfma_pair_d64"
    assert ops.decode_kernel_name(mlp_d64(chunk=256)) == "ttt_decode_stream_d64"
    assert ops.decode_kernel_name(mlp_d64(chunk=256, decode_split=True)) == "ttt_decode_split_d64"
    assert ops.decode_kernel_name(mlp_d64(chunk=256, one_wg_per_head=True)) == ""
    assert ops.bwd_kernel_name(mlp_d64(chunk=256)) == ""
    with pytest.raises(ops.TTTError):
        ops.workspace_size(mlp_d64(chunk=256), ops.TTT_OP_BWD)
    with pytest.raises(ops.TTTError):
        ops.workspace_size(mlp_d64(chunk=256), ops.TTT_OP_FWD_MOMENTUM)
    assert ops.saved_size(mlp_d64(chunk=256)) == 8 * 12 * 32 * 2 * 64 * 256 * 4


class _FakeTensor:
    """Stands in for a device tensor: only data_ptr() is read, and every call below is
    rejected by host validation before any pointer could be dereferenced."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr

    def numel(self):
        return 1 << 40


def _fwd_call(cfg, ptrs, ws_bytes=1 << 40, W0=(0x10000, 0x20000)):
    L = ops.lib()
    P = ctypes.c_void_p
    w = ctypes.byref(ops.CWeights(*W0))
    return L.ttt_scan_fwd(ctypes.byref(cfg.c()), *[P(x) for x in ptrs], w, P(0x80000), None,
                          None, None, P(0x90000), ws_bytes, None)


def test_fwd_rejects_null_misaligned_and_small_workspace():
    c = mlp_d64()
    good = [0x1000 * (i + 1) for i in range(6)]
    assert _fwd_call(c, [0] + good[1:]) == 1
    assert _fwd_call(c, good, W0=(0x10000, 0)) == 1
    assert _fwd_call(c, [0x1008] + good[1:]) == 5
    assert _fwd_call(c, good, ws_bytes=16) == 6
    assert _fwd_call(mlp_d64(T=17), good) == 2


def test_decode_rejects_bad_position():
    L = ops.lib()
    P = ctypes.c_void_p
    c = mlp_d64()
    w = ctypes.byref(ops.CWeights(0x10000, 0x20000))
    args = [P(0x1000 * (i + 1)) for i in range(6)]
    for pos in (-1, 16):
        assert L.ttt_decode_step(ctypes.byref(c.c()), *args, w, w, pos, P(0x70000), P(0x90000),
                                 256, None) == 9
    assert L.ttt_decode_step(ctypes.byref(c.c()), *args, w, w, 3, P(0x70000), None, 256,
                             None) == 6
    # the four-workgroup kernel's exchange area must fit in the workspace
    cs = mlp_d64(decode_split=True)
    need = ops.workspace_size(cs, ops.TTT_OP_DECODE)
    assert L.ttt_decode_step(ctypes.byref(cs.c()), *args, w, w, 3, P(0x70000), P(0x90000),
                             need - 16, None) == 6


def test_bwd_rejects_missing_saved_buffer():
    L = ops.lib()
    P = ctypes.c_void_p
    c = mlp_d64()
    w = ctypes.byref(ops.CWeights(0x10000, 0x20000))
    args = [P(0x1000 * (i + 1)) for i in range(6)]
    code = L.ttt_scan_bwd(ctypes.byref(c.c()), *args, None, P(0x40000), None, P(0x50000),
                          P(0x60000), P(0x70000), P(0x71000), w, None, None, P(0x90000),
                          1 << 40, None)
    assert code == 1


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "_LIB_PATH", "/nonexistent/libttt.so")
    with pytest.raises(RuntimeError, match="missing"):
        ops.lib()


def test_momentum_fwd_checks_before_launch():
    """ttt_scan_fwd_momentum: null, alignment, workspace and unsupported-flag errors are
    reported on the host, before anything is enqueued (fake device addresses, no GPU)."""
    L = ops.lib()
    P = ctypes.c_void_p
    c = mlp_d64()
    need = ops.workspace_size(c, ops.TTT_OP_FWD_MOMENTUM)
    assert need >= 256 + c.B * c.H * 2 * 2 * c.d * c.hidden * 4
    w = ctypes.byref(ops.CWeights(0x10000, 0x20000))

    def call(cfg, first=0x1000, ws=need, ws_ptr=0x90000):
        args = [P(first)] + [P(0x1000 * (i + 2)) for i in range(7)]  # Q K V theta mom alpha gamma beta
        return L.ttt_scan_fwd_momentum(ctypes.byref(cfg.c()), *args, w, None, P(0x70000), w, w, None,
                                       P(ws_ptr), ws, None)
    assert call(c, first=0) == 1                    # TTT_ERR_NULL
    assert call(c, first=0x1008) == 5               # TTT_ERR_ALIGN
    assert call(c, ws=need - 16) == 6               # TTT_ERR_WORKSPACE
    assert call(c, ws_ptr=0) == 6
    assert call(mlp_d64(T=17)) == 2                 # TTT_ERR_SHAPE
    assert call(mlp_d64(output_key=True)) == 4      # TTT_ERR_UNSUPPORTED


def test_static_fwd_checks_before_launch():
    """ttt_scan_fwd_static: null, alignment and shape errors, and a configuration whose
    workspace exceeds the library's 16 MiB device array, are reported on the host before any
    HIP call (fake device addresses, no GPU)."""
    L = ops.lib()
    P = ctypes.c_void_p
    w = ctypes.byref(ops.CWeights(0x10000, 0x20000))

    def call(cfg, first=0x1000, status=None):
        args = [P(first)] + [P(0x1000 * (i + 2)) for i in range(5)]  # Q K V eta gamma beta
        return L.ttt_scan_fwd_static(ctypes.byref(cfg.c()), *args, w, P(0x80000), None, None, None,
                                     P(status) if status else None, None)
    assert call(mlp_d64(), first=0) == 1                  # TTT_ERR_NULL
    assert call(mlp_d64(), first=0x1008) == 5             # TTT_ERR_ALIGN
    assert call(mlp_d64(), status=0x90002) == 5           # status word not 4-byte aligned
    assert call(mlp_d64(T=17)) == 2                       # TTT_ERR_SHAPE
    # 32 heads of the d=128 shape: the portable fallback's per-head weights alone are 16 MiB
    big = ops.Config(kind="mlp", B=1, H=32, T=64, d=128, hidden=512, chunk=16, io="bf16")
    assert ops.workspace_size(big) > 16 << 20
    assert call(big) == 6                                 # TTT_ERR_WORKSPACE
    # the paired kernel's largest launch (128 heads) fits
    assert ops.workspace_size(mlp_d64(B=8, H=16)) <= 16 << 20


def test_lact_configuration_checks():
    """The large-chunk SwiGLU layer's host checks (ttt_validate and its workspace size)."""
    cfg = ops.Config(kind="swiglu", B=2, H=3, T=256, d=64, hidden=256, chunk=64)
    assert ops.validate(cfg) == 0
    heads = 6
    assert ops.workspace_size(cfg, ops.TTT_OP_LACT) == 256 + heads * (2 * 3 * 64 * 256 + 2 * 2 * 64) * 4
    bad = lambda **kw: ops.validate(ops.Config(**{**cfg.__dict__, **kw}))
    assert bad(chunk=48, T=240) == 4               # chunk not a multiple of 64
    assert bad(T=250) == 2                         # T not a multiple of chunk
    assert bad(io="f32") == 4
    assert bad(d=128, hidden=512) == 4
    assert bad(hidden=128) == 4
    assert bad(force_generic=True) == 9            # not a flag of this layer
    assert bad(eta_scale=float("nan")) == 9
    assert bad(read_before=True, w0_per_seq=True) == 0
    # the other entry points do not take this kind, and this op does not take theirs
    with pytest.raises(ops.TTTError):
        ops.workspace_size(cfg, ops.TTT_OP_FWD)
    with pytest.raises(ops.TTTError):
        ops.workspace_size(mlp_d64(), ops.TTT_OP_LACT)
    assert ops.fwd_kernel_name(cfg) == ""
    assert ops.validate(mlp_d64(read_before=True)) == 9
