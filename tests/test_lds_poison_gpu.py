"""Parity cases of every kernel family run on the LDS-poisoning test build (libttt_poison.so,
the same sources compiled with -DTTT_LDS_POISON: each kernel fills its LDS with all-ones words,
a NaN as fp32 and as bf16, before anything else touches it). A kernel that reads LDS it did
not write first (a missing barrier, a wrong index, unwritten padding fed to a product) turns
its outputs non-finite there and fails the same oracle comparison it passes on libttt.so.
Each case is an existing parity test, called with the binding switched to the test build."""
import os

import pytest

import test_bwd_gpu
import test_lact_gpu
import test_large_chunk_gpu
import test_momentum_gpu
import test_parity_gpu
from test_weight_sequence_amd import ops
from test_weight_sequence_amd.build import LIB_POISON

pytestmark = pytest.mark.gpu

P, M, B, L, LC = test_parity_gpu, test_momentum_gpu, test_bwd_gpu, test_lact_gpu, test_large_chunk_gpu
CASES = [
    ("pair_fwd", P.test_mlp_bf16_d64_all_heads_short, ("pair",)),
    ("pair_fwd_partial_groups", P.test_pair_partial_groups_all_heads, (2, 3, 16)),
    ("one_wg_fwd", P.test_mlp_bf16_d64_all_heads_short, ("one_wg",)),
    ("portable_fwd_bf16", P.test_mlp_bf16_d64_all_heads_short, ("generic",)),
    ("portable_fwd_f32_mlp", P.test_edge_shapes_fp32, ("mlp", 48, 4, 44, "tanh", 0.25, True)),
    ("portable_fwd_f32_linear", P.test_edge_shapes_fp32, ("linear", 32, 3, 33, "erf", 1.0, False)),
    ("key_output_fwd", P.test_key_output_tuned_variants, (2, 3, 160, "tanh", True)),
    ("split_d128_fwd", P.test_mlp_bf16_d128_reduced_T, ("split",)),
    ("large_chunk_fwd", LC.test_large_chunk_all_heads, (64,)),
    ("decode_stream", P.test_decode_stream_equals_oracle, ("bf16", "erf", "stream")),
    ("decode_split", P.test_decode_stream_equals_oracle, ("bf16", "erf", "split")),
    ("decode_portable", P.test_decode_stream_equals_oracle, ("f32", "tanh", "generic")),
    ("momentum_mfma", M.test_momentum_scan_matches_oracle, ("ttt_mlp_bf16_d64_T8k", 2, 5, 256, None, "mfma")),
    ("momentum_portable", M.test_momentum_scan_matches_oracle, ("ttt_mlp_fp32_d16", 1, 1, 256, 5, "generic")),
    ("bwd_split", B.test_bwd_mlp_bf16_d64_shape, (64, "split")),
    ("bwd_one_wg", B.test_bwd_mlp_bf16_d64_shape, (64, "one_wg")),
    ("bwd_portable", B.test_bwd_fp32_matches_oracle_autograd, ("mlp", 16, 4, 24, True, False, "tanh")),
    ("lact", L.test_lact_small, (64, 192, False, True, 0.5)),
    ("lact_read_before", L.test_lact_small, (128, 256, True, False, 1.0)),
]


@pytest.mark.parametrize("fn,args", [c[1:] for c in CASES], ids=[c[0] for c in CASES])
def test_parity_with_poisoned_lds(fn, args):
    if not os.path.exists(LIB_POISON):
        pytest.skip("the LDS-poisoning test build is missing: python -m test_weight_sequence_amd.build --poison")
    with ops.library(LIB_POISON):
        fn(*args)
