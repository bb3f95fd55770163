"""Accuracy of the branch-free GELU used by the MFMA kernels (csrc/ttt_gelu.hpp),
compiled for the host with g++ and compared with the exact erf form in fp64.

A&S 7.1.26 bounds |erf error| by 1.5e-7, i.e. |Phi error| <= 7.5e-8; the fp32
evaluation adds a few ulp. The forward kernels' lower-order form (A&S 7.1.25) bounds
|erf error| by 2.5e-5, i.e. |Phi error| <= 1.25e-5."""
import math
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "test_weight_sequence_amd", "csrc", "ttt_gelu.hpp")

SRC = r"""
#include <cmath>
#include <cstdio>
#include "%s"
int main() {
  for (int i = -16000; i <= 16000; ++i) {
    float x = i * 0.0005f;
    float v, d1, d2;
    ttt_gelu::gelu_d2(x, v, d1, d2);
    float fv, fd1;
    ttt_gelu::gelu_d_fast(x, fv, fd1);
    std::printf("%%.9g %%.9g %%.9g %%.9g %%.9g %%.9g %%.9g %%.9g\n", x, v, d1, d2, ttt_gelu::gelu(x),
                fv, fd1, ttt_gelu::gelu_fast(x));
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def table(tmp_path_factory):
    d = tmp_path_factory.mktemp("gelu")
    src = d / "g.cpp"
    src.write_text(SRC % HDR)
    exe = d / "g"
    r = subprocess.run(["g++", "-O2", "-std=c++17", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    return np.array([[float(t) for t in ln.split()] for ln in out.strip().splitlines()])


def _exact(x):
    cdf = np.array([0.5 * math.erfc(-t / math.sqrt(2.0)) for t in x])
    pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return x * cdf, cdf + x * pdf, pdf * (2.0 - x * x)


def test_gelu_value_and_derivatives_match_exact_erf_form(table):
    x, v, d1, d2, g = table.T[:5]
    ev, ed1, ed2 = _exact(x)
    scale = np.maximum(1.0, np.abs(x))
    assert np.max(np.abs(v - ev) / scale) < 4e-7
    assert np.max(np.abs(g - ev) / scale) < 4e-7
    assert np.max(np.abs(d1 - ed1) / scale) < 4e-7
    assert np.max(np.abs(d2 - ed2) / scale ** 2) < 4e-7


def test_gelu_tails_and_sign(table):
    x, v, d1 = table.T[:3]
    assert np.all(v[x < -6] <= 0) and np.all(v[x < -6] > -1e-7)
    assert np.allclose(v[x > 6], x[x > 6], rtol=1e-7)
    assert np.allclose(d1[x > 6], 1.0, atol=1e-7)


def test_forward_gelu_within_as_7_1_25_bound(table):
    """gelu_fast / gelu_d_fast: |Phi error| <= 1.25e-5 (A&S 7.1.25), so the value is within
    1.25e-5 |x| and the derivative within 1.25e-5 (plus fp32 rounding)."""
    x = table[:, 0]
    fv, fd1, fg = table[:, 5], table[:, 6], table[:, 7]
    ev, ed1, _ = _exact(x)
    scale = np.maximum(1.0, np.abs(x))
    assert np.max(np.abs(fv - ev) / scale) < 1.3e-5
    assert np.max(np.abs(fg - ev) / scale) < 1.3e-5
    assert np.max(np.abs(fd1 - ed1) / scale) < 1.3e-5
    # the bound is not loose: the lower-order form is visibly less exact than 7.1.26
    assert np.max(np.abs(fv - ev) / scale) > 1e-6
    # sign structure: GELU(x) < 0 for x < 0, GELU(x) -> x and GELU'(x) -> 1 for large x
    assert np.all(fg[x < 0] <= 0) and np.all(fv[x < 0] <= 0)
    assert np.allclose(fg[x > 6], x[x > 6], rtol=1e-6) and np.allclose(fd1[x > 6], 1.0, atol=1e-6)
