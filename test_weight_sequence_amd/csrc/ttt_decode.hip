// One decode token per (batch, head). The weights of the running chunk are kept as
// W_start (weights at the chunk start) plus acc (eta_scale * sum eta_s grad l_s(W_start)
// over the chunk's tokens so far); the output uses W_start - acc including the
// current token, exactly as the scan does, and a step commits when the chunk is
// full (E2E paper review, section 2.3.2: "take a gradient step only when the decoded
// tokens fill a mini-batch"). Memory-bound: it streams W_start and acc once or twice.
// With TTT_OUTPUT_KEY (Eq. 9 of the same review, section 2.4.2) z = f(k; W_start), the
// key-side prediction of the LayerNorm step, and q does not enter the output.
#include "ttt_device.hpp"

namespace ttt {
namespace {

constexpr int NT = kThreads;
constexpr int MAXH = 512;
constexpr int MAXD = 128;

template <typename IO, int KIND>
__global__ void __launch_bounds__(NT) decode_kernel(DecodeParams p) {
  __shared__ float sq[MAXD], sk[MAXD], sv[MAXD], sZ[MAXD], sE[MAXD];
  __shared__ float sA[MAXH], sG[MAXH], sAQ[MAXH];
  __shared__ float sPart[NT];
  __shared__ float sEta;
  TTT_POISON(sq);
  TTT_POISON(sk);
  TTT_POISON(sv);
  TTT_POISON(sZ);
  TTT_POISON(sE);
  TTT_POISON(sA);
  TTT_POISON(sG);
  TTT_POISON(sAQ);
  TTT_POISON(sPart);
  TTT_POISON(sEta);
  TTT_POISON_DONE();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x, hidx = bh % p.H;
  const int d = p.d, h = p.hid;
  const size_t nW1 = KIND == TTT_MLP ? static_cast<size_t>(d) * h : static_cast<size_t>(d) * d;
  const size_t nW2 = KIND == TTT_MLP ? static_cast<size_t>(h) * d : 0;
  float* W1 = p.ws_1 + bh * nW1;
  float* W2 = KIND == TTT_MLP ? p.ws_2 + bh * nW2 : nullptr;
  float* P1 = p.acc_1 + bh * nW1;
  float* P2 = KIND == TTT_MLP ? p.acc_2 + bh * nW2 : nullptr;
  const bool commit = p.pos == p.chunk - 1;
  const bool key_out = (p.flags & TTT_OUTPUT_KEY) != 0;
  const float* gam = p.gamma + static_cast<size_t>(hidx) * d;
  const float* bet = p.beta + static_cast<size_t>(hidx) * d;

  for (int i = tid; i < d; i += NT) {
    sq[i] = to_f32(static_cast<const IO*>(p.q)[static_cast<size_t>(bh) * d + i]);
    sk[i] = to_f32(static_cast<const IO*>(p.k)[static_cast<size_t>(bh) * d + i]);
    sv[i] = to_f32(static_cast<const IO*>(p.v)[static_cast<size_t>(bh) * d + i]);
  }
  if (tid == 0) sEta = p.eta[bh] * p.eta_scale;
  __syncthreads();

  // ---- gradient at W_start: forward of the key ----
  if (KIND == TTT_MLP) {
    for (int j = tid; j < h; j += NT) {
      float a = 0.f;
      for (int k = 0; k < d; ++k) a = fmaf(sk[k], W1[static_cast<size_t>(k) * h + j], a);
      float v, d1;
      gelu_d(a, p.gelu, v, d1);
      sA[j] = v;
      sG[j] = d1;
    }
    __syncthreads();
  }
  {
    // z^K[c] over column owners; the contraction is split across NT / d groups
    const int ngrp = NT / d, grp = tid / d, col = tid % d;
    const int n = KIND == TTT_MLP ? h : d;
    float a = 0.f;
    if (grp < ngrp) {
      for (int j = grp; j < n; j += ngrp) {
        const float x = KIND == TTT_MLP ? sA[j] : sk[j];
        const float* W = KIND == TTT_MLP ? W2 : W1;
        a = fmaf(x, W[static_cast<size_t>(j) * d + col], a);
      }
    }
    sPart[tid] = a;
    __syncthreads();
    if (tid < d) {
      float z = 0.f;
      for (int g = 0; g < ngrp; ++g) z += sPart[g * d + tid];
      sZ[tid] = z;
    }
    __syncthreads();
  }
  // ---- LayerNorm forward/backward (wave 0): E2 = eta * delta2 ----
  if (wave == 0) {
    const bool h0 = lane < d, h1 = lane + 64 < d;
    const float z0 = h0 ? sZ[lane] : 0.f, z1 = h1 ? sZ[lane + 64] : 0.f;
    const float mu = wave_sum(z0 + z1) / d;
    const float c0 = h0 ? z0 - mu : 0.f, c1 = h1 ? z1 - mu : 0.f;
    const float rs = 1.0f / sqrtf(wave_sum(c0 * c0 + c1 * c1) / d + p.eps);
    const float x0 = c0 * rs, x1 = c1 * rs;
    const float r0 = h0 ? sk[lane] + gam[lane] * x0 + bet[lane] - sv[lane] : 0.f;
    const float r1 = h1 ? sk[lane + 64] + gam[lane + 64] * x1 + bet[lane + 64] - sv[lane + 64] : 0.f;
    const float gg0 = h0 ? 2.f * r0 * gam[lane] : 0.f, gg1 = h1 ? 2.f * r1 * gam[lane + 64] : 0.f;
    const float mg = wave_sum(gg0 + gg1) / d, mgx = wave_sum(gg0 * x0 + gg1 * x1) / d;
    const float loss = wave_sum(r0 * r0 + r1 * r1);
    if (h0) sE[lane] = sEta * (gg0 - mg - x0 * mgx) * rs;
    if (h1) sE[lane + 64] = sEta * (gg1 - mg - x1 * mgx) * rs;
    if (lane == 0) flag_nonfinite(p.status, loss);
    if (key_out) {
      IO* zo = static_cast<IO*>(p.z) + static_cast<size_t>(bh) * d;
      if (h0) zo[lane] = from_f32<IO>(r0 + sv[lane]);
      if (h1) zo[lane + 64] = from_f32<IO>(r1 + sv[lane + 64]);
    }
  }
  __syncthreads();

  if (KIND == TTT_MLP) {
    // E1 = (E2 W2^T) (.) G
    for (int j = tid; j < h; j += NT) {
      float a = 0.f;
      for (int c = 0; c < d; ++c) a = fmaf(sE[c], W2[static_cast<size_t>(j) * d + c], a);
      sG[j] *= a;
    }
    __syncthreads();
    // acc1 += k^T E1 ; H^Q = q (W1 - acc1) ; commit if the chunk is full
    for (int j = tid; j < h; j += NT) {
      const float e1 = sG[j];
      float hq = 0.f;
      for (int k = 0; k < d; ++k) {
        const size_t i = static_cast<size_t>(k) * h + j;
        const float a = fmaf(sk[k], e1, P1[i]);
        const float w = W1[i] - a;
        hq = fmaf(sq[k], w, hq);
        if (commit) {
          W1[i] = w;
          P1[i] = 0.f;
        } else {
          P1[i] = a;
        }
      }
      sAQ[j] = gelu(hq, p.gelu);
    }
    __syncthreads();
  }
  // Z^Q[c] = sum_j x_j (W[j][c] - acc[j][c]) with acc[j][c] += y_j E[c]
  {
    const int ngrp = NT / d, grp = tid / d, col = tid % d;
    const int n = KIND == TTT_MLP ? h : d;
    float* W = KIND == TTT_MLP ? W2 : W1;
    float* P = KIND == TTT_MLP ? P2 : P1;
    const float* xs = KIND == TTT_MLP ? sAQ : sq;
    const float* ys = KIND == TTT_MLP ? sA : sk;
    float a = 0.f;
    if (grp < ngrp) {
      const float e = sE[col];
      for (int j = grp; j < n; j += ngrp) {
        const size_t i = static_cast<size_t>(j) * d + col;
        const float pa = fmaf(ys[j], e, P[i]);
        const float w = W[i] - pa;
        a = fmaf(xs[j], w, a);
        if (commit) {
          W[i] = w;
          P[i] = 0.f;
        } else {
          P[i] = pa;
        }
      }
    }
    sPart[tid] = a;
    __syncthreads();
    if (tid < d) {
      float z = 0.f;
      for (int g = 0; g < ngrp; ++g) z += sPart[g * d + tid];
      sZ[tid] = z;
    }
    __syncthreads();
  }
  if (wave == 0 && !key_out) {
    const bool h0 = lane < d, h1 = lane + 64 < d;
    const float z0 = h0 ? sZ[lane] : 0.f, z1 = h1 ? sZ[lane + 64] : 0.f;
    const float mu = wave_sum(z0 + z1) / d;
    const float c0 = h0 ? z0 - mu : 0.f, c1 = h1 ? z1 - mu : 0.f;
    const float rs = 1.0f / sqrtf(wave_sum(c0 * c0 + c1 * c1) / d + p.eps);
    IO* zo = static_cast<IO*>(p.z) + static_cast<size_t>(bh) * d;
    float o0 = 0.f, o1 = 0.f;
    if (h0) {
      o0 = sq[lane] + gam[lane] * c0 * rs + bet[lane];
      zo[lane] = from_f32<IO>(o0);
    }
    if (h1) {
      o1 = sq[lane + 64] + gam[lane + 64] * c1 * rs + bet[lane + 64];
      zo[lane + 64] = from_f32<IO>(o1);
    }
    const float chk = wave_sum(o0 + o1);
    if (lane == 0) flag_nonfinite(p.status, chk);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.B * p.H), block(NT);
  if (p.io == TTT_BF16) {
    if (p.kind == TTT_MLP)
      hipLaunchKernelGGL((decode_kernel<bf16_t, TTT_MLP>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_kernel<bf16_t, TTT_LINEAR>), grid, block, 0, stream, p);
  } else {
    if (p.kind == TTT_MLP)
      hipLaunchKernelGGL((decode_kernel<float, TTT_MLP>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_kernel<float, TTT_LINEAR>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ttt
