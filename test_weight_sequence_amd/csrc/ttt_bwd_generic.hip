// Outer-loop backward of the TTT scan (gradients through the inner updates, i.e.
// gradients of gradients; the outer loop of "LLM : 빠른 논문 리뷰 : End-to-End Test-Time
// Training for Long Context", section 2.2, applied to the layer of "Test-Time
// Training(TTT)과 LLM 메모리", section "TTT layer").
//
// Portable fp32 kernel: one workgroup of 256 threads per (batch, head) walks the chunks
// backwards. Each chunk's forward is recomputed from the fp32 chunk-start weights the
// forward saved, then the adjoint is pushed through the dual-form outputs, the chunk-end
// weight update and the inner gradient (LayerNorm backward differentiated once more,
// GELU''). dW, the adjoint of the chunk-start weights, is carried in a per-head workspace
// slice. [b x d] / [b x b] arrays live in LDS, [b x h] arrays in a per-head workspace slice.
//
// Forward of one chunk (E rows carry eta' = eta_scale * eta):
//   HK = K W1, AK = s(HK), G = s'(HK); ZK = AK W2; xk = LN-normalised ZK (1/sigma = rk)
//   r = K + gamma xk + beta - V; g = 2 r gamma; d2 = rk (g - mean g - xk mean(g xk)); E2 = eta' d2
//   gA = E2 W2^T; E1 = gA (.) G; P1 = tril(Q K^T); HQ = Q W1 - P1 E1; AQ = s(HQ), GQ = s'(HQ)
//   P2 = tril(AQ AK^T); ZQ = AQ W2 - P2 E2; z = Q + gamma xq + beta
//   W1' = W1 - K^T E1;  W2' = W2 - AK^T E2
// (Linear: ZK = K W, E = eta' d2, ZQ = Q W - P1 E, W' = W - K^T E.)
// With TTT_OUTPUT_KEY (Eq. 9 of the E2E paper review, section 2.4.2) the output is
// z = K + gamma xk + beta: dz reaches dK directly and ZK through the first-order LayerNorm
// backward, and the query side gets a zero adjoint (dQ = 0).
#include "ttt_device.hpp"

namespace ttt {
namespace {

constexpr int NT = kThreads;
constexpr int MAXB = kMaxChunk;

enum { A_AK = 0, A_G, A_G2, A_GA, A_E1, A_AQ, A_GQ, A_DHQ, A_DAK, A_DE1, A_DHK, A_DGA, A_COUNT };
static_assert(A_COUNT == kBwdArrays, "per-head workspace layout");

struct LdsB {
  float *K, *V, *Q, *dO, *XK, *R, *D2, *E2, *XQ, *DZQ, *DE2, *DZK, *DQ, *DK, *DV;
  float *rk, *rq, *eta, *mgx, *P1, *P2, *dP1, *dP2, *red;
  float* end;  // one past the last float used
};

__device__ __forceinline__ LdsB carve_b(float* p, int b, int d) {
  LdsB s;
  float** rows[] = {&s.K, &s.V, &s.Q, &s.dO, &s.XK, &s.R, &s.D2, &s.E2,
                    &s.XQ, &s.DZQ, &s.DE2, &s.DZK, &s.DQ, &s.DK, &s.DV};
  for (float** r : rows) {
    *r = p;
    p += b * d;
  }
  s.rk = p; p += MAXB;
  s.rq = p; p += MAXB;
  s.eta = p; p += MAXB;
  s.mgx = p; p += MAXB;
  s.P1 = p; p += b * b;
  s.P2 = p; p += b * b;
  s.dP1 = p; p += b * b;
  s.dP2 = p; p += b * b;
  s.red = p;  // 2 * NT floats for the final gamma/beta reduction
  s.end = p + 2 * NT;
  return s;
}

// wave-level LayerNorm statistics of one row (lane owns elements lane, lane + 64)
struct Row2 {
  float a0, a1;
};

__device__ __forceinline__ float row_mean(float a0, float a1, int d) { return wave_sum(a0 + a1) / d; }

template <typename IO, int KIND>
__global__ void __launch_bounds__(NT) bwd_generic_kernel(BwdParams p) {
  extern __shared__ float lds_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x, hidx = bh % p.H;
  const int d = p.d, h = p.hid, b = p.chunk, T = p.T, nchunks = T / b;
  const size_t nW1 = KIND == TTT_MLP ? static_cast<size_t>(d) * h : static_cast<size_t>(d) * d;
  const size_t nW2 = KIND == TTT_MLP ? static_cast<size_t>(h) * d : 0;
  const size_t nW = nW1 + nW2;
  LdsB s = carve_b(lds_raw, b, d);
  TTT_POISON_BYTES(lds_raw, (s.end - lds_raw) * sizeof(float));
  TTT_POISON_DONE();
  float* work = p.work + static_cast<size_t>(bh) * bwd_work_floats_per_head(KIND, d, h, b);
  float* dW1 = work;
  float* dW2 = work + nW1;
  float* arr = work + nW;
  auto A = [&](int which) { return arr + static_cast<size_t>(which) * b * h; };
  const float* gam = p.gamma + static_cast<size_t>(hidx) * d;
  const float* bet = p.beta + static_cast<size_t>(hidx) * d;
  const float g0 = lane < d ? gam[lane] : 0.f, g1 = lane + 64 < d ? gam[lane + 64] : 0.f;
  const float b0 = lane < d ? bet[lane] : 0.f, b1 = lane + 64 < d ? bet[lane + 64] : 0.f;
  const bool h0 = lane < d, h1 = lane + 64 < d;
  const bool key_out = (p.flags & TTT_OUTPUT_KEY) != 0;
  float dgam0 = 0.f, dgam1 = 0.f, dbet0 = 0.f, dbet1 = 0.f;

  for (size_t i = tid; i < nW1; i += NT) dW1[i] = p.dwt_1 ? p.dwt_1[bh * nW1 + i] : 0.f;
  for (size_t i = tid; i < nW2; i += NT) dW2[i] = p.dwt_2 ? p.dwt_2[bh * nW2 + i] : 0.f;

  const size_t io_off = static_cast<size_t>(bh) * T * d;
  const IO* Qg = static_cast<const IO*>(p.Q) + io_off;
  const IO* Kg = static_cast<const IO*>(p.K) + io_off;
  const IO* Vg = static_cast<const IO*>(p.V) + io_off;
  const IO* dZg = static_cast<const IO*>(p.dZ) + io_off;
  IO* dQg = static_cast<IO*>(p.dQ) + io_off;
  IO* dKg = static_cast<IO*>(p.dK) + io_off;
  IO* dVg = static_cast<IO*>(p.dV) + io_off;
  const float* etag = p.eta + static_cast<size_t>(bh) * T;
  const int col = tid % d, ngrp = NT / d, grp = tid / d;
  __syncthreads();

  for (int c = nchunks - 1; c >= 0; --c) {
    const int t0 = c * b;
    const float* W1 = p.saved + (static_cast<size_t>(bh) * nchunks + c) * nW;
    const float* W2 = W1 + nW1;
    for (int i = tid; i < b * d; i += NT) {
      const size_t gi = static_cast<size_t>(t0) * d + i;
      s.K[i] = to_f32(Kg[gi]);
      s.V[i] = to_f32(Vg[gi]);
      s.Q[i] = to_f32(Qg[gi]);
      s.dO[i] = to_f32(dZg[gi]);
      s.DQ[i] = 0.f;
      s.DK[i] = 0.f;
      s.DE2[i] = 0.f;
    }
    if (tid < b) s.eta[tid] = etag[t0 + tid] * p.eta_scale;
    __syncthreads();

    // ================= forward recompute =================
    if (KIND == TTT_MLP) {
      // HK -> AK, G, G2 ; Q W1 parked in AQ
      for (int j = tid; j < h; j += NT) {
        float hk[MAXB], qw[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) hk[t] = qw[t] = 0.f;
        for (int k = 0; k < d; ++k) {
          const float w = W1[static_cast<size_t>(k) * h + j];
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) {
              hk[t] = fmaf(s.K[t * d + k], w, hk[t]);
              qw[t] = fmaf(s.Q[t * d + k], w, qw[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            const Gelu3 gv = gelu_d2(hk[t], p.gelu);
            A(A_AK)[t * h + j] = gv.v;
            A(A_G)[t * h + j] = gv.d1;
            A(A_G2)[t * h + j] = gv.d2;
            A(A_AQ)[t * h + j] = qw[t];
          }
      }
      __syncthreads();
    }
    // ZK (into XK for now)
    if (grp < ngrp) {
      float acc[MAXB];
#pragma unroll
      for (int m = 0; m < MAXB; ++m) acc[m] = 0.f;
      const int n = KIND == TTT_MLP ? h : d;
      for (int j = 0; j < n; ++j) {
        const float w = KIND == TTT_MLP ? W2[static_cast<size_t>(j) * d + col]
                                        : W1[static_cast<size_t>(j) * d + col];
#pragma unroll
        for (int m = 0; m < MAXB; ++m) {
          const int t = grp + m * ngrp;
          if (t < b) acc[m] = fmaf(KIND == TTT_MLP ? A(A_AK)[t * h + j] : s.K[t * d + j], w, acc[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < MAXB; ++m) {
        const int t = grp + m * ngrp;
        if (t < b) s.XK[t * d + col] = acc[m];
      }
    }
    __syncthreads();
    // LN(K): xk, r, d2 (unscaled), E2, rk, mgx
    for (int t = wave; t < b; t += NT / 64) {
      const float z0 = h0 ? s.XK[t * d + lane] : 0.f, z1 = h1 ? s.XK[t * d + lane + 64] : 0.f;
      const float mu = row_mean(z0, z1, d);
      const float c0 = h0 ? z0 - mu : 0.f, c1 = h1 ? z1 - mu : 0.f;
      const float rs = 1.0f / sqrtf(wave_sum(c0 * c0 + c1 * c1) / d + p.eps);
      const float x0 = c0 * rs, x1 = c1 * rs;
      const float r0 = h0 ? s.K[t * d + lane] + g0 * x0 + b0 - s.V[t * d + lane] : 0.f;
      const float r1 = h1 ? s.K[t * d + lane + 64] + g1 * x1 + b1 - s.V[t * d + lane + 64] : 0.f;
      const float gg0 = 2.f * r0 * g0, gg1 = 2.f * r1 * g1;
      const float mg = row_mean(gg0, gg1, d), mgx = row_mean(gg0 * x0, gg1 * x1, d);
      const float e = s.eta[t];
      if (h0) {
        const float d2 = (gg0 - mg - x0 * mgx) * rs;
        s.XK[t * d + lane] = x0;
        s.R[t * d + lane] = r0;
        s.D2[t * d + lane] = d2;
        s.E2[t * d + lane] = e * d2;
      }
      if (h1) {
        const float d2 = (gg1 - mg - x1 * mgx) * rs;
        s.XK[t * d + lane + 64] = x1;
        s.R[t * d + lane + 64] = r1;
        s.D2[t * d + lane + 64] = d2;
        s.E2[t * d + lane + 64] = e * d2;
      }
      if (lane == 0) {
        s.rk[t] = rs;
        s.mgx[t] = mgx;
      }
    }
    // P1 = tril(Q K^T)
    for (int i = tid; i < b * b; i += NT) {
      const int t = i / b, u = i % b;
      float a = 0.f;
      if (u <= t)
        for (int k = 0; k < d; ++k) a = fmaf(s.Q[t * d + k], s.K[u * d + k], a);
      s.P1[i] = a;
    }
    __syncthreads();
    if (KIND == TTT_MLP) {
      // gA = E2 W2^T, E1 = gA (.) G
      for (int j = tid; j < h; j += NT) {
        float ga[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) ga[t] = 0.f;
        const float4* w2row = reinterpret_cast<const float4*>(W2 + static_cast<size_t>(j) * d);
        for (int k4 = 0; k4 < d / 4; ++k4) {
          const float4 w = w2row[k4];
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) {
              const float* e = s.E2 + t * d + 4 * k4;
              ga[t] = fmaf(e[0], w.x, fmaf(e[1], w.y, fmaf(e[2], w.z, fmaf(e[3], w.w, ga[t]))));
            }
        }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            A(A_GA)[t * h + j] = ga[t];
            A(A_E1)[t * h + j] = ga[t] * A(A_G)[t * h + j];
          }
      }
      __syncthreads();
      // HQ = QW1 - P1 E1 -> AQ, GQ
      for (int j = tid; j < h; j += NT) {
        float hq[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) hq[t] = t < b ? A(A_AQ)[t * h + j] : 0.f;
#pragma unroll
        for (int u = 0; u < MAXB; ++u)
          if (u < b) {
            const float e1 = A(A_E1)[u * h + j];
#pragma unroll
            for (int t = 0; t < MAXB; ++t)
              if (t < b && u <= t) hq[t] = fmaf(-s.P1[t * b + u], e1, hq[t]);
          }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            float v, d1;
            gelu_d(hq[t], p.gelu, v, d1);
            A(A_AQ)[t * h + j] = v;
            A(A_GQ)[t * h + j] = d1;
          }
      }
      __syncthreads();
      // P2 = tril(AQ AK^T)
      for (int i = tid; i < b * b; i += NT) {
        const int t = i / b, u = i % b;
        float a = 0.f;
        if (u <= t)
          for (int j = 0; j < h; ++j) a = fmaf(A(A_AQ)[t * h + j], A(A_AK)[u * h + j], a);
        s.P2[i] = a;
      }
      __syncthreads();
    }
    // ZQ (into XQ)
    if (grp < ngrp) {
      float acc[MAXB];
#pragma unroll
      for (int m = 0; m < MAXB; ++m) acc[m] = 0.f;
      const int n = KIND == TTT_MLP ? h : d;
      for (int j = 0; j < n; ++j) {
        const float w = KIND == TTT_MLP ? W2[static_cast<size_t>(j) * d + col]
                                        : W1[static_cast<size_t>(j) * d + col];
#pragma unroll
        for (int m = 0; m < MAXB; ++m) {
          const int t = grp + m * ngrp;
          if (t < b) acc[m] = fmaf(KIND == TTT_MLP ? A(A_AQ)[t * h + j] : s.Q[t * d + j], w, acc[m]);
        }
      }
      const float* P = KIND == TTT_MLP ? s.P2 : s.P1;
#pragma unroll
      for (int m = 0; m < MAXB; ++m) {
        const int t = grp + m * ngrp;
        if (t < b) {
          float a = acc[m];
          for (int u = 0; u <= t; ++u) a = fmaf(-P[t * b + u], s.E2[u * d + col], a);
          s.XQ[t * d + col] = a;
        }
      }
    }
    __syncthreads();

    // ================= backward =================
    // LN(Q) and the output: dQ = dO, dgamma/dbeta, dZQ (zero with the key-side output)
    for (int t = wave; t < b; t += NT / 64) {
      if (key_out) {
        if (h0) {
          s.DZQ[t * d + lane] = 0.f;
          s.DQ[t * d + lane] = 0.f;
        }
        if (h1) {
          s.DZQ[t * d + lane + 64] = 0.f;
          s.DQ[t * d + lane + 64] = 0.f;
        }
        continue;
      }
      const float z0 = h0 ? s.XQ[t * d + lane] : 0.f, z1 = h1 ? s.XQ[t * d + lane + 64] : 0.f;
      const float mu = row_mean(z0, z1, d);
      const float c0 = h0 ? z0 - mu : 0.f, c1 = h1 ? z1 - mu : 0.f;
      const float rs = 1.0f / sqrtf(wave_sum(c0 * c0 + c1 * c1) / d + p.eps);
      const float x0 = c0 * rs, x1 = c1 * rs;
      const float o0 = h0 ? s.dO[t * d + lane] : 0.f, o1 = h1 ? s.dO[t * d + lane + 64] : 0.f;
      dgam0 += o0 * x0;
      dgam1 += o1 * x1;
      dbet0 += o0;
      dbet1 += o1;
      const float v0 = o0 * g0, v1 = o1 * g1;
      const float mv = row_mean(v0, v1, d), mvx = row_mean(v0 * x0, v1 * x1, d);
      if (h0) {
        s.XQ[t * d + lane] = x0;
        s.DZQ[t * d + lane] = (v0 - mv - x0 * mvx) * rs;
        s.DQ[t * d + lane] = o0;
      }
      if (h1) {
        s.XQ[t * d + lane + 64] = x1;
        s.DZQ[t * d + lane + 64] = (v1 - mv - x1 * mvx) * rs;
        s.DQ[t * d + lane + 64] = o1;
      }
      if (lane == 0) s.rq[t] = rs;
    }
    __syncthreads();

    const float* P = KIND == TTT_MLP ? s.P2 : s.P1;
    float* dP = KIND == TTT_MLP ? s.dP2 : s.dP1;
    // dP (the P multiplying E2 in ZQ) = -dZQ E2^T (masked); dE2 = -P^T dZQ
    for (int i = tid; i < b * b; i += NT) {
      const int t = i / b, u = i % b;
      float a = 0.f;
      if (u <= t)
        for (int k = 0; k < d; ++k) a = fmaf(s.DZQ[t * d + k], s.E2[u * d + k], a);
      dP[i] = -a;
    }
    if (grp < ngrp) {
#pragma unroll
      for (int m = 0; m < MAXB; ++m) {
        const int u = grp + m * ngrp;
        if (u < b) {
          float a = 0.f;
          for (int t = u; t < b; ++t) a = fmaf(P[t * b + u], s.DZQ[t * d + col], a);
          s.DE2[u * d + col] -= a;
        }
      }
    }
    __syncthreads();

    if (KIND == TTT_MLP) {
      // dAQ = dZQ W2^T + dP2 AK ; dAK = dP2^T AQ ; dHQ = dAQ (.) GQ
      for (int j = tid; j < h; j += NT) {
        float da[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) da[t] = 0.f;
        const float4* w2row = reinterpret_cast<const float4*>(W2 + static_cast<size_t>(j) * d);
        for (int k4 = 0; k4 < d / 4; ++k4) {
          const float4 w = w2row[k4];
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) {
              const float* e = s.DZQ + t * d + 4 * k4;
              da[t] = fmaf(e[0], w.x, fmaf(e[1], w.y, fmaf(e[2], w.z, fmaf(e[3], w.w, da[t]))));
            }
        }
        float dak[MAXB];
#pragma unroll
        for (int u = 0; u < MAXB; ++u) dak[u] = 0.f;
#pragma unroll
        for (int u = 0; u < MAXB; ++u)
          if (u < b) {
            const float ak = A(A_AK)[u * h + j];
#pragma unroll
            for (int t = 0; t < MAXB; ++t)
              if (t < b && u <= t) da[t] = fmaf(s.dP2[t * b + u], ak, da[t]);
          }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            const float aq = A(A_AQ)[t * h + j];
#pragma unroll
            for (int u = 0; u < MAXB; ++u)
              if (u < b && u <= t) dak[u] = fmaf(s.dP2[t * b + u], aq, dak[u]);
          }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            A(A_DHQ)[t * h + j] = da[t] * A(A_GQ)[t * h + j];
            A(A_DAK)[t * h + j] = dak[t];
          }
      }
      __syncthreads();
      // dP1 = -dHQ E1^T (masked)
      for (int i = tid; i < b * b; i += NT) {
        const int t = i / b, u = i % b;
        float a = 0.f;
        if (u <= t)
          for (int j = 0; j < h; ++j) a = fmaf(A(A_DHQ)[t * h + j], A(A_E1)[u * h + j], a);
        s.dP1[i] = -a;
      }
      // dE1 = -P1^T dHQ - K dW1'   (dW1 still holds the chunk-end adjoint)
      for (int j = tid; j < h; j += NT) {
        float de[MAXB];
#pragma unroll
        for (int u = 0; u < MAXB; ++u) de[u] = 0.f;
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            const float dh = A(A_DHQ)[t * h + j];
#pragma unroll
            for (int u = 0; u < MAXB; ++u)
              if (u < b && u <= t) de[u] = fmaf(-s.P1[t * b + u], dh, de[u]);
          }
        for (int k = 0; k < d; ++k) {
          const float w = dW1[static_cast<size_t>(k) * h + j];
#pragma unroll
          for (int u = 0; u < MAXB; ++u)
            if (u < b) de[u] = fmaf(-s.K[u * d + k], w, de[u]);
        }
        // dAK += -E2 dW2'^T
        float dak[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) dak[t] = 0.f;
        const float4* dw2row = reinterpret_cast<const float4*>(dW2 + static_cast<size_t>(j) * d);
        for (int k4 = 0; k4 < d / 4; ++k4) {
          const float4 w = dw2row[k4];
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) {
              const float* e = s.E2 + t * d + 4 * k4;
              dak[t] = fmaf(e[0], w.x, fmaf(e[1], w.y, fmaf(e[2], w.z, fmaf(e[3], w.w, dak[t]))));
            }
        }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            A(A_DAK)[t * h + j] -= dak[t];
            // dgA = dE1 (.) G ; dHK = dE1 (.) gA (.) G2
            const float de1 = de[t];
            A(A_DE1)[t * h + j] = de1;
            A(A_DGA)[t * h + j] = de1 * A(A_G)[t * h + j];
            A(A_DHK)[t * h + j] = de1 * A(A_GA)[t * h + j] * A(A_G2)[t * h + j];
          }
      }
      __syncthreads();
    }

    // column-owner pass over d: dQ, dK from the dual terms and the update adjoint; dE2
    if (grp < ngrp) {
#pragma unroll
      for (int m = 0; m < MAXB; ++m) {
        const int t = grp + m * ngrp;
        if (t >= b) continue;
        float dq = 0.f, dk = 0.f, de2 = 0.f;
        if (KIND == TTT_MLP) {
          // dQ += dHQ W1^T ; dK += -E1 dW1'^T ; dE2 += dgA W2 - AK dW2'
          for (int j = 0; j < h; ++j) {
            const size_t wi = static_cast<size_t>(col) * h + j;
            dq = fmaf(A(A_DHQ)[t * h + j], W1[wi], dq);
            dk = fmaf(-A(A_E1)[t * h + j], dW1[wi], dk);
            const size_t w2i = static_cast<size_t>(j) * d + col;
            de2 = fmaf(A(A_DGA)[t * h + j], W2[w2i], de2);
            de2 = fmaf(-A(A_AK)[t * h + j], dW2[w2i], de2);
          }
        } else {
          // Linear: dQ += dZQ W^T ; dK += -E dW'^T ; dE += -K dW'
          for (int k = 0; k < d; ++k) {
            const size_t wi = static_cast<size_t>(col) * d + k;
            dq = fmaf(s.DZQ[t * d + k], W1[wi], dq);
            dk = fmaf(-s.E2[t * d + k], dW1[wi], dk);
            de2 = fmaf(-s.K[t * d + k], dW1[static_cast<size_t>(k) * d + col], de2);
          }
        }
        // dQ += dP1 K ; dK += dP1^T Q
        for (int u = 0; u <= t; ++u) dq = fmaf(s.dP1[t * b + u], s.K[u * d + col], dq);
        for (int u = t; u < b; ++u) dk = fmaf(s.dP1[u * b + t], s.Q[u * d + col], dk);
        s.DQ[t * d + col] += dq;
        s.DK[t * d + col] += dk;
        s.DE2[t * d + col] += de2;
      }
    }
    __syncthreads();

    // inner-gradient backward per token: deta, dV, dK (residual), dgamma/dbeta, dZK
    for (int t = wave; t < b; t += NT / 64) {
      const float rs = s.rk[t], mgx = s.mgx[t], e = s.eta[t];
      const float x0 = h0 ? s.XK[t * d + lane] : 0.f, x1 = h1 ? s.XK[t * d + lane + 64] : 0.f;
      const float r0 = h0 ? s.R[t * d + lane] : 0.f, r1 = h1 ? s.R[t * d + lane + 64] : 0.f;
      const float q0 = h0 ? s.D2[t * d + lane] : 0.f, q1 = h1 ? s.D2[t * d + lane + 64] : 0.f;
      const float de0 = h0 ? s.DE2[t * d + lane] : 0.f, de1 = h1 ? s.DE2[t * d + lane + 64] : 0.f;
      const float deta = wave_sum(de0 * q0 + de1 * q1) * p.eta_scale;
      const float u0 = e * de0, u1 = e * de1;
      const float mu = row_mean(u0, u1, d), mux = row_mean(u0 * x0, u1 * x1, d);
      const float gg0 = 2.f * r0 * g0, gg1 = 2.f * r1 * g1;
      const float dg0 = rs * (u0 - mu - x0 * mux), dg1 = rs * (u1 - mu - x1 * mux);
      float dx0 = -rs * (u0 * mgx + gg0 * mux), dx1 = -rs * (u1 * mgx + gg1 * mux);
      const float ds = -rs * wave_sum(u0 * q0 + u1 * q1);
      const float dr0 = 2.f * g0 * dg0, dr1 = 2.f * g1 * dg1;
      dgam0 += 2.f * r0 * dg0 + dr0 * x0;
      dgam1 += 2.f * r1 * dg1 + dr1 * x1;
      dbet0 += dr0;
      dbet1 += dr1;
      dx0 += g0 * dr0;
      dx1 += g1 * dr1;
      // key-side output z = K + gamma xk + beta: its adjoint dO enters through the LayerNorm
      float o0 = 0.f, o1 = 0.f;
      if (key_out) {
        o0 = h0 ? s.dO[t * d + lane] : 0.f;
        o1 = h1 ? s.dO[t * d + lane + 64] : 0.f;
        dgam0 += o0 * x0;
        dgam1 += o1 * x1;
        dbet0 += o0;
        dbet1 += o1;
        dx0 += g0 * o0;
        dx1 += g1 * o1;
      }
      const float mdx = row_mean(dx0, dx1, d), mdxx = row_mean(dx0 * x0, dx1 * x1, d);
      if (h0) {
        s.DZK[t * d + lane] = rs * (dx0 - mdx - x0 * mdxx) + ds * x0 / d;
        s.DK[t * d + lane] += dr0 + o0;
        s.DV[t * d + lane] = -dr0;
      }
      if (h1) {
        s.DZK[t * d + lane + 64] = rs * (dx1 - mdx - x1 * mdxx) + ds * x1 / d;
        s.DK[t * d + lane + 64] += dr1 + o1;
        s.DV[t * d + lane + 64] = -dr1;
      }
      if (lane == 0) p.deta[static_cast<size_t>(bh) * T + t0 + t] = deta;
    }
    __syncthreads();

    if (KIND == TTT_MLP) {
      // dAK += dZK W2^T ; dHK += dAK (.) G
      for (int j = tid; j < h; j += NT) {
        float da[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) da[t] = 0.f;
        const float4* w2row = reinterpret_cast<const float4*>(W2 + static_cast<size_t>(j) * d);
        for (int k4 = 0; k4 < d / 4; ++k4) {
          const float4 w = w2row[k4];
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) {
              const float* e = s.DZK + t * d + 4 * k4;
              da[t] = fmaf(e[0], w.x, fmaf(e[1], w.y, fmaf(e[2], w.z, fmaf(e[3], w.w, da[t]))));
            }
        }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            const float dak = A(A_DAK)[t * h + j] + da[t];
            A(A_DAK)[t * h + j] = dak;
            A(A_DHK)[t * h + j] += dak * A(A_G)[t * h + j];
          }
      }
      __syncthreads();
    }
    // dK += dHK W1^T (Linear: dK += dZK W^T); write dQ, dK, dV
    if (grp < ngrp) {
#pragma unroll
      for (int m = 0; m < MAXB; ++m) {
        const int t = grp + m * ngrp;
        if (t >= b) continue;
        float dk = 0.f;
        if (KIND == TTT_MLP) {
          for (int j = 0; j < h; ++j)
            dk = fmaf(A(A_DHK)[t * h + j], W1[static_cast<size_t>(col) * h + j], dk);
        } else {
          for (int k = 0; k < d; ++k) dk = fmaf(s.DZK[t * d + k], W1[static_cast<size_t>(col) * d + k], dk);
        }
        const size_t gi = static_cast<size_t>(t0 + t) * d + col;
        dKg[gi] = from_f32<IO>(s.DK[t * d + col] + dk);
        dQg[gi] = from_f32<IO>(s.DQ[t * d + col]);
        dVg[gi] = from_f32<IO>(s.DV[t * d + col]);
      }
    }
    // dW (adjoint of the chunk-start weights) = dW' + this chunk's direct terms
    if (KIND == TTT_MLP) {
      for (int i = tid; i < d * h; i += NT) {
        const int k = i / h, j = i % h;
        float a = dW1[i];
        for (int t = 0; t < b; ++t) {
          a = fmaf(s.Q[t * d + k], A(A_DHQ)[t * h + j], a);
          a = fmaf(s.K[t * d + k], A(A_DHK)[t * h + j], a);
        }
        dW1[i] = a;
      }
      for (int i = tid; i < h * d; i += NT) {
        const int j = i / d, cc = i % d;
        float a = dW2[i];
        for (int t = 0; t < b; ++t) {
          a = fmaf(A(A_AQ)[t * h + j], s.DZQ[t * d + cc], a);
          a = fmaf(A(A_DGA)[t * h + j], s.E2[t * d + cc], a);
          a = fmaf(A(A_AK)[t * h + j], s.DZK[t * d + cc], a);
        }
        dW2[i] = a;
      }
    } else {
      for (int i = tid; i < d * d; i += NT) {
        const int k = i / d, cc = i % d;
        float a = dW1[i];
        for (int t = 0; t < b; ++t) {
          a = fmaf(s.Q[t * d + k], s.DZQ[t * d + cc], a);
          a = fmaf(s.K[t * d + k], s.DZK[t * d + cc], a);
        }
        dW1[i] = a;
      }
    }
    __syncthreads();
  }

  // per-head dgamma / dbeta partials (summed over the waves), finalised over the batch
  s.red[tid] = dgam0;
  s.red[NT + tid] = dgam1;
  __syncthreads();
  if (tid < 64) {
    float a0 = 0.f, a1 = 0.f;
    for (int w = 0; w < NT / 64; ++w) {
      a0 += s.red[w * 64 + tid];
      a1 += s.red[NT + w * 64 + tid];
    }
    if (tid < d) p.dgb[static_cast<size_t>(bh) * 2 * d + tid] = a0;
    if (tid + 64 < d) p.dgb[static_cast<size_t>(bh) * 2 * d + tid + 64] = a1;
  }
  __syncthreads();
  s.red[tid] = dbet0;
  s.red[NT + tid] = dbet1;
  __syncthreads();
  if (tid < 64) {
    float a0 = 0.f, a1 = 0.f;
    for (int w = 0; w < NT / 64; ++w) {
      a0 += s.red[w * 64 + tid];
      a1 += s.red[NT + w * 64 + tid];
    }
    if (tid < d) p.dgb[static_cast<size_t>(bh) * 2 * d + d + tid] = a0;
    if (tid + 64 < d) p.dgb[static_cast<size_t>(bh) * 2 * d + d + tid + 64] = a1;
  }
}

// dW0 (summed over the batch unless W0 is per sequence), dgamma, dbeta
__global__ void __launch_bounds__(NT) bwd_finalize_kernel(BwdParams p) {
  const int d = p.d, h = p.hid;
  const size_t nW1 = p.kind == TTT_MLP ? static_cast<size_t>(d) * h : static_cast<size_t>(d) * d;
  const size_t nW2 = p.kind == TTT_MLP ? static_cast<size_t>(h) * d : 0;
  const size_t per_head = bwd_work_floats_per_head(p.kind, d, h, p.chunk);
  const bool per_seq = (p.flags & TTT_W0_PER_SEQ) != 0;
  const int hidx = blockIdx.y;
  const size_t n = nW1 + nW2 + 2 * d;
  for (size_t i = static_cast<size_t>(blockIdx.x) * NT + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * NT) {
    if (i < nW1 + nW2) {
      if (per_seq) {
        for (int bb = 0; bb < p.B; ++bb) {
          const size_t bh = static_cast<size_t>(bb) * p.H + hidx;
          const float v = p.work[bh * per_head + i];
          if (i < nW1) p.dw0_1[bh * nW1 + i] = v;
          else p.dw0_2[bh * nW2 + (i - nW1)] = v;
        }
      } else {
        float a = 0.f;
        for (int bb = 0; bb < p.B; ++bb) a += p.work[(static_cast<size_t>(bb) * p.H + hidx) * per_head + i];
        if (i < nW1) p.dw0_1[hidx * nW1 + i] = a;
        else p.dw0_2[hidx * nW2 + (i - nW1)] = a;
      }
    } else {
      const size_t k = i - nW1 - nW2;  // 0 .. 2d-1
      float a = 0.f;
      for (int bb = 0; bb < p.B; ++bb) a += p.dgb[(static_cast<size_t>(bb) * p.H + hidx) * 2 * d + k];
      if (k < static_cast<size_t>(d)) {
        if (p.dgamma) p.dgamma[hidx * d + k] = a;
      } else if (p.dbeta) {
        p.dbeta[hidx * d + (k - d)] = a;
      }
    }
  }
}

}  // namespace

size_t bwd_generic_lds_bytes(int, int d, int, int chunk) {
  const size_t f = 15 * static_cast<size_t>(chunk) * d + 4 * MAXB + 4 * static_cast<size_t>(chunk) * chunk +
                   2 * NT;
  return f * sizeof(float);
}

hipError_t launch_bwd_generic(const BwdParams& p, hipStream_t stream) {
  const size_t lds = bwd_generic_lds_bytes(p.kind, p.d, p.hid, p.chunk);
  const dim3 grid(p.B * p.H), block(NT);
  hipError_t e;
#define TTT_LAUNCH_B(IO, KIND)                                                            \
  do {                                                                                    \
    auto fn = bwd_generic_kernel<IO, KIND>;                                               \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),                            \
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)); \
    if (e != hipSuccess) return e;                                                        \
    hipLaunchKernelGGL(fn, grid, block, lds, stream, p);                                  \
  } while (0)
  if (p.io == TTT_BF16) {
    if (p.kind == TTT_MLP) TTT_LAUNCH_B(bf16_t, TTT_MLP); else TTT_LAUNCH_B(bf16_t, TTT_LINEAR);
  } else {
    if (p.kind == TTT_MLP) TTT_LAUNCH_B(float, TTT_MLP); else TTT_LAUNCH_B(float, TTT_LINEAR);
  }
#undef TTT_LAUNCH_B
  return hipGetLastError();
}

hipError_t launch_bwd_finalize(const BwdParams& p, hipStream_t stream) {
  const size_t n = n_weights(p.kind, p.d, p.hid) + 2 * static_cast<size_t>(p.d);
  const int bx = static_cast<int>((n + NT - 1) / NT);
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3(bx < 1024 ? bx : 1024, p.H), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ttt
