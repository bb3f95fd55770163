// Portable fp32 forward scan for gfx950: any supported (kind, d, hidden, chunk, io
// dtype). One workgroup of 256 threads per (batch, head); the fp32 fast weights of
// each head live in a global workspace slice (L2-resident at the sizes used), the
// chunk's intermediates live in LDS.
//
// Per chunk (all quantities at the chunk-start weights, E = eta-scaled rows):
//   H^K = K W1, A^K = GELU(H^K), G = GELU'(H^K), Z^K = A^K W2
//   LN forward/backward on Z^K  -> delta2;  E2 = eta (.) delta2
//   E1 = (E2 W2^T) (.) G
//   H^Q = Q W1 - tril(Q K^T) E1,  A^Q = GELU(H^Q)
//   Z^Q = A^Q W2 - tril(A^Q A^K^T) E2,  z = Q + LN(Z^Q)
//   W1 -= K^T E1,  W2 -= A^K^T E2
// This is the dual form of the per-token rule: expanding W_t = W_start - sum_{s<=t}
// eta_s grad l_s(W_start) inside f(Q_t; W_t) gives exactly these products (page
// "Test-Time Training(TTT)과 LLM 메모리", section "TTT layer": Eq. 2/4/5, dual form;
// mini-batch rule from the E2E paper review, section 2.3, Eq. 5).
// TTT-Linear drops the hidden layer: Z^K = K W, E = eta (.) delta, Z^Q = Q W - tril(Q K^T) E,
// W -= K^T E.
// With TTT_OUTPUT_KEY (the simplified output rule, E2E paper review section 2.4.2, Eq. 9)
// the output is the key-side prediction at the chunk-start weights, z = K + LN(Z^K), and
// the query side (H^Q, Z^Q) is skipped.
//
// With momentum and a forget gate (page "Test-Time Training(TTT)과 LLM 메모리", section
// "Titans와 Miras", Eq. 14: S_t = m_t S_{t-1} - theta_t grad_t, Eq. 13: M_t = (1 - a_t) M_{t-1}
// + S_t, gradients at the chunk-start memory) the two linear recurrences unroll, inside a
// chunk, into M_t = A_t M + B_t S - sum_{s<=t} C_ts theta_s grad_s and S_t = P_t S -
// sum_{s<=t} D_ts theta_s grad_s, with scalar coefficients of the chunk's gates:
//   P_t = m_t P_{t-1}, D_ts = m_t D_{t-1,s} (D_tt = 1), A_t = (1 - a_t) A_{t-1},
//   B_t = (1 - a_t) B_{t-1} + P_t, C_ts = (1 - a_t) C_{t-1,s} + D_ts  (A_0 = P_0 = 1, B_0 = 0).
// The dual form then scales the chunk-start products per token (A_t Q W1 + B_t Q S1) and
// weights the causal masks by C; the memory and the momentum are both carried.
#include "ttt_device.hpp"

namespace ttt {
namespace {

constexpr int NT = kThreads;
constexpr int MAXB = kMaxChunk;

struct Lds {
  float *K, *V, *Q, *E, *A, *G, *AQ, *Z, *ZQ, *S;
  float *C, *Dl, *Av, *Bv;  // momentum coefficients: C [b x b], last row of D, A_t, B_t, P_b
  float* end;               // one past the last float used
};

__device__ __forceinline__ Lds carve(float* base, int kind, int b, int d, int h, bool mom) {
  Lds s;
  float* p = base;
  s.K = p; p += b * d;
  s.V = p; p += b * d;
  s.Q = p; p += b * d;
  s.Z = p; p += b * d;
  s.ZQ = p; p += b * d;
  s.E = p; p += 16;
  s.S = p; p += b * b;
  if (kind == TTT_MLP) {
    s.A = p; p += b * h;
    s.G = p; p += b * h;
    s.AQ = p; p += b * h;
  } else {
    s.A = s.G = s.AQ = nullptr;
  }
  if (mom) {
    s.C = p; p += b * b;
    s.Dl = p; p += b;
    s.Av = p; p += b;
    s.Bv = p; p += b + 1;
  } else {
    s.C = s.Dl = s.Av = s.Bv = nullptr;
  }
  s.end = p;
  return s;
}

// LayerNorm statistics of one row held by a wave (lane owns elements lane, lane+64).
struct RowLN {
  float xh0, xh1, rsig;
};

__device__ __forceinline__ RowLN ln_row(float z0, float z1, int lane, int d, float eps) {
  const bool has0 = lane < d, has1 = lane + 64 < d;
  float s = (has0 ? z0 : 0.f) + (has1 ? z1 : 0.f);
  float mu = wave_sum(s) / d;
  float c0 = has0 ? z0 - mu : 0.f, c1 = has1 ? z1 - mu : 0.f;
  float var = wave_sum(c0 * c0 + c1 * c1) / d;
  RowLN r;
  r.rsig = 1.0f / sqrtf(var + eps);
  r.xh0 = c0 * r.rsig;
  r.xh1 = c1 * r.rsig;
  return r;
}

template <typename IO, int KIND, bool MOM>
__global__ void __launch_bounds__(NT) fwd_generic_kernel(ScanParams p) {
  extern __shared__ float lds_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x;
  const int hidx = bh % p.H;
  const int d = p.d, h = p.hid, b = p.chunk;
  const size_t nW1 = KIND == TTT_MLP ? static_cast<size_t>(d) * h : static_cast<size_t>(d) * d;
  const size_t nW2 = KIND == TTT_MLP ? static_cast<size_t>(h) * d : 0;
  const size_t nW = nW1 + nW2;
  Lds s = carve(lds_raw, KIND, b, d, h, MOM);
  TTT_POISON_BYTES(lds_raw, (s.end - lds_raw) * sizeof(float));
  TTT_POISON_DONE();

  float* W1 = p.wbuf + static_cast<size_t>(bh) * (MOM ? 2 * nW : nW);
  float* W2 = W1 + nW1;
  float* S1 = W1 + nW;  // momentum (MOM only)
  float* S2 = S1 + nW1;
  const bool per_seq = (p.flags & TTT_W0_PER_SEQ) != 0;
  const bool key_out = (p.flags & TTT_OUTPUT_KEY) != 0;
  const size_t w0_head = per_seq ? static_cast<size_t>(bh) : static_cast<size_t>(hidx);
  for (size_t i = tid; i < nW1; i += NT) W1[i] = p.w0_1[w0_head * nW1 + i];
  for (size_t i = tid; i < nW2; i += NT) W2[i] = p.w0_2[w0_head * nW2 + i];
  if (MOM) {
    for (size_t i = tid; i < nW1; i += NT) S1[i] = p.s0_1 ? p.s0_1[static_cast<size_t>(bh) * nW1 + i] : 0.f;
    for (size_t i = tid; i < nW2; i += NT) S2[i] = p.s0_2 ? p.s0_2[static_cast<size_t>(bh) * nW2 + i] : 0.f;
  }
  const float* gam = p.gamma + static_cast<size_t>(hidx) * d;
  const float* bet = p.beta + static_cast<size_t>(hidx) * d;
  const float g0 = lane < d ? gam[lane] : 0.f, g1 = lane + 64 < d ? gam[lane + 64] : 0.f;
  const float b0 = lane < d ? bet[lane] : 0.f, b1 = lane + 64 < d ? bet[lane + 64] : 0.f;
  __syncthreads();

  const IO* Qg = static_cast<const IO*>(p.Q) + static_cast<size_t>(bh) * p.T * d;
  const IO* Kg = static_cast<const IO*>(p.K) + static_cast<size_t>(bh) * p.T * d;
  const IO* Vg = static_cast<const IO*>(p.V) + static_cast<size_t>(bh) * p.T * d;
  IO* Zg = static_cast<IO*>(p.Z) + static_cast<size_t>(bh) * p.T * d;
  const float* etag = p.eta + static_cast<size_t>(bh) * p.T;
  const int nchunks = p.T / b;
  // column-owner mapping for the [b x d] outputs
  const int col = tid % d, ngrp = NT / d, grp = tid / d;

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * b;
    if (p.saved) {
      float* sv = p.saved + (static_cast<size_t>(bh) * nchunks + c) * nW;
      for (size_t i = tid; i < nW; i += NT) sv[i] = W1[i];
    }
    for (int i = tid; i < b * d; i += NT) {
      s.K[i] = to_f32(Kg[static_cast<size_t>(t0) * d + i]);
      s.V[i] = to_f32(Vg[static_cast<size_t>(t0) * d + i]);
      s.Q[i] = to_f32(Qg[static_cast<size_t>(t0) * d + i]);
    }
    if (tid < b) s.E[tid] = etag[t0 + tid] * p.eta_scale;
    if (MOM && tid == 0) {
      // the chunk's coefficients (header comment), token by token
      const float* mg = p.mom + static_cast<size_t>(bh) * p.T + t0;
      const float* ag = p.alpha + static_cast<size_t>(bh) * p.T + t0;
      float D[MAXB], Cr[MAXB];
#pragma unroll
      for (int u = 0; u < MAXB; ++u) D[u] = Cr[u] = 0.f;
      float A = 1.f, Bc = 0.f, P = 1.f;
      for (int t = 0; t < b; ++t) {
        const float m = mg[t], keep = 1.f - ag[t];
        P *= m;
        A *= keep;
        Bc = keep * Bc + P;
#pragma unroll
        for (int u = 0; u < MAXB; ++u) {
          if (u < t) D[u] *= m;
          if (u == t) D[u] = 1.f;
          if (u <= t) Cr[u] = keep * Cr[u] + D[u];
        }
        for (int u = 0; u < b; ++u) s.C[t * b + u] = u <= t ? Cr[u] : 0.f;
        s.Av[t] = A;
        s.Bv[t] = Bc;
      }
      for (int u = 0; u < b; ++u) s.Dl[u] = D[u];
      s.Bv[b] = P;
    }
    __syncthreads();

    // ---- K side forward: Z^K ----
    if (KIND == TTT_MLP) {
      for (int j = tid; j < h; j += NT) {
        float acc[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) acc[t] = 0.f;
        for (int k = 0; k < d; ++k) {
          const float w = W1[static_cast<size_t>(k) * h + j];
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) acc[t] = fmaf(s.K[t * d + k], w, acc[t]);
        }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) {
            float v, d1;
            gelu_d(acc[t], p.gelu, v, d1);
            s.A[t * h + j] = v;
            s.G[t * h + j] = d1;
          }
      }
      __syncthreads();
      if (grp < ngrp) {
        float acc[MAXB];
#pragma unroll
        for (int m = 0; m < MAXB; ++m) acc[m] = 0.f;
        for (int j = 0; j < h; ++j) {
          const float w = W2[static_cast<size_t>(j) * d + col];
#pragma unroll
          for (int m = 0; m < MAXB; ++m) {
            const int t = grp + m * ngrp;
            if (t < b) acc[m] = fmaf(s.A[t * h + j], w, acc[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < MAXB; ++m) {
          const int t = grp + m * ngrp;
          if (t < b) s.Z[t * d + col] = acc[m];
        }
      }
    } else {
      if (grp < ngrp) {
        float acc[MAXB];
#pragma unroll
        for (int m = 0; m < MAXB; ++m) acc[m] = 0.f;
        for (int k = 0; k < d; ++k) {
          const float w = W1[static_cast<size_t>(k) * d + col];
#pragma unroll
          for (int m = 0; m < MAXB; ++m) {
            const int t = grp + m * ngrp;
            if (t < b) acc[m] = fmaf(s.K[t * d + k], w, acc[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < MAXB; ++m) {
          const int t = grp + m * ngrp;
          if (t < b) s.Z[t * d + col] = acc[m];
        }
      }
    }
    __syncthreads();

    // ---- LayerNorm forward + backward per token: delta2, E2 = eta * delta2, loss ----
    for (int t = wave; t < b; t += NT / 64) {
      const float z0 = lane < d ? s.Z[t * d + lane] : 0.f;
      const float z1 = lane + 64 < d ? s.Z[t * d + lane + 64] : 0.f;
      RowLN ln = ln_row(z0, z1, lane, d, p.eps);
      float r0 = 0.f, r1 = 0.f;
      if (lane < d) r0 = s.K[t * d + lane] + g0 * ln.xh0 + b0 - s.V[t * d + lane];
      if (lane + 64 < d) r1 = s.K[t * d + lane + 64] + g1 * ln.xh1 + b1 - s.V[t * d + lane + 64];
      const float loss = wave_sum(r0 * r0 + r1 * r1);
      const float gg0 = 2.f * r0 * g0, gg1 = 2.f * r1 * g1;
      const float mg = wave_sum(gg0 + gg1) / d;
      const float mgx = wave_sum(gg0 * ln.xh0 + gg1 * ln.xh1) / d;
      const float et = s.E[t];
      if (lane < d) s.Z[t * d + lane] = et * (gg0 - mg - ln.xh0 * mgx) * ln.rsig;
      if (lane + 64 < d) s.Z[t * d + lane + 64] = et * (gg1 - mg - ln.xh1 * mgx) * ln.rsig;
      if (lane == 0) {
        if (p.loss) p.loss[static_cast<size_t>(bh) * p.T + t0 + t] = loss;
        flag_nonfinite(p.status, loss);
      }
      if (key_out) {
        // z = f(K; W_start) = K + LN(Z^K) = r + V
        if (lane < d) Zg[static_cast<size_t>(t0 + t) * d + lane] = from_f32<IO>(r0 + s.V[t * d + lane]);
        if (lane + 64 < d)
          Zg[static_cast<size_t>(t0 + t) * d + lane + 64] = from_f32<IO>(r1 + s.V[t * d + lane + 64]);
      }
    }
    // S = tril(Q K^T) (eta is carried by the E rows)
    for (int i = tid; i < b * b && !key_out; i += NT) {
      const int t = i / b, u = i % b;
      float acc = 0.f;
      if (u <= t)
        for (int k = 0; k < d; ++k) acc = fmaf(s.Q[t * d + k], s.K[u * d + k], acc);
      s.S[i] = MOM ? acc * s.C[i] : acc;
    }
    __syncthreads();

    if (KIND == TTT_MLP) {
      // ---- E1 = (E2 W2^T) (.) G, in place over G ----
      for (int j = tid; j < h; j += NT) {
        float acc[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) acc[t] = 0.f;
        const float4* w2row = reinterpret_cast<const float4*>(W2 + static_cast<size_t>(j) * d);
        for (int k4 = 0; k4 < d / 4; ++k4) {
          const float4 w = w2row[k4];
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) {
              const float* e = s.Z + t * d + 4 * k4;
              acc[t] = fmaf(e[0], w.x, fmaf(e[1], w.y, fmaf(e[2], w.z, fmaf(e[3], w.w, acc[t]))));
            }
        }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) s.G[t * h + j] *= acc[t];
      }
      __syncthreads();
      if (!key_out) {
      // ---- H^Q = Q W1 - S E1, A^Q = GELU(H^Q) ----
      for (int j = tid; j < h; j += NT) {
        float acc[MAXB];
#pragma unroll
        for (int t = 0; t < MAXB; ++t) acc[t] = 0.f;
        for (int k = 0; k < d; ++k) {
          const float w = W1[static_cast<size_t>(k) * h + j];
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) acc[t] = fmaf(s.Q[t * d + k], w, acc[t]);
        }
        if (MOM) {
          float am[MAXB];
#pragma unroll
          for (int t = 0; t < MAXB; ++t) am[t] = 0.f;
          for (int k = 0; k < d; ++k) {
            const float w = S1[static_cast<size_t>(k) * h + j];
#pragma unroll
            for (int t = 0; t < MAXB; ++t)
              if (t < b) am[t] = fmaf(s.Q[t * d + k], w, am[t]);
          }
#pragma unroll
          for (int t = 0; t < MAXB; ++t)
            if (t < b) acc[t] = s.Av[t] * acc[t] + s.Bv[t] * am[t];
        }
#pragma unroll
        for (int u = 0; u < MAXB; ++u) {
          if (u < b) {
            const float e1 = s.G[u * h + j];
#pragma unroll
            for (int t = 0; t < MAXB; ++t)
              if (t < b && u <= t) acc[t] = fmaf(-s.S[t * b + u], e1, acc[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < MAXB; ++t)
          if (t < b) s.AQ[t * h + j] = gelu(acc[t], p.gelu);
      }
      __syncthreads();
      // ---- S2 = tril(A^Q A^K^T) ----
      for (int i = tid; i < b * b; i += NT) {
        const int t = i / b, u = i % b;
        float acc = 0.f;
        if (u <= t)
          for (int j = 0; j < h; ++j) acc = fmaf(s.AQ[t * h + j], s.A[u * h + j], acc);
        s.S[i] = MOM ? acc * s.C[i] : acc;
      }
      __syncthreads();
      // ---- Z^Q = A^Q W2 - S2 E2 ----
      if (grp < ngrp) {
        float acc[MAXB];
#pragma unroll
        for (int m = 0; m < MAXB; ++m) acc[m] = 0.f;
        for (int j = 0; j < h; ++j) {
          const float w = W2[static_cast<size_t>(j) * d + col];
#pragma unroll
          for (int m = 0; m < MAXB; ++m) {
            const int t = grp + m * ngrp;
            if (t < b) acc[m] = fmaf(s.AQ[t * h + j], w, acc[m]);
          }
        }
        if (MOM) {
          float am[MAXB];
#pragma unroll
          for (int m = 0; m < MAXB; ++m) am[m] = 0.f;
          for (int j = 0; j < h; ++j) {
            const float w = S2[static_cast<size_t>(j) * d + col];
#pragma unroll
            for (int m = 0; m < MAXB; ++m) {
              const int t = grp + m * ngrp;
              if (t < b) am[m] = fmaf(s.AQ[t * h + j], w, am[m]);
            }
          }
#pragma unroll
          for (int m = 0; m < MAXB; ++m) {
            const int t = grp + m * ngrp;
            if (t < b) acc[m] = s.Av[t] * acc[m] + s.Bv[t] * am[m];
          }
        }
#pragma unroll
        for (int m = 0; m < MAXB; ++m) {
          const int t = grp + m * ngrp;
          if (t < b) {
            float a = acc[m];
            for (int u = 0; u <= t; ++u) a = fmaf(-s.S[t * b + u], s.Z[u * d + col], a);
            s.ZQ[t * d + col] = a;
          }
        }
      }
      }  // !key_out
    } else if (!key_out) {
      // ---- Z^Q = Q W - S E ----
      if (grp < ngrp) {
        float acc[MAXB];
#pragma unroll
        for (int m = 0; m < MAXB; ++m) acc[m] = 0.f;
        for (int k = 0; k < d; ++k) {
          const float w = W1[static_cast<size_t>(k) * d + col];
#pragma unroll
          for (int m = 0; m < MAXB; ++m) {
            const int t = grp + m * ngrp;
            if (t < b) acc[m] = fmaf(s.Q[t * d + k], w, acc[m]);
          }
        }
        if (MOM) {
          float am[MAXB];
#pragma unroll
          for (int m = 0; m < MAXB; ++m) am[m] = 0.f;
          for (int k = 0; k < d; ++k) {
            const float w = S1[static_cast<size_t>(k) * d + col];
#pragma unroll
            for (int m = 0; m < MAXB; ++m) {
              const int t = grp + m * ngrp;
              if (t < b) am[m] = fmaf(s.Q[t * d + k], w, am[m]);
            }
          }
#pragma unroll
          for (int m = 0; m < MAXB; ++m) {
            const int t = grp + m * ngrp;
            if (t < b) acc[m] = s.Av[t] * acc[m] + s.Bv[t] * am[m];
          }
        }
#pragma unroll
        for (int m = 0; m < MAXB; ++m) {
          const int t = grp + m * ngrp;
          if (t < b) {
            float a = acc[m];
            for (int u = 0; u <= t; ++u) a = fmaf(-s.S[t * b + u], s.Z[u * d + col], a);
            s.ZQ[t * d + col] = a;
          }
        }
      }
    }
    __syncthreads();

    // ---- output: z = Q + LN(Z^Q) ----
    for (int t = wave; t < b && !key_out; t += NT / 64) {
      const float z0 = lane < d ? s.ZQ[t * d + lane] : 0.f;
      const float z1 = lane + 64 < d ? s.ZQ[t * d + lane + 64] : 0.f;
      RowLN ln = ln_row(z0, z1, lane, d, p.eps);
      float o0 = 0.f, o1 = 0.f;
      if (lane < d) {
        o0 = s.Q[t * d + lane] + g0 * ln.xh0 + b0;
        Zg[static_cast<size_t>(t0 + t) * d + lane] = from_f32<IO>(o0);
      }
      if (lane + 64 < d) {
        o1 = s.Q[t * d + lane + 64] + g1 * ln.xh1 + b1;
        Zg[static_cast<size_t>(t0 + t) * d + lane + 64] = from_f32<IO>(o1);
      }
      const float chk = wave_sum(o0 + o1);
      if (lane == 0) flag_nonfinite(p.status, chk);
    }
    // ---- weight update (chunk end) ----
    if (MOM) {
      // M = A_b M + B_b S - K^T (C_b . E1) ..., S = P_b S - K^T (D_b . E1) ... (old S in both)
      const float Ab = s.Av[b - 1], Bb = s.Bv[b - 1], Pb = s.Bv[b];
      const float* Cb = s.C + (b - 1) * b;
      const size_t n1 = KIND == TTT_MLP ? static_cast<size_t>(d) * h : static_cast<size_t>(d) * d;
      const int w1c = KIND == TTT_MLP ? h : d;
      const float* E1 = KIND == TTT_MLP ? s.G : s.Z;
      for (size_t i = tid; i < n1; i += NT) {
        const int k = static_cast<int>(i / w1c), j = static_cast<int>(i % w1c);
        const float sv = S1[i];
        float am = Ab * W1[i] + Bb * sv, as = Pb * sv;
        for (int t = 0; t < b; ++t) {
          const float ke = s.K[t * d + k] * E1[t * w1c + j];
          am = fmaf(-Cb[t], ke, am);
          as = fmaf(-s.Dl[t], ke, as);
        }
        W1[i] = am;
        S1[i] = as;
      }
      if (KIND == TTT_MLP) {
        for (int i = tid; i < h * d; i += NT) {
          const int j = i / d, cc = i % d;
          const float sv = S2[i];
          float am = Ab * W2[i] + Bb * sv, as = Pb * sv;
          for (int t = 0; t < b; ++t) {
            const float ae = s.A[t * h + j] * s.Z[t * d + cc];
            am = fmaf(-Cb[t], ae, am);
            as = fmaf(-s.Dl[t], ae, as);
          }
          W2[i] = am;
          S2[i] = as;
        }
      }
    } else if (KIND == TTT_MLP) {
      for (int i = tid; i < d * h; i += NT) {
        const int k = i / h, j = i % h;
        float acc = W1[i];
        for (int t = 0; t < b; ++t) acc = fmaf(-s.K[t * d + k], s.G[t * h + j], acc);
        W1[i] = acc;
      }
      for (int i = tid; i < h * d; i += NT) {
        const int j = i / d, cc = i % d;
        float acc = W2[i];
        for (int t = 0; t < b; ++t) acc = fmaf(-s.A[t * h + j], s.Z[t * d + cc], acc);
        W2[i] = acc;
      }
    } else {
      for (int i = tid; i < d * d; i += NT) {
        const int k = i / d, cc = i % d;
        float acc = W1[i];
        for (int t = 0; t < b; ++t) acc = fmaf(-s.K[t * d + k], s.Z[t * d + cc], acc);
        W1[i] = acc;
      }
    }
    __syncthreads();
  }

  if (p.wt_1) {
    float* o1 = p.wt_1 + static_cast<size_t>(bh) * nW1;
    for (size_t i = tid; i < nW1; i += NT) o1[i] = W1[i];
  }
  if (p.wt_2 && nW2) {
    float* o2 = p.wt_2 + static_cast<size_t>(bh) * nW2;
    for (size_t i = tid; i < nW2; i += NT) o2[i] = W2[i];
  }
  if (MOM && p.st_1) {
    for (size_t i = tid; i < nW1; i += NT) p.st_1[static_cast<size_t>(bh) * nW1 + i] = S1[i];
    for (size_t i = tid; i < nW2; i += NT) p.st_2[static_cast<size_t>(bh) * nW2 + i] = S2[i];
  }
}

__global__ void reset_status_kernel(unsigned* status) {
  if (threadIdx.x == 0) *status = 0u;
}

__global__ void copy_status_kernel(const unsigned* src, unsigned* dst) {
  if (threadIdx.x == 0) *dst = *src;
}

}  // namespace

size_t fwd_generic_lds_bytes(int kind, int d, int hid, int chunk, bool momentum) {
  size_t f = 5 * static_cast<size_t>(chunk) * d + 16 + static_cast<size_t>(chunk) * chunk;
  if (kind == TTT_MLP) f += 3 * static_cast<size_t>(chunk) * hid;
  if (momentum) f += static_cast<size_t>(chunk) * chunk + 3 * static_cast<size_t>(chunk) + 1;
  return f * sizeof(float);
}

hipError_t launch_fwd_generic(const ScanParams& p, hipStream_t stream) {
  const bool mom = p.mom != nullptr;
  const size_t lds = fwd_generic_lds_bytes(p.kind, p.d, p.hid, p.chunk, mom);
  const dim3 grid(p.B * p.H), block(NT);
  hipError_t e;
#define TTT_LAUNCH(IO, KIND)                                                              \
  do {                                                                                    \
    auto fn = mom ? fwd_generic_kernel<IO, KIND, true> : fwd_generic_kernel<IO, KIND, false>; \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),                            \
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)); \
    if (e != hipSuccess) return e;                                                        \
    hipLaunchKernelGGL(fn, grid, block, lds, stream, p);                                  \
  } while (0)
  if (p.io == TTT_BF16) {
    if (p.kind == TTT_MLP) TTT_LAUNCH(bf16_t, TTT_MLP); else TTT_LAUNCH(bf16_t, TTT_LINEAR);
  } else {
    if (p.kind == TTT_MLP) TTT_LAUNCH(float, TTT_MLP); else TTT_LAUNCH(float, TTT_LINEAR);
  }
#undef TTT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_reset_status(unsigned* status, hipStream_t stream) {
  hipLaunchKernelGGL(reset_status_kernel, dim3(1), dim3(64), 0, stream, status);
  return hipGetLastError();
}

hipError_t launch_copy_status(const unsigned* src, unsigned* dst, hipStream_t stream) {
  hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(64), 0, stream, src, dst);
  return hipGetLastError();
}

}  // namespace ttt
