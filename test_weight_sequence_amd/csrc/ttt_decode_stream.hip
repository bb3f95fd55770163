// Tuned decode step for the TTT-MLP head shape d = 64, hidden = 256 (fp32 weights, bf16 or
// fp32 q/k/v/z): one token per (batch, head), the mini-batch rule of decoding in "LLM : 빠른
// 논문 리뷰 : End-to-End Test-Time Training for Long Context", section 2.3.2 (the gradient
// step is taken only when the decoded tokens fill a mini-batch), on the layer of "Test-Time
// Training(TTT)과 LLM 메모리", section "TTT layer", Eq. 2/4/5.
//
// The step is bound by HBM traffic: per head it must read W_start and acc (the running
// eta-weighted gradient sum of the chunk) and write acc back, or on the chunk's last token
// write W_start - acc and clear acc. One workgroup of 1024 threads per head issues all of
// its loads at once: each thread holds a 4 x 4 block of each of W1, acc1, W2 and acc2 in
// registers (64 floats, float4 loads, each wave reading whole rows), so every matrix
// crosses HBM exactly once per step and the rest of the step is register arithmetic with
// LDS and cross-lane reductions.
//
//   HK = k W1, AK = GELU, G = GELU';  ZK = AK W2;  E2 = eta' LN-backward(ZK)   (at W_start)
//   E1 = (E2 W2^T) (.) G;  acc1 += k^T E1;  acc2 += AK^T E2
//   HQ = q (W1 - acc1), AQ = GELU;  ZQ = AQ (W2 - acc2);  z = q + LN(ZQ)
// HQ is formed as q (W1 - acc1_before) - (q . k) E1, so its reduction over d runs before E1 is
// known, while wave 0 takes the LayerNorm of ZK; acc2 and acc1 are stored as soon as they are
// final.
#include "ttt_device.hpp"

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int HID = 256;
constexpr int NT = 1024;
constexpr int NWV = NT / 64;  // waves

template <int GELU_KIND>
__device__ __forceinline__ void act_dv(float x, float& v, float& d1) {
  if (GELU_KIND == TTT_GELU_ERF)
    ttt_gelu::gelu_d(x, v, d1);
  else
    gelu_d(x, GELU_KIND, v, d1);
}

template <typename IO, int GELU_KIND>
__global__ void __launch_bounds__(NT) decode_stream_kernel(DecodeParams p) {
  __shared__ float sq[D], sk[D], sv[D], sE2[D];
  __shared__ float sA[HID], sG[HID], sE1[HID], sPQ[HID], sAQ[HID];
  __shared__ float4 red1[NWV][HID / 4];  // [row block][h]: k W1 partials
  __shared__ float4 redq[NWV][HID / 4];  // [row block][h]: q (W1 - acc1) partials (acc1 before this token)
  __shared__ float4 red2[NWV][D / 4];    // [wave][d]: A W2 partials
  __shared__ float sEta, sQK;
  TTT_POISON(sq);
  TTT_POISON(sk);
  TTT_POISON(sv);
  TTT_POISON(sE2);
  TTT_POISON(sA);
  TTT_POISON(sG);
  TTT_POISON(sE1);
  TTT_POISON(sPQ);
  TTT_POISON(sAQ);
  TTT_POISON(red1);
  TTT_POISON(redq);
  TTT_POISON(red2);
  TTT_POISON(sEta);
  TTT_POISON(sQK);
  TTT_POISON_DONE();
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bh = blockIdx.x, hidx = bh % p.H;
  const bool commit = p.pos == p.chunk - 1;

  // W1 / acc1: wave wv holds rows 4 wv .. 4 wv + 3, lane holds columns 4 lane .. 4 lane + 3
  float* W1 = p.ws_1 + static_cast<size_t>(bh) * D * HID;
  float* A1 = p.acc_1 + static_cast<size_t>(bh) * D * HID;
  // W2 / acc2: thread holds rows 4 rb .. 4 rb + 3 (hidden) and columns 4 cg .. 4 cg + 3 (d)
  float* W2 = p.ws_2 + static_cast<size_t>(bh) * HID * D;
  float* A2 = p.acc_2 + static_cast<size_t>(bh) * HID * D;
  const int cg = tid & 15, rb = tid >> 4;
  // loads in the order of first use (W1, W2, acc1, acc2), so that the first products start
  // while the rest of the head's 256 KiB is still arriving
  float4 w1[4], a1[4], w2[4], a2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w1[i] = *reinterpret_cast<const float4*>(W1 + (4 * wv + i) * HID + 4 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) w2[i] = *reinterpret_cast<const float4*>(W2 + (4 * rb + i) * D + 4 * cg);
#pragma unroll
  for (int i = 0; i < 4; ++i) a1[i] = *reinterpret_cast<const float4*>(A1 + (4 * wv + i) * HID + 4 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) a2[i] = *reinterpret_cast<const float4*>(A2 + (4 * rb + i) * D + 4 * cg);
  if (tid < D) {
    const size_t o = static_cast<size_t>(bh) * D + tid;
    sq[tid] = to_f32(static_cast<const IO*>(p.q)[o]);
    sk[tid] = to_f32(static_cast<const IO*>(p.k)[o]);
    sv[tid] = to_f32(static_cast<const IO*>(p.v)[o]);
  }
  if (tid == 0) sEta = p.eta[bh] * p.eta_scale;
  __syncthreads();

  // ---- H^K = k W1 (partial over this wave's four rows) ----
  {
    float4 h = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = sk[4 * wv + i];
      h.x = fmaf(x, w1[i].x, h.x);
      h.y = fmaf(x, w1[i].y, h.y);
      h.z = fmaf(x, w1[i].z, h.z);
      h.w = fmaf(x, w1[i].w, h.w);
    }
    red1[wv][lane] = h;
  }
  __syncthreads();
  if (tid < HID) {
    const float* r = reinterpret_cast<const float*>(red1);
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < NWV; ++b) s += r[b * HID + tid];
    float v, d1;
    act_dv<GELU_KIND>(s, v, d1);
    sA[tid] = v;
    sG[tid] = d1;
  } else if (wv == HID / 64) {
    const float qk = wave_sum(sq[lane] * sk[lane]);
    if (lane == 0) sQK = qk;
  }
  __syncthreads();

  // partial of x W2 (or x (W2 - acc2)) over this thread's four hidden rows, summed over the
  // four row blocks of the wave that share the columns (lanes 16 apart)
  auto w2_partial = [&](const float* x, const float4* m, const float4* sub) {
    float4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = x[4 * rb + i];
      const float4 wv4 = sub ? float4{m[i].x - sub[i].x, m[i].y - sub[i].y, m[i].z - sub[i].z, m[i].w - sub[i].w}
                             : m[i];
      z.x = fmaf(a, wv4.x, z.x);
      z.y = fmaf(a, wv4.y, z.y);
      z.z = fmaf(a, wv4.z, z.z);
      z.w = fmaf(a, wv4.w, z.w);
    }
#pragma unroll
    for (int m2 = 16; m2 <= 32; m2 <<= 1) {
      z.x += __shfl_xor(z.x, m2, 64);
      z.y += __shfl_xor(z.y, m2, 64);
      z.z += __shfl_xor(z.z, m2, 64);
      z.w += __shfl_xor(z.w, m2, 64);
    }
    if (lane < 16) red2[wv][cg] = z;
  };
  // ---- Z^K = A^K W2; the part of H^Q that does not depend on this token's gradient:
  //      q (W1 - acc1), acc1 before this token (H^Q = that - (q . k) E1) ----
  w2_partial(sA, w2, nullptr);
  {
    float4 h = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = sq[4 * wv + i];
      h.x = fmaf(x, w1[i].x - a1[i].x, h.x);
      h.y = fmaf(x, w1[i].y - a1[i].y, h.y);
      h.z = fmaf(x, w1[i].z - a1[i].z, h.z);
      h.w = fmaf(x, w1[i].w - a1[i].w, h.w);
    }
    redq[wv][lane] = h;
  }
  __syncthreads();
  // ---- LayerNorm forward/backward (wave 0, one d per lane): E2 = eta' delta2; meanwhile
  //      waves 4-7 sum the q (W1 - acc1) partials ----
  if (wv == 0) {
    const float* r = reinterpret_cast<const float*>(red2);
    float z = 0.f;
#pragma unroll
    for (int b = 0; b < NWV; ++b) z += r[b * D + lane];
    const float mu = wave_sum(z) * (1.0f / D);
    const float c = z - mu;
    const float rs = 1.0f / sqrtf(wave_sum(c * c) * (1.0f / D) + p.eps);
    const float x = c * rs;
    const float gam = p.gamma[hidx * D + lane], bet = p.beta[hidx * D + lane];
    const float res = sk[lane] + gam * x + bet - sv[lane];
    const float gg = 2.f * res * gam;
    const float mg = wave_sum(gg) * (1.0f / D), mgx = wave_sum(gg * x) * (1.0f / D);
    sE2[lane] = sEta * (gg - mg - x * mgx) * rs;
    const float loss = wave_sum(res * res);
    if (lane == 0) flag_nonfinite(p.status, loss);
  } else if (tid >= HID && tid < 2 * HID) {
    const float* r = reinterpret_cast<const float*>(redq);
    const int j = tid - HID;
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < NWV; ++b) s += r[b * HID + j];
    sPQ[j] = s;
  }
  __syncthreads();

  // ---- E1 = (E2 W2^T) (.) G for this thread's four hidden rows; acc2 += A^K^T E2 (stored
  //      now: nothing after this changes it) ----
  {
    const float4 e = reinterpret_cast<const float4*>(sE2)[cg];
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float t = w2[i].x * e.x;
      t = fmaf(w2[i].y, e.y, t);
      t = fmaf(w2[i].z, e.z, t);
      s[i] = fmaf(w2[i].w, e.w, t);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // sum over the 16 lanes holding the columns of these rows (aligned lane groups)
#pragma unroll
      for (int m2 = 1; m2 < 16; m2 <<= 1) s[i] += __shfl_xor(s[i], m2, 64);
    }
    if (cg == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sE1[4 * rb + i] = s[i] * sG[4 * rb + i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = sA[4 * rb + i];
      a2[i].x = fmaf(a, e.x, a2[i].x);
      a2[i].y = fmaf(a, e.y, a2[i].y);
      a2[i].z = fmaf(a, e.z, a2[i].z);
      a2[i].w = fmaf(a, e.w, a2[i].w);
      const size_t o2 = static_cast<size_t>(4 * rb + i) * D + 4 * cg;
      if (commit) {
        *reinterpret_cast<float4*>(W2 + o2) =
            float4{w2[i].x - a2[i].x, w2[i].y - a2[i].y, w2[i].z - a2[i].z, w2[i].w - a2[i].w};
        *reinterpret_cast<float4*>(A2 + o2) = float4{0.f, 0.f, 0.f, 0.f};
      } else {
        *reinterpret_cast<float4*>(A2 + o2) = a2[i];
      }
    }
  }
  __syncthreads();

  // ---- H^Q = q (W1 - acc1) - (q . k) E1, A^Q = GELU;  acc1 += k^T E1 (stored) ----
  if (tid < HID) {
    const float hq = fmaf(-sQK, sE1[tid], sPQ[tid]);
    sAQ[tid] = GELU_KIND == TTT_GELU_ERF ? ttt_gelu::gelu(hq) : gelu(hq, GELU_KIND);
  }
  {
    const float4 e1 = reinterpret_cast<const float4*>(sE1)[lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float kk = sk[4 * wv + i];
      a1[i].x = fmaf(kk, e1.x, a1[i].x);
      a1[i].y = fmaf(kk, e1.y, a1[i].y);
      a1[i].z = fmaf(kk, e1.z, a1[i].z);
      a1[i].w = fmaf(kk, e1.w, a1[i].w);
      const size_t o1 = static_cast<size_t>(4 * wv + i) * HID + 4 * lane;
      if (commit) {
        *reinterpret_cast<float4*>(W1 + o1) =
            float4{w1[i].x - a1[i].x, w1[i].y - a1[i].y, w1[i].z - a1[i].z, w1[i].w - a1[i].w};
        *reinterpret_cast<float4*>(A1 + o1) = float4{0.f, 0.f, 0.f, 0.f};
      } else {
        *reinterpret_cast<float4*>(A1 + o1) = a1[i];
      }
    }
  }
  __syncthreads();

  // ---- Z^Q = A^Q (W2 - acc2) ----
  w2_partial(sAQ, w2, a2);
  __syncthreads();
  // ---- z = q + LN(Z^Q) ----
  if (wv == 0) {
    const float* r = reinterpret_cast<const float*>(red2);
    float z = 0.f;
#pragma unroll
    for (int b = 0; b < NWV; ++b) z += r[b * D + lane];
    const float mu = wave_sum(z) * (1.0f / D);
    const float c = z - mu;
    const float rs = 1.0f / sqrtf(wave_sum(c * c) * (1.0f / D) + p.eps);
    const float o = sq[lane] + p.gamma[hidx * D + lane] * c * rs + p.beta[hidx * D + lane];
    static_cast<IO*>(p.z)[static_cast<size_t>(bh) * D + lane] = from_f32<IO>(o);
    const float chk = wave_sum(o);
    if (lane == 0) flag_nonfinite(p.status, chk);
  }
}

}  // namespace

bool decode_stream_supported(const DecodeParams& p) {
  return p.kind == TTT_MLP && p.d == D && p.hid == HID;
}

hipError_t launch_decode_stream(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.B * p.H), block(NT);
  const bool tanh_form = p.gelu == TTT_GELU_TANH;
  if (p.io == TTT_BF16) {
    if (tanh_form)
      hipLaunchKernelGGL((decode_stream_kernel<bf16_t, TTT_GELU_TANH>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_stream_kernel<bf16_t, TTT_GELU_ERF>), grid, block, 0, stream, p);
  } else {
    if (tanh_form)
      hipLaunchKernelGGL((decode_stream_kernel<float, TTT_GELU_TANH>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_stream_kernel<float, TTT_GELU_ERF>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ttt
