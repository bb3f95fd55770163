// Tuned outer-loop backward for the TTT-MLP head shape d = 64, hidden = 256, chunk 16, bf16
// Q/K/V/dZ/dQ/dK/dV, fp32 weights (gfx950, bf16 MFMA with fp32 accumulation): the gradients
// of the scan's outputs with respect to its inputs through the inner updates (gradients of
// gradients; the outer loop of "LLM : 빠른 논문 리뷰 : End-to-End Test-Time Training for Long
// Context", section 2.2, applied to the layer of "Test-Time Training(TTT)과 LLM 메모리",
// section "TTT layer", Eq. 2/4/5 with the mini-batch rule of the review's Eq. 5).
//
// One workgroup of 8 waves per (batch, head) walks the chunks backwards, two waves per SIMD
// (each with half of the SIMD's registers, and each able to run while the other waits).
// Wave w owns hidden units [32w, 32w + 32): its slices of the chunk-start weights (read from
// the forward's saved copy) become bf16 MFMA operand tiles, and its slices of dW (the adjoint
// of the chunk-start weights, carried from chunk to chunk) stay in fp32 accumulator registers
// for the whole scan. The per-token phases (LayerNorm forward and backward) run on all waves,
// two tokens per wave and 32 lanes per token. Same register-layout rule and identity-operand transposes as the forward
// MFMA kernels (ttt_mfma_common.hpp).
//
// Forward of one chunk, recomputed from its start weights W1, W2 (E rows carry -eta):
//   HK = K W1, AK = s(HK), G = s'(HK), G2 = s''(HK);  ZK = AK W2
//   per token: xk = LN-normalised ZK, r = K + gamma xk + beta - V, g = 2 r gamma,
//              d2 = rk (g - mean g - xk mean(g xk)), E2 = -eta d2
//   gA = E2 W2^T, E1 = gA (.) G;  P1 = tril(Q K^T);  HQ = Q W1 + P1 E1, AQ = s(HQ), GQ = s'(HQ)
//   P2 = tril(AQ AK^T);  ZQ = AQ W2 + P2 E2;  z = Q + LN(ZQ)
//   chunk-end weights: W1' = W1 + K^T E1, W2' = W2 + AK^T E2
// Adjoints, with dW1', dW2' the adjoint of the chunk-end weights (the carried dW):
//   dZQ = LN backward of dz;  dQ = dz + dHQ W1^T + dP1 K
//   dP2 = tril(dZQ E2^T);  dAQ = dZQ W2^T + dP2 AK;  dHQ = dAQ (.) GQ
//   dP1 = tril(dHQ E1^T);  dE1 = P1^T dHQ + K dW1';  dgA = dE1 (.) G
//   dE2 = P2^T dZQ + dgA W2 + AK dW2'  -> per token: deta, dZK, dK (residual), dV, dgamma, dbeta
//   dAK = dP2^T AQ + E2 dW2'^T + dZK W2^T;  dHK = dAK (.) G + dE1 (.) gA (.) G2
//   dK = (residual) + E1 dW1'^T + dHK W1^T + dP1^T Q
//   dW1 = dW1' + Q^T dHQ + K^T dHK;  dW2 = dW2' + AQ^T dZQ + AK^T dZK + dgA^T E2
// Products over the hidden units are split across the waves and their [chunk x d] partials
// summed in LDS in a fixed order, so the result is deterministic.
#include "ttt_mfma_common.hpp"

namespace ttt {
namespace {

using namespace mfma;

constexpr int NW = 8;           // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;
constexpr int HS = HID / NW;    // hidden units per wave
constexpr int NHT = HS / 16;    // h tiles per wave
constexpr int NKH = NHT / 2;    // 32-wide k-steps over a wave's hidden slice
constexpr int TS = BC + 8;  // padded row stride of the [16 x 16] dP1 arrays
constexpr int NLN = 4;          // waves 0..3 run the per-token phases: 16 lanes per token
static_assert(NLN * 64 == BC * 16, "LayerNorm phases: 16 lanes per token");

// One chunk's rows.
struct BStage {
  alignas(16) __bf16 K[BC * RS];
  alignas(16) __bf16 Q[BC * RS];
  alignas(16) __bf16 V[BC * RS];
  alignas(16) __bf16 dZ[BC * RS];
  float eta[BC];
};

// Cross-wave partial sums of [chunk x d] products: per wave, per d tile, the four rows of
// its accumulator tile, lane-rotated by 16 per row so that both the writes (one row, all
// lanes) and the LayerNorm reads (four tokens of 16 lanes) touch 64 distinct banks.
struct Partials {
  float v[NW][NDT][4][64];
};
__device__ __forceinline__ int prot(int r, int lane) { return (lane + 16 * r) & 63; }

struct BSmem {
  BStage st[2];                       // chunk c lives in st[c & 1]
  alignas(16) __bf16 E2[BC * RS];     // E2 (= -eta d2): [token][d]
  alignas(16) __bf16 dZQ[BC * RS];
  alignas(16) __bf16 dZK[BC * RS];
  alignas(16) __bf16 dP1r[BC * TS];   // dP1 [t][u]
  alignas(16) __bf16 dP1c[BC * TS];   // dP1 [u][t]
  float dKres[BC * D];                // residual part of dK, [t][d]
  float dp1p[NW][4][64];              // per-wave dP1 partials (accumulator-tile order)
  Partials red[3];                    // [0]: ZK, ZQ, dE2;  [1]: dQ;  [2]: dK
  float dgb[NW][2][D];                // per-wave dgamma / dbeta partials
};

template <int GELU_KIND>
__device__ __forceinline__ void act_d2(float x, float& v, float& d1, float& d2) {
  if (GELU_KIND == TTT_GELU_ERF) {
    ttt_gelu::gelu_d2(x, v, d1, d2);
  } else {
    const Gelu3 r = gelu_d2(x, GELU_KIND);
    v = r.v;
    d1 = r.d1;
    d2 = r.d2;
  }
}

// The identity operand passed through an empty asm statement: transposes made in different
// phases are then distinct values, so the compiler recomputes them instead of keeping every
// transposed weight tile live across the whole chunk.
__device__ __forceinline__ bf16x4 fresh(bf16x4 I4) {
  asm volatile("" : "+v"(I4));
  return I4;
}
__device__ __forceinline__ f4 wide(bf16x4 x) { return f4{bf(x[0]), bf(x[1]), bf(x[2]), bf(x[3])}; }
__device__ __forceinline__ bf16x4 tr(bf16x4 x, bf16x4 I4) { return cvt4(mfma16(x, I4, zero4())); }
// k-step ks over a wave's hidden slice from an array of [.. x h] tiles
__device__ __forceinline__ bf16x8 hcat(const bf16x4 (&x)[NHT], int ks) { return cat(x[2 * ks], x[2 * ks + 1]); }

// The chunk-start weights of one wave in the transposed tile orientations: W1^T tiles
// (C[h][d]: lane holds W1[d][h .. h+3], four consecutive hidden units of one row) and W2^T
// tiles (C[d][h]: lane holds W2[h][d .. d+3]), so every lane reads 16 contiguous bytes per
// tile from the row-major [d][h] / [h][d] saved copy.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void wT_load(const float* w1, const float* w2, int g, int c16, int hs,
                                        f4 (&W1T)[NHT][NDT], f4 (&W2T)[NDT][NHT]) {
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w1), 0, D * HID * 4, kBufFlags);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w2), 0, D * HID * 4, kBufFlags);
  const int v1 = (c16 * HID + hs + 4 * g) * 4, v2 = ((hs + c16) * D + 4 * g) * 4;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      W1T[ht][dt] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r1, v1, (16 * dt * HID + 16 * ht) * 4, 0));
      W2T[dt][ht] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r2, v2, (16 * ht * D + 16 * dt) * 4, 0));
    }
}

// rows of a [token][d] LDS array as the A operand of a contraction over d (permuted k order)
__device__ __forceinline__ void rows2(const __bf16* a, int c16, int g, bf16x8 (&o)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    o[ks] = cat(lds4(&a[c16 * RS + 32 * ks + 4 * g]), lds4(&a[c16 * RS + 32 * ks + 16 + 4 * g]));
}
// [token][d] LDS array as the B operand of a contraction over tokens (k = token, n = d),
// through the transposing LDS load
__device__ __forceinline__ bf16x4 colsT(const __bf16* a, int dt, int c16, int g) {
  return tgroup(a, RS, dt, g, c16);
}
// four d values of one token, [token][d] array
__device__ __forceinline__ float red_sum(const Partials& P, int i, int t, int c16) {
  float s = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) s += P.v[ww][i][t & 3][prot(t & 3, 16 * (t >> 2) + c16)];
  return s;
}
// Per-token phases: 32 lanes per token (two tokens per wave); lane value i is d = 32 i + lane % 32.
constexpr int PL = 2;
__device__ __forceinline__ float sum32(float v) {
  v = sum16(v);
  // add the other row of the 32-lane half (lane ^ 16), through the LDS crossbar (no memory)
  return v + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ __forceinline__ LnStats ln_stats32(const float (&z)[PL], float eps) {
  const float mu = sum32(z[0] + z[1]) * (1.0f / D);
  float var = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) var += (z[i] - mu) * (z[i] - mu);
  var = sum32(var) * (1.0f / D);
  return LnStats{mu, __builtin_amdgcn_rsqf(var + eps)};
}
__device__ __forceinline__ void put_tile(Partials& P, int w, int dt, int lane, f4 v) {
#pragma unroll
  for (int r = 0; r < 4; ++r) P.v[w][dt][r][prot(r, lane)] = v[r];
}
__device__ __forceinline__ f4 get_tile(const Partials& P, int w, int dt, int lane) {
  f4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = P.v[w][dt][r][prot(r, lane)];
  return v;
}

template <int GELU_KIND>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_mfma_kernel(BwdParams p) {
  __shared__ BSmem sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.x, hidx = bh % p.H;
  const int hs = w * HS;
  const int T = p.T, nchunks = T / BC;
  bf16x4 I4 = make_ident(g, c16).i4;

  float* work = p.work + static_cast<size_t>(bh) * bwd_work_floats_per_head(TTT_MLP, D, HID, BC);

  // ---- carried adjoint of the chunk-end weights ----
  f4 dW1c[NDT][NHT], dW2c[NHT][NDT];
  if (p.dwt_1) {
    wtiles_load<NHT>(p.dwt_1 + static_cast<size_t>(bh) * D * HID,
                     p.dwt_2 + static_cast<size_t>(bh) * HID * D, g, c16, hs, dW1c, dW2c);
  } else {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        dW1c[dt][ht] = zero4();
        dW2c[ht][dt] = zero4();
      }
  }

  // LayerNorm lane mapping (all waves): token 4w + lane/16, 16 lanes per token, d = 16 i + lane%16
  const int ln_t = 2 * w + (lane >> 5), c32 = lane & 31;
  float gam[PL], bet[PL], dgam[PL], dbet[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    gam[i] = p.gamma[hidx * D + 32 * i + c32];
    bet[i] = p.beta[hidx * D + 32 * i + c32];
    dgam[i] = 0.f;
    dbet[i] = 0.f;
  }

  const size_t io_off = static_cast<size_t>(bh) * T * D;
  const __bf16* Qg = static_cast<const __bf16*>(p.Q) + io_off;
  const __bf16* Kg = static_cast<const __bf16*>(p.K) + io_off;
  const __bf16* Vg = static_cast<const __bf16*>(p.V) + io_off;
  const __bf16* dZg = static_cast<const __bf16*>(p.dZ) + io_off;
  __bf16* dQg = static_cast<__bf16*>(p.dQ) + io_off;
  __bf16* dKg = static_cast<__bf16*>(p.dK) + io_off;
  __bf16* dVg = static_cast<__bf16*>(p.dV) + io_off;
  const float* etag = p.eta + static_cast<size_t>(bh) * T;
  const float* saved = p.saved + static_cast<size_t>(bh) * nchunks * (2 * D * HID);

  // Row staging: thread -> token st_t, four consecutive d from st_d.
  const int st_t = tid >> 4, st_d = (tid & 15) * 4;
  auto gload = [&](int chunk, uint2& kk, uint2& qq, uint2& vv, uint2& zz, float& e) {
    const size_t off = (static_cast<size_t>(chunk) * BC + st_t) * D + st_d;
    if (tid >= NLN * 64) return;
    kk = *reinterpret_cast<const uint2*>(Kg + off);
    qq = *reinterpret_cast<const uint2*>(Qg + off);
    vv = *reinterpret_cast<const uint2*>(Vg + off);
    zz = *reinterpret_cast<const uint2*>(dZg + off);
    e = tid < BC ? etag[chunk * BC + tid] : 0.f;
  };
  auto stage_write = [&](BStage& S, uint2 kk, uint2 qq, uint2 vv, uint2 zz, float e) {
    if (tid >= NLN * 64) return;
    *reinterpret_cast<uint2*>(&S.K[st_t * RS + st_d]) = kk;
    *reinterpret_cast<uint2*>(&S.Q[st_t * RS + st_d]) = qq;
    *reinterpret_cast<uint2*>(&S.V[st_t * RS + st_d]) = vv;
    *reinterpret_cast<uint2*>(&S.dZ[st_t * RS + st_d]) = zz;
    if (tid < BC) S.eta[tid] = e * p.eta_scale;
  };
  // Final dQ, dK of chunk cc from the per-wave partials (four elements per thread).
  auto emit_dqdk = [&](int cc) {
    if (tid >= NLN * 64) return;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = st_t, d = st_d + k;
      const int dt = d >> 4, n = d & 15, r = t & 3, l = 16 * (t >> 2) + n;
      float q = 0.f, kk = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        q += sm.red[1].v[ww][dt][r][prot(r, l)];
        kk += sm.red[2].v[ww][dt][r][prot(r, l)];
      }
      const size_t gi = static_cast<size_t>(cc * BC + t) * D + d;
      dQg[gi] = (__bf16)q;
      dKg[gi] = (__bf16)kk;
    }
  };

  {
    uint2 kk, qq, vv, zz;
    float e;
    gload(nchunks - 1, kk, qq, vv, zz, e);
    stage_write(sm.st[(nchunks - 1) & 1], kk, qq, vv, zz, e);
  }
  __syncthreads();

  for (int c = nchunks - 1; c >= 0; --c) {
    BStage& S = sm.st[c & 1];
    const int t0 = c * BC;
    const bool has_next = c > 0;
    // next (earlier) chunk's rows, staged after the first LayerNorm
    uint2 nk{}, nq{}, nv{}, nz{};
    float ne = 0.f;
    if (has_next) gload(c - 1, nk, nq, nv, nz, ne);

    // this chunk's start weights, as bf16 operand tiles in both orientations: the transposed
    // ones straight from memory, the others by one identity transpose each
    bf16x4 W1b[NDT][NHT], W2b[NHT][NDT], W1T[NHT][NDT], W2T[NDT][NHT];
    {
      f4 Wn1[NHT][NDT], Wn2[NDT][NHT];
      wT_load(saved + static_cast<size_t>(c) * 2 * D * HID,
              saved + static_cast<size_t>(c) * 2 * D * HID + D * HID, g, c16, hs, Wn1, Wn2);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          W1T[ht][dt] = cvt4(Wn1[ht][dt]);
          W2T[dt][ht] = cvt4(Wn2[dt][ht]);
        }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          W1b[dt][ht] = tr(W1T[ht][dt], I4);
          W2b[ht][dt] = tr(W2T[dt][ht], I4);
        }
    }

    bf16x8 aK[2], aQ[2];
    rows2(S.K, c16, g, aK);
    rows2(S.Q, c16, g, aQ);

    // ================= A: K side and Q W1 =================
    // GELU' and GELU'' of H^K are kept in bf16: every product they enter is rounded to bf16
    bf16x4 akR[NHT], akT[NHT], gk[NHT], gk2[NHT];
    f4 hq[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 acc = zero4(), accq = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 wb = cat(W1b[2 * ks][ht], W1b[2 * ks + 1][ht]);
        acc = mfma32(aK[ks], wb, acc);
        accq = mfma32(aQ[ks], wb, accq);
      }
      hq[ht] = accq;
      f4 a, d1v, d2v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v, d1, d2;
        act_d2<GELU_KIND>(acc[r], v, d1, d2);
        a[r] = v;
        d1v[r] = d1;
        d2v[r] = d2;
      }
      akR[ht] = cvt4(a);
      gk[ht] = cvt4(d1v);
      gk2[ht] = cvt4(d2v);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) akT[ht] = tr(akR[ht], I4);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks)
        acc = mfma32(hcat(akT, ks), cat(W2b[2 * ks][dt], W2b[2 * ks + 1][dt]), acc);
      put_tile(sm.red[0], w, dt, lane, acc);
    }
    // P1 both ways: s1[u][t] = K_u . Q_t (A operand: P1), p1[t][u] (A operand: P1^T)
    bf16x4 s1a, p1a;
    {
      f4 s1 = zero4(), p1 = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        s1 = mfma32(aK[ks], aQ[ks], s1);
        p1 = mfma32(aQ[ks], aK[ks], p1);
      }
      f4 m1, m2;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m1[r] = (4 * g + r) <= c16 ? s1[r] : 0.f;
        m2[r] = c16 <= (4 * g + r) ? p1[r] : 0.f;
      }
      s1a = cvt4(m1);
      p1a = cvt4(m2);
    }
    __syncthreads();  // ---- 1

    // ================= B: inner-gradient LayerNorm of Z^K; dQ, dK of chunk c + 1; staging
    // of chunk c - 1 =================
    float xk[PL], rk_[PL], d2k[PL], rsk, mgxk, etak;
    {
      const int t = ln_t;
      float z[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) z[i] = red_sum(sm.red[0], 2 * i + (c32 >> 4), t, c32 & 15);
      const LnStats ls = ln_stats32(z, p.eps);
      float sg = 0.f, sgx = 0.f, gg[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 32 * i + c32;
        xk[i] = (z[i] - ls.mu) * ls.rs;
        rk_[i] = bf(S.K[t * RS + d]) + gam[i] * xk[i] + bet[i] - bf(S.V[t * RS + d]);
        gg[i] = 2.f * rk_[i] * gam[i];
        sg += gg[i];
        sgx += gg[i] * xk[i];
      }
      const float mg = sum32(sg) * (1.0f / D);
      mgxk = sum32(sgx) * (1.0f / D);
      rsk = ls.rs;
      etak = S.eta[t];
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 32 * i + c32;
        d2k[i] = (gg[i] - mg - xk[i] * mgxk) * rsk;
        const __bf16 e = (__bf16)(-etak * d2k[i]);
        sm.E2[t * RS + d] = e;
      }
    }
    if (c + 1 < nchunks) emit_dqdk(c + 1);
    if (has_next) stage_write(sm.st[(c - 1) & 1], nk, nq, nv, nz, ne);
    __syncthreads();  // ---- 2

    // ================= C: E1, H^Q, A^Q, Z^Q =================
    I4 = fresh(I4);
    bf16x8 aE[2];
    rows2(sm.E2, c16, g, aE);
    bf16x4 e1R[NHT], e1T[NHT], aqR[NHT], aqT[NHT], gq[NHT], gg2[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 ga = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        ga = mfma32(aE[ks], cat(W2T[2 * ks][ht], W2T[2 * ks + 1][ht]), ga);
      e1R[ht] = cvt4(ga * wide(gk[ht]));
      gg2[ht] = cvt4(ga * wide(gk2[ht]));
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const f4 h = mfma16(s1a, e1R[ht], hq[ht]);
      f4 a, d1v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v, d1;
        act_d<GELU_KIND>(h[r], v, d1);
        a[r] = v;
        d1v[r] = d1;
      }
      aqR[ht] = cvt4(a);
      gq[ht] = cvt4(d1v);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      aqT[ht] = tr(aqR[ht], I4);
      e1T[ht] = tr(e1R[ht], I4);
    }
    // P2 over this wave's hidden slice, both ways
    bf16x4 s2a, p2a;
    {
      f4 s2 = zero4(), p2 = zero4();
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks) {
        s2 = mfma32(hcat(akT, ks), hcat(aqT, ks), s2);
        p2 = mfma32(hcat(aqT, ks), hcat(akT, ks), p2);
      }
      f4 m1, m2;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m1[r] = (4 * g + r) <= c16 ? s2[r] : 0.f;
        m2[r] = c16 <= (4 * g + r) ? p2[r] : 0.f;
      }
      s2a = cvt4(m1);
      p2a = cvt4(m2);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 acc = mfma16(s2a, colsT(sm.E2, dt, c16, g), zero4());
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks)
        acc = mfma32(hcat(aqT, ks), cat(W2b[2 * ks][dt], W2b[2 * ks + 1][dt]), acc);
      put_tile(sm.red[0], w, dt, lane, acc);
    }
    __syncthreads();  // ---- 3

    // ================= D: output LayerNorm backward =================
    {
      const int t = ln_t;
      float z[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) z[i] = red_sum(sm.red[0], 2 * i + (c32 >> 4), t, c32 & 15);
      const LnStats ls = ln_stats32(z, p.eps);
      float x[PL], v[PL], sv = 0.f, svx = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 32 * i + c32;
        x[i] = (z[i] - ls.mu) * ls.rs;
        const float o = bf(S.dZ[t * RS + d]);
        dgam[i] += o * x[i];
        dbet[i] += o;
        v[i] = o * gam[i];
        sv += v[i];
        svx += v[i] * x[i];
      }
      const float mv = sum32(sv) * (1.0f / D), mvx = sum32(svx) * (1.0f / D);
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 32 * i + c32;
        const __bf16 e = (__bf16)((v[i] - mv - x[i] * mvx) * ls.rs);
        sm.dZQ[t * RS + d] = e;
      }
    }
    __syncthreads();  // ---- 4

    // ================= E: Q-side adjoints, dE1, dE2 partial, dW terms =================
    I4 = fresh(I4);
    // (operands staged in LDS are read again rather than kept in registers across barriers)
    rows2(sm.E2, c16, g, aE);
    rows2(S.K, c16, g, aK);
    bf16x8 aZ[2];
    rows2(sm.dZQ, c16, g, aZ);
    // dP2 both ways: dp2[t][u] (A operand: dP2^T), dp2t[u][t] (A operand: dP2)
    bf16x4 dp2a, dp2ta;
    {
      f4 dp2 = zero4(), dp2t = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dp2 = mfma32(aZ[ks], aE[ks], dp2);
        dp2t = mfma32(aE[ks], aZ[ks], dp2t);
      }
      f4 m1, m2;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m1[r] = c16 <= (4 * g + r) ? dp2[r] : 0.f;
        m2[r] = (4 * g + r) <= c16 ? dp2t[r] : 0.f;
      }
      dp2a = cvt4(m1);
      dp2ta = cvt4(m2);
    }
    bf16x4 dhqR[NHT], dhqT[NHT], dgR[NHT], dgT[NHT];
    f4 dak[NHT], dhk[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      // dAQ = dZQ W2^T + dP2 AK ; dHQ = dAQ (.) GQ
      f4 da = mfma16(dp2ta, akR[ht], zero4());
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        da = mfma32(aZ[ks], cat(W2T[2 * ks][ht], W2T[2 * ks + 1][ht]), da);
      dhqR[ht] = cvt4(da * wide(gq[ht]));
      // dAK, first two terms: dP2^T AQ + E2 dW2'^T
      f4 a2 = mfma16(dp2a, aqR[ht], zero4());
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        a2 = mfma32(aE[ks], cat(tr(cvt4(dW2c[ht][2 * ks]), I4), tr(cvt4(dW2c[ht][2 * ks + 1]), I4)), a2);
      dak[ht] = a2;
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) dhqT[ht] = tr(dhqR[ht], I4);
    // dP1 partial over this wave's hidden slice: dHQ E1^T, [t][u]
    {
      f4 dp1 = zero4();
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks) dp1 = mfma32(hcat(dhqT, ks), hcat(e1T, ks), dp1);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.dp1p[w][r][lane] = c16 <= (4 * g + r) ? dp1[r] : 0.f;
    }
    // dE1 = P1^T dHQ + K dW1';  dgA = dE1 (.) G;  dHK (second-order part) = dE1 (.) gA G2
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 de = mfma16(p1a, dhqR[ht], zero4());
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        de = mfma32(aK[ks], cat(cvt4(dW1c[2 * ks][ht]), cvt4(dW1c[2 * ks + 1][ht])), de);
      dgR[ht] = cvt4(de * wide(gk[ht]));
      dhk[ht] = de * wide(gg2[ht]);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) dgT[ht] = tr(dgR[ht], I4);
    // per d tile: dE2 partial = P2^T dZQ + dgA W2 + AK dW2', dQ partial = dHQ W1^T and the
    // first dK term E1 dW1'^T (all before dW takes this chunk's terms)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 de2 = mfma16(p2a, colsT(sm.dZQ, dt, c16, g), zero4());
      f4 dq = zero4(), dk = zero4();
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks) {
        de2 = mfma32(hcat(dgT, ks), cat(W2b[2 * ks][dt], W2b[2 * ks + 1][dt]), de2);
        de2 = mfma32(hcat(akT, ks), cat(cvt4(dW2c[2 * ks][dt]), cvt4(dW2c[2 * ks + 1][dt])), de2);
        dq = mfma32(hcat(dhqT, ks), cat(W1T[2 * ks][dt], W1T[2 * ks + 1][dt]), dq);
        dk = mfma32(hcat(e1T, ks),
                    cat(tr(cvt4(dW1c[dt][2 * ks]), I4), tr(cvt4(dW1c[dt][2 * ks + 1]), I4)), dk);
      }
      put_tile(sm.red[0], w, dt, lane, de2);
      put_tile(sm.red[1], w, dt, lane, dq);
      put_tile(sm.red[2], w, dt, lane, dk);
    }
    // this chunk's direct dW terms
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x4 qt = colsT(S.Q, dt, c16, g);
      const bf16x4 zq = colsT(sm.dZQ, dt, c16, g);
      const bf16x4 e2 = colsT(sm.E2, dt, c16, g);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        dW1c[dt][ht] = mfma16(qt, dhqR[ht], dW1c[dt][ht]);
        dW2c[ht][dt] = mfma16(aqR[ht], zq, dW2c[ht][dt]);
        dW2c[ht][dt] = mfma16(dgR[ht], e2, dW2c[ht][dt]);
      }
    }
    __syncthreads();  // ---- 5

    // ================= F: inner-gradient backward per token; dP1 =================
    {
      const int t = ln_t;
      float de[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) de[i] = -red_sum(sm.red[0], 2 * i + (c32 >> 4), t, c32 & 15);  // adjoint of eta d2
      float sq = 0.f, su = 0.f, sux = 0.f, u[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        sq += de[i] * d2k[i];
        u[i] = etak * de[i];
        su += u[i];
        sux += u[i] * xk[i];
      }
      const float deta = sum32(sq) * p.eta_scale;
      const float mu = sum32(su) * (1.0f / D), mux = sum32(sux) * (1.0f / D);
      float suq = 0.f, dx[PL], dr[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        suq += u[i] * d2k[i];
        const float ggi = 2.f * rk_[i] * gam[i];
        const float dg = rsk * (u[i] - mu - xk[i] * mux);
        dx[i] = -rsk * (u[i] * mgxk + ggi * mux);
        dr[i] = 2.f * gam[i] * dg;
        dgam[i] += 2.f * rk_[i] * dg + dr[i] * xk[i];
        dbet[i] += dr[i];
        dx[i] += gam[i] * dr[i];
      }
      const float ds = -rsk * sum32(suq);
      float sdx = 0.f, sdxx = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        sdx += dx[i];
        sdxx += dx[i] * xk[i];
      }
      const float mdx = sum32(sdx) * (1.0f / D), mdxx = sum32(sdxx) * (1.0f / D);
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 32 * i + c32;
        const __bf16 e = (__bf16)(rsk * (dx[i] - mdx - xk[i] * mdxx) + ds * xk[i] * (1.0f / D));
        sm.dZK[t * RS + d] = e;
        sm.dKres[t * D + d] = dr[i];
        dVg[static_cast<size_t>(t0 + t) * D + d] = (__bf16)(-dr[i]);
      }
      if (c32 == 0) {
        p.deta[static_cast<size_t>(bh) * T + t0 + t] = deta;
        flag_nonfinite(p.status, deta);
      }
    }
    if (tid < NLN * 64) {
      // dP1 = sum of the waves' partials, as two bf16 operand layouts
      const int t = tid >> 4, u = tid & 15;
      const int r = t & 3, l = 16 * (t >> 2) + u;
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) s += sm.dp1p[ww][r][l];
      const __bf16 e = (__bf16)s;
      sm.dP1r[t * TS + u] = e;
      sm.dP1c[u * TS + t] = e;
    }
    __syncthreads();  // ---- 6

    // ================= G: dAK, dHK, dK, remaining dW terms =================
    I4 = fresh(I4);
    bf16x8 aZK[2];
    rows2(sm.dZK, c16, g, aZK);
    bf16x4 dhkR[NHT], dhkT[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 da = dak[ht];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        da = mfma32(aZK[ks], cat(W2T[2 * ks][ht], W2T[2 * ks + 1][ht]), da);
      dhkR[ht] = cvt4(dhk[ht] + da * wide(gk[ht]));
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) dhkT[ht] = tr(dhkR[ht], I4);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 dk = get_tile(sm.red[2], w, dt, lane);
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks)
        dk = mfma32(hcat(dhkT, ks), cat(W1T[2 * ks][dt], W1T[2 * ks + 1][dt]), dk);
      if (dt == w) {
        // the terms not split over hidden units, one d tile per wave: the residual and
        // dP1^T Q into dK, dz and dP1 K into dQ
        dk = mfma16(lds4(&sm.dP1c[c16 * TS + 4 * g]), colsT(S.Q, dt, c16, g), dk);
#pragma unroll
        for (int r = 0; r < 4; ++r) dk[r] += sm.dKres[(4 * g + r) * D + 16 * dt + c16];
        f4 dq = get_tile(sm.red[1], w, dt, lane);
        dq = mfma16(lds4(&sm.dP1r[c16 * TS + 4 * g]), colsT(S.K, dt, c16, g), dq);
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[r] += bf(S.dZ[(4 * g + r) * RS + 16 * dt + c16]);
        put_tile(sm.red[1], w, dt, lane, dq);
      }
      put_tile(sm.red[2], w, dt, lane, dk);
      const bf16x4 kt = colsT(S.K, dt, c16, g);
      const bf16x4 zkt = colsT(sm.dZK, dt, c16, g);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        dW1c[dt][ht] = mfma16(kt, dhkR[ht], dW1c[dt][ht]);
        dW2c[ht][dt] = mfma16(akR[ht], zkt, dW2c[ht][dt]);
      }
    }
    __syncthreads();  // ---- 7
  }
  emit_dqdk(0);

  // dW of the first chunk's start = dW0 of this head; dgamma / dbeta partials
  wtiles_store<NHT>(work, work + D * HID, g, c16, hs, dW1c, dW2c);
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    // sum over the two tokens of this wave (lanes with equal lane%32)
    float a = dgam[i], b = dbet[i];
    a += __shfl_xor(a, 32, 64);
    b += __shfl_xor(b, 32, 64);
    if (lane < 32) {
      sm.dgb[w][0][32 * i + c32] = a;
      sm.dgb[w][1][32 * i + c32] = b;
    }
  }
  __syncthreads();
  if (tid < 2 * D) {
    const int k = tid >> 6, d = tid & 63;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += sm.dgb[ww][k][d];
    p.dgb[static_cast<size_t>(bh) * 2 * D + k * D + d] = s;
  }
}

}  // namespace

bool bwd_mfma_supported(const BwdParams& p) {
  return p.kind == TTT_MLP && p.d == D && p.hid == HID && p.chunk == BC && p.io == TTT_BF16;
}

hipError_t launch_bwd_mfma(const BwdParams& p, hipStream_t stream) {
  const dim3 grid(p.B * p.H), block(NT);
  if (p.gelu == TTT_GELU_TANH)
    hipLaunchKernelGGL(bwd_mfma_kernel<TTT_GELU_TANH>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_mfma_kernel<TTT_GELU_ERF>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace ttt
