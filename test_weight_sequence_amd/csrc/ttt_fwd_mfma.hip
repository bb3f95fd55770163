// Tuned forward scan for the TTT-MLP head shape d = 64, hidden = 256, chunk 16, bf16
// Q/K/V/Z, fp32 fast weights (gfx950, bf16 MFMA with fp32 accumulation).
//
// One persistent workgroup of NW waves per (batch, head); wave w owns hidden units
// [w*HS, (w+1)*HS), HS = 256 / NW. The fp32 fast weights never leave registers: each wave
// keeps its slice of W1 (d x h) and W2 (h x d) as 16x16 MFMA accumulator tiles that the
// chunk-end update accumulates into.
//
// Register-layout rule used throughout: an MFMA accumulator tile C[m][n] puts m on
// (lane/16)*4 + r and n on lane%16. A tile can feed another MFMA as an operand only
// through its m axis as the contraction index. W1 is contracted over d (its rows) and
// W2 over h (its rows); the one product that contracts W2 over d (E2 W2^T) uses bf16
// tiles of W2^T made each chunk by an MFMA with the identity matrix, which transposes
// bf16 values exactly. Two tiles stacked along m give the 8 k-values of a 16x16x32
// operand in a permuted k order, and the other operand is read in the same permuted
// order. Activations needed in the other orientation are transposed the same way.
//
// Per chunk (E = eta-scaled, negated rows; all at the chunk-start weights):
//   H^K = K W1 -> A^K = GELU, G = GELU'      Z^K = A^K W2 (partial per wave, summed in LDS)
//   LN fwd/bwd of Z^K per token -> En2 = -eta * delta2 (LDS, bf16)
//   E1n = (En2 W2^T) (.) G
//   H^Q = Q W1 + tril(Q K^T) E1n,  A^Q = GELU(H^Q)
//   Z^Q = A^Q W2 + tril(A^Q A^K^T) En2 (partial per wave, summed in LDS), z = Q + LN(Z^Q)
//   W1 += K^T E1n,  W2 += A^K^T En2
// (dual form of the per-token rule on the page "Test-Time Training(TTT)과 LLM 메모리",
// section "TTT layer", Eq. 2/4/5; mini-batch rule of the E2E paper review, section 2.3,
// Eq. 5.)
#include "ttt_mfma_common.hpp"

namespace ttt {
namespace {

using namespace mfma;

template <int NW>
struct Smem {
  Stage st[3];                   // chunk c lives in st[c % 3]
  float red[2][NW][NDT][4][PS];  // [0]: Z^K partials, [1]: Z^Q partials (64 used per row)
  alignas(16) __bf16 E2[BC * RS];  // En2, [token][d]
};

template <int GELU_KIND, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
fwd_mfma_kernel(ScanParams p) {
  constexpr int NT = 64 * NW;
  constexpr int HS = HID / NW;     // hidden units per wave
  constexpr int NHT = HS / 16;     // h tiles per wave
  constexpr int NKH = NHT / 2;     // 32-wide k-steps over this wave's h slice
  constexpr int EPT = BC * D / NT; // staged elements per thread and tensor
  // LayerNorm: waves 0..3, 4 tokens per wave, 16 lanes per token, 4 d values per lane
  constexpr int DPL = D / 16;
  static_assert(NW == 8, "LayerNorm of Z^K runs on waves 0..3 while waves 4..7 emit the previous chunk");
  static_assert(NHT % 2 == 0 && EPT * NT == BC * D, "wave split");
  using SV = StageVec<EPT>;
  using LdT = typename SV::T;

  __shared__ Smem<NW> sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.x, hidx = bh % p.H;
  const int hs = w * HS;
  const int T = p.T, nchunks = T / BC;
  const bool per_seq = (p.flags & TTT_W0_PER_SEQ) != 0;

  // ---- fast weights: fp32 accumulator tiles ----
  f4 W1c[NDT][NHT], W2c[NHT][NDT];
  {
    const size_t wh = per_seq ? static_cast<size_t>(bh) : static_cast<size_t>(hidx);
    const float* w1 = p.w0_1 + wh * D * HID;
    const float* w2 = p.w0_2 + wh * HID * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 16 * dt + 4 * g + r, h = hs + 16 * ht + c16;
          W1c[dt][ht][r] = w1[d * HID + h];
          const int h2 = hs + 16 * ht + 4 * g + r, d2 = 16 * dt + c16;
          W2c[ht][dt][r] = w2[h2 * D + d2];
        }
  }
  // identity operand for exact transposes (B[k][n] = [k == n], k = 4g + j, n = lane%16)
  const bf16x4 I4 = make_ident(g, c16).i4;

  // LayerNorm lane mapping (waves 0..3 for Z^K): token ln_t = 4w + lane/16, d = 16 i + lane%16
  const bool ln_wave = w < 4;
  const int ln_t = 4 * w + g;
  float gam[DPL], bet[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    gam[i] = p.gamma[hidx * D + 16 * i + c16];
    bet[i] = p.beta[hidx * D + 16 * i + c16];
  }

  const __bf16* Qg = static_cast<const __bf16*>(p.Q) + static_cast<size_t>(bh) * T * D;
  const __bf16* Kg = static_cast<const __bf16*>(p.K) + static_cast<size_t>(bh) * T * D;
  const __bf16* Vg = static_cast<const __bf16*>(p.V) + static_cast<size_t>(bh) * T * D;
  __bf16* Zg = static_cast<__bf16*>(p.Z) + static_cast<size_t>(bh) * T * D;
  const float* etag = p.eta + static_cast<size_t>(bh) * T;

  // staging: thread -> (token st_t, EPT consecutive d from st_d)
  const int st_t = tid / (D / EPT), st_d = (tid % (D / EPT)) * EPT;
  auto stage_write = [&](Stage& S, LdT kk, LdT qq, LdT vv, float e) {
    *reinterpret_cast<LdT*>(&S.K[st_t * RS + st_d]) = kk;
    *reinterpret_cast<LdT*>(&S.Q[st_t * RS + st_d]) = qq;
    *reinterpret_cast<LdT*>(&S.V[st_t * RS + st_d]) = vv;
    if (tid < BC) S.eta[tid] = e * p.eta_scale;
  };
  auto gload = [&](int chunk, LdT& kk, LdT& qq, LdT& vv, float& e) {
    const size_t off = (static_cast<size_t>(chunk) * BC + st_t) * D + st_d;
    kk = *reinterpret_cast<const LdT*>(Kg + off);
    qq = *reinterpret_cast<const LdT*>(Qg + off);
    vv = *reinterpret_cast<const LdT*>(Vg + off);
    e = tid < BC ? etag[chunk * BC + tid] : 0.f;
  };
  // output z = Q + LN(Z^Q) of chunk cc, from the Z^Q partials in red[1] (waves 4..7,
  // token 4 (w - 4) + lane/16, 16 lanes per token)
  auto ln_out = [&](int cc) {
    const Stage& So = sm.st[cc % 3];
    const int t = 4 * (w - 4) + g;
    float z[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) s += sm.red[1][ww][i][t & 3][16 * (t >> 2) + c16];
      z[i] = s;
    }
    float zs = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) zs += z[i];
    const float mu = sum16(zs) * (1.0f / D);
    float var = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) var += (z[i] - mu) * (z[i] - mu);
    var = sum16(var) * (1.0f / D);
    const float rs = 1.0f / sqrtf(var + p.eps);
    float chk = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int d = 16 * i + c16;
      const float o = bf(So.Q[t * RS + d]) + gam[i] * (z[i] - mu) * rs + bet[i];
      chk += o;
      Zg[static_cast<size_t>(cc * BC + t) * D + d] = (__bf16)o;
    }
    chk = sum16(chk);
    if (c16 == 0) flag_nonfinite(p.status, chk);
  };
  {
    LdT kk, qq, vv;
    float e;
    gload(0, kk, qq, vv, e);
    stage_write(sm.st[0], kk, qq, vv, e);
  }
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    Stage& S = sm.st[c % 3];
    const int t0 = c * BC;
    LdT nk{}, nq{}, nv{};
    float ne = 0.f;
    const bool has_next = c + 1 < nchunks;
    if (has_next) gload(c + 1, nk, nq, nv, ne);
    if (p.saved) {
      // chunk-start weights for the backward pass; buffer stores keep the per-lane
      // address to one register (the tile offsets are scalar constants). The element is
      // copied to a scalar float first: a bit_cast applied directly to a vector element
      // was compiled as a read of element 0.
      float* sv = p.saved + (static_cast<size_t>(bh) * nchunks + c) * (2 * D * HID);
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc(sv, 0, 2 * D * HID * 4, 0x00020000);
      const int v1 = (4 * g * HID + hs + c16) * 4;
      const int v2 = (D * HID + (hs + 4 * g) * D + c16) * 4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(static_cast<float>(W1c[dt][ht][r])),
                                                  rsrc, v1, ((16 * dt + r) * HID + 16 * ht) * 4, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(static_cast<float>(W2c[ht][dt][r])),
                                                  rsrc, v2, ((16 * ht + r) * D + 16 * dt) * 4, 0);
          }
    }

    // operands from the staged chunk: rows (token = lane%16) with the permuted d order
    bf16x8 aK[2], aQ[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      aK[ks] = cat(lds4(&S.K[c16 * RS + 32 * ks + 4 * g]), lds4(&S.K[c16 * RS + 32 * ks + 16 + 4 * g]));
      aQ[ks] = cat(lds4(&S.Q[c16 * RS + 32 * ks + 4 * g]), lds4(&S.Q[c16 * RS + 32 * ks + 16 + 4 * g]));
    }
    // bf16 operand copies of the chunk-start weights
    bf16x4 W1b[NDT][NHT], W2b[NHT][NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        W1b[dt][ht] = cvt4(W1c[dt][ht]);
        W2b[ht][dt] = cvt4(W2c[ht][dt]);
      }

    // ---- K side: H^K = K W1 (token x h, R layout) ----
    bf16x4 akR[NHT], akT[NHT];
    f4 gk[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma32(aK[ks], cat(W1b[2 * ks][ht], W1b[2 * ks + 1][ht]), acc);
      f4 a, gd;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v, d1;
        act_d_fwd<GELU_KIND>(acc[r], v, d1);
        a[r] = v;
        gd[r] = d1;
      }
      gk[ht] = gd;
      akR[ht] = cvt4(a);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) akT[ht] = cvt4(mfma16(akR[ht], I4, f4{0.f, 0.f, 0.f, 0.f}));
    // Z^K partial over this wave's h slice (token x d)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks)
        acc = mfma32(cat(akT[2 * ks], akT[2 * ks + 1]), cat(W2b[2 * ks][dt], W2b[2 * ks + 1][dt]), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[0][w][dt][r][lane] = acc[r];
    }
    // Q side products that need only the chunk-start W1: Q W1 and tril(Q K^T)^T
    f4 hq[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma32(aQ[ks], cat(W1b[2 * ks][ht], W1b[2 * ks + 1][ht]), acc);
      hq[ht] = acc;
    }
    f4 s1t = {0.f, 0.f, 0.f, 0.f};  // C[s][t] = K_s . Q_t
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) s1t = mfma32(aK[ks], aQ[ks], s1t);
    __syncthreads();

    // ---- LayerNorm forward/backward of Z^K: 4 tokens per wave, 16 lanes each ----
    if (ln_wave) {
      const int t = ln_t;
      float z[DPL];
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int dt = i;
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += sm.red[0][ww][dt][t & 3][16 * (t >> 2) + c16];
        z[i] = s;
      }
      float zs = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) zs += z[i];
      const float mu = sum16(zs) * (1.0f / D);
      float var = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) var += (z[i] - mu) * (z[i] - mu);
      var = sum16(var) * (1.0f / D);
      const float rs = 1.0f / sqrtf(var + p.eps);
      float xh[DPL], gg[DPL], l2 = 0.f, sg = 0.f, sgx = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = 16 * i + c16;
        xh[i] = (z[i] - mu) * rs;
        const float r = bf(S.K[t * RS + d]) + gam[i] * xh[i] + bet[i] - bf(S.V[t * RS + d]);
        l2 += r * r;
        gg[i] = 2.f * r * gam[i];
        sg += gg[i];
        sgx += gg[i] * xh[i];
      }
      const float loss = sum16(l2);
      const float mg = sum16(sg) * (1.0f / D), mgx = sum16(sgx) * (1.0f / D);
      const float ne2 = -S.eta[t] * rs;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = 16 * i + c16;
        const __bf16 e = (__bf16)(ne2 * (gg[i] - mg - xh[i] * mgx));
        sm.E2[t * RS + d] = e;
      }
      if (c16 == 0) {
        if (p.loss) p.loss[static_cast<size_t>(bh) * T + t0 + t] = loss;
        flag_nonfinite(p.status, loss);
      }
    } else if (c > 0) {
      ln_out(c - 1);  // the previous chunk's output, off the chunk-to-chunk critical path
    }
    // stage the next chunk (its buffer last held chunk c - 2, whose readers are done)
    if (has_next) stage_write(sm.st[(c + 1) % 3], nk, nq, nv, ne);
    __syncthreads();

    // ---- E1n = (En2 W2^T) (.) G ----
    bf16x8 aE[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      aE[ks] = cat(lds4(&sm.E2[c16 * RS + 32 * ks + 4 * g]), lds4(&sm.E2[c16 * RS + 32 * ks + 16 + 4 * g]));
    bf16x4 bE[NDT];  // En2 with k = token (4g + j), n = d (lane%16)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) bE[dt] = tgroup(sm.E2, RS, dt, g, c16);
    bf16x4 e1[NHT];
    {
      // W2^T tiles (d x h) from the bf16 W2 tiles: exact transpose through the identity
      bf16x4 W2Tb[NDT][NHT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          W2Tb[dt][ht] = cvt4(mfma16(W2b[ht][dt], I4, f4{0.f, 0.f, 0.f, 0.f}));
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          acc = mfma32(aE[ks], cat(W2Tb[2 * ks][ht], W2Tb[2 * ks + 1][ht]), acc);
        e1[ht] = cvt4(acc * gk[ht]);
      }
    }
    // ---- H^Q = Q W1 + tril(Q K^T) E1n ; A^Q = GELU(H^Q) ----
    f4 s1m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s1m[r] = (4 * g + r) <= c16 ? s1t[r] : 0.f;
    const bf16x4 s1a = cvt4(s1m);
    bf16x4 aqR[NHT], aqT[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 h = mfma16(s1a, e1[ht], hq[ht]);
      f4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = act_fwd<GELU_KIND>(h[r]);
      aqR[ht] = cvt4(a);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) aqT[ht] = cvt4(mfma16(aqR[ht], I4, f4{0.f, 0.f, 0.f, 0.f}));
    // ---- Z^Q partial = A^Q W2 + tril(A^Q A^K^T) En2 over this wave's h slice ----
    f4 s2t = {0.f, 0.f, 0.f, 0.f};  // C[s][t] = A^K_s . A^Q_t (this slice)
#pragma unroll
    for (int ks = 0; ks < NKH; ++ks)
      s2t = mfma32(cat(akT[2 * ks], akT[2 * ks + 1]), cat(aqT[2 * ks], aqT[2 * ks + 1]), s2t);
    f4 s2m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s2m[r] = (4 * g + r) <= c16 ? s2t[r] : 0.f;
    const bf16x4 s2a = cvt4(s2m);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks)
        acc = mfma32(cat(aqT[2 * ks], aqT[2 * ks + 1]), cat(W2b[2 * ks][dt], W2b[2 * ks + 1][dt]), acc);
      acc = mfma16(s2a, bE[dt], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[1][w][dt][r][lane] = acc[r];
    }
    // ---- chunk-end update of the fp32 fast weights ----
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x4 kt = tgroup(S.K, RS, dt, g, c16);  // K^T: m = d, k = token
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        W1c[dt][ht] = mfma16(kt, e1[ht], W1c[dt][ht]);
        W2c[ht][dt] = mfma16(akR[ht], bE[dt], W2c[ht][dt]);
      }
    }
  }
  // output of the last chunk
  __syncthreads();
  if (!ln_wave) ln_out(nchunks - 1);

  if (p.wt_1) {
    float* o1 = p.wt_1 + static_cast<size_t>(bh) * D * HID;
    float* o2 = p.wt_2 + static_cast<size_t>(bh) * HID * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o1[(16 * dt + 4 * g + r) * HID + hs + 16 * ht + c16] = W1c[dt][ht][r];
          o2[(hs + 16 * ht + 4 * g + r) * D + 16 * dt + c16] = W2c[ht][dt][r];
        }
  }
}

}  // namespace

// Waves per workgroup: two per SIMD, 32 hidden units per wave.
#define TTT_MFMA_WAVES 8

bool fwd_mfma_supported(const ScanParams& p) {
  return p.kind == TTT_MLP && p.d == D && p.hid == HID && p.chunk == BC && p.io == TTT_BF16;
}

hipError_t launch_fwd_mfma(const ScanParams& p, hipStream_t stream) {
  constexpr int NW = TTT_MFMA_WAVES;
  const dim3 grid(p.B * p.H), block(64 * NW);
  if (p.gelu == TTT_GELU_TANH)
    hipLaunchKernelGGL((fwd_mfma_kernel<TTT_GELU_TANH, NW>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<TTT_GELU_ERF, NW>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace ttt
