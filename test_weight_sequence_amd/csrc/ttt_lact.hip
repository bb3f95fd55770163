// The large-chunk SwiGLU TTT layer ("Test-Time Training(TTT)과 LLM 메모리", section "LaCT":
// fast weights f_W(x) = (SiLU(x W1) * (x W3)) W2 (Eq. 6, row vectors, W1 and W3 [d, h], W2
// [h, d]); per chunk of b tokens the gradient of the eta-weighted loss sum_t -f_W(k_t).v_t at the
// chunk-start weights (Eq. 7 and 4), the update W <- L2-Normalize(W - g) with every output
// unit's weight vector scaled to unit norm (Eq. 8), and the read-out o_t = f_W(q_t) (Eq. 2), with
// the weights after the chunk's update, or with its start weights under TTT_LACT_READ_BEFORE).
// Shape: d = 64, h = 256, bf16 Q/K/V/Z, fp32 weights, b a multiple of 64.
//
// With b in the thousands every product of the chunk is a real matrix product, so the layer is
// written as two bf16 MFMA roles launched together, one launch per chunk step:
//  - gradient blocks, one per (head, half of the hidden units): 8 waves, two per SIMD, wave w
//    owning 16 hidden units, every 32-token step of the chunk. Per step
//      A = K W1, C = K W3, P = V W2^T   (the step's tokens x the wave's hidden units)
//      gU = -eta P, s = sigmoid(A), gA = gU C SiLU'(A), gC = gU SiLU(A), u~ = -eta SiLU(A) C
//    and the gradients are summed over the chunk's tokens on the matrix cores:
//      gW1 += K^T gA, gW3 += K^T gC, gW2 += u~^T V.
//    Everything per hidden unit is local to its wave. W1 and W3 columns (one per hidden unit,
//    over d) are normalised where they are computed. A W2 column (one per output unit, over all
//    256 hidden units) spans both blocks of a head, so W2 is stored unnormalised together with
//    each block's partial sum of squares per column; every reader scales W2 by
//    1 / sqrt(the sum of the two partials) as it loads it.
//  - read-out blocks, one per (head, up to 512 tokens of a chunk): the weights as bf16 MFMA
//    operands in LDS (96 KiB), each of the 8 waves computing z for 64 tokens at a time:
//      A^Q^T = W1^T Q^T, C^Q^T = W3^T Q^T, U^T = SiLU(A^Q^T) C^Q^T, z^T = W2^T U^T.
//  - copy-out blocks: W_T from the last state, in the launch that reads out the last chunk
//    (or in a launch of their own when the read-out comes before the update).
// The weights live in two state buffers of the workspace: the step that runs the gradient of
// chunk i reads buffer i and writes buffer i + 1 while the read-out of chunk i - 1 (or, reading
// before the update, of chunk i) reads buffer i, so both roles share one launch. Buffer 0 of
// chunk 0 is the caller's W0 (no normalisation scale).
#include "ttt_mfma_common.hpp"

namespace ttt {
namespace {

using namespace mfma;

constexpr int LH = 256;          // hidden units
constexpr int NW = 8;            // waves per block
constexpr int NT = NW * 64;
constexpr int NHB = 2;           // gradient blocks per head
constexpr int HB = LH / NHB;     // hidden units per gradient block
constexpr int GT = HB / 16 / NW; // 16-unit hidden tiles per gradient wave
constexpr int SS = 32;           // tokens per gradient step
constexpr int ST = 128;          // tokens staged per barrier (64 when the chunk is not a multiple)
constexpr int KRS = D + 8;       // LDS row stride of staged K / V rows (bf16)
constexpr int W_FLOATS = 3 * D * LH;  // W1, W3 [d][h] then W2 [h][d], fp32
constexpr int OR = 64;           // tokens per read-out round of a wave
constexpr int FP = 8;            // copy-out blocks per head

struct GStage {
  alignas(16) __bf16 K[ST * KRS];
  alignas(16) __bf16 V[ST * KRS];
  float eta[ST];
};
struct GSmem {
  GStage st[2];
  float scale[D];        // W2 column scales of the state read
  float part[NW][D];     // per-wave partial column sums of squares of the new W2
};
struct OSmem {
  bf16x8 w1[16][2][64];  // W1^T operand tiles [h tile][d half][lane]
  bf16x8 w3[16][2][64];
  bf16x8 w2[4][8][64];   // W2^T operand tiles [d tile][h tile pair][lane]
  float scale[D];
};
union LSmem {
  GSmem g;
  OSmem o;
};

struct LactParams {
  int B, H, T, chunk, flags, nheads;
  float eta_scale;
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const float* eta;
  const float* w0_1;
  const float* w0_2;
  const float* w0_3;
  __bf16* Z;
  float* state;   // [2][nheads][W_FLOATS]
  float* part;    // [2][nheads][NHB][D]
  unsigned* status;
  int g_chunk;    // chunk whose gradient this launch takes (-1: none)
  int o_chunk;    // chunk this launch reads out (-1: none)
  int o_state;    // state the read-out uses (o_chunk or o_chunk + 1)
  int nG;         // gradient blocks (heads rounded up to 8, times NHB)
  int nO;         // read-out blocks
  int tbo;        // tokens per read-out block
  int f_state;    // state the copy-out blocks write to W_T (-1: none)
  float* wt1;
  float* wt2;
  float* wt3;
};

// Weights of state k of a head: W1, W3 [d][h], W2 [h][d] (unnormalised for k >= 1) and the
// partial column sums of squares of W2 (null for k = 0: W0 is used as given).
struct WRef {
  const float* w1;
  const float* w3;
  const float* w2;
  const float* part;
};
__device__ __forceinline__ WRef wref(const LactParams& p, int k, int head) {
  WRef r;
  if (k == 0) {
    const size_t wi = (p.flags & TTT_W0_PER_SEQ) ? static_cast<size_t>(head) : static_cast<size_t>(head % p.H);
    r.w1 = p.w0_1 + wi * D * LH;
    r.w3 = p.w0_3 + wi * D * LH;
    r.w2 = p.w0_2 + wi * LH * D;
    r.part = nullptr;
  } else {
    const float* s = p.state + (static_cast<size_t>(k & 1) * p.nheads + head) * W_FLOATS;
    r.w1 = s;
    r.w3 = s + D * LH;
    r.w2 = s + 2 * D * LH;
    r.part = p.part + (static_cast<size_t>(k & 1) * p.nheads + head) * NHB * D;
  }
  return r;
}
__device__ __forceinline__ float col_scale(const WRef& r, int d) {
  if (!r.part) return 1.f;
  float s = 0.f;
#pragma unroll
  for (int b = 0; b < NHB; ++b) s += r.part[b * D + d];
  return __builtin_amdgcn_rsqf(s);
}

__device__ __forceinline__ float sigmoid(float a) { return __builtin_amdgcn_rcpf(1.f + __expf(-a)); }

// blockIdx -> (head, sub-block) so that the sub-blocks of a head share an XCD (blocks are
// dealt to the 8 XCDs round-robin)
__device__ __forceinline__ void xcd_map(int b, int per_head, int& head, int& sub) {
  const int x = b & 7, j = b >> 3;
  head = (j / per_head) * 8 + x;
  sub = j % per_head;
}

// ---------------------------------------------------------------------------------------
// gradient role
// ---------------------------------------------------------------------------------------
// Staging of `rows` tokens (64 or 128) of K and V (rows x 8 16-byte pieces each) and eta: two
// or four pieces per thread, all loads issued before any is used.
struct GLoad {
  uint4 q0, q1, q2, q3;
  float e;
};
__device__ __forceinline__ const __bf16* g_src(const LactParams& p, size_t tok0, int n, int idx) {
  const int k = idx < n ? idx : idx - n;
  return (idx < n ? p.K : p.V) + (tok0 + (k >> 3)) * D + (k & 7) * 8;
}
__device__ __forceinline__ __bf16* g_dst(GStage& st, int n, int idx) {
  const int k = idx < n ? idx : idx - n;
  return &(idx < n ? st.K : st.V)[(k >> 3) * KRS + (k & 7) * 8];
}
__device__ __forceinline__ GLoad g_load(const LactParams& p, size_t tok0, int rows, int tid) {
  const int n = rows * 8;  // 512 or 1024 pieces per tensor
  GLoad l;
  l.q0 = *reinterpret_cast<const uint4*>(g_src(p, tok0, n, tid));
  l.q1 = *reinterpret_cast<const uint4*>(g_src(p, tok0, n, NT + tid));
  if (rows == ST) {
    l.q2 = *reinterpret_cast<const uint4*>(g_src(p, tok0, n, 2 * NT + tid));
    l.q3 = *reinterpret_cast<const uint4*>(g_src(p, tok0, n, 3 * NT + tid));
  }
  l.e = tid < rows ? p.eta[tok0 + tid] * p.eta_scale : 0.f;
  return l;
}
__device__ __forceinline__ void g_store(GStage& st, int rows, int tid, const GLoad& l) {
  const int n = rows * 8;
  *reinterpret_cast<uint4*>(g_dst(st, n, tid)) = l.q0;
  *reinterpret_cast<uint4*>(g_dst(st, n, NT + tid)) = l.q1;
  if (rows == ST) {
    *reinterpret_cast<uint4*>(g_dst(st, n, 2 * NT + tid)) = l.q2;
    *reinterpret_cast<uint4*>(g_dst(st, n, 3 * NT + tid)) = l.q3;
  }
  if (tid < rows) st.eta[tid] = l.e;
}

__device__ void g_role(const LactParams& p, int head, int hb, LSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int h0 = HB * hb + 16 * GT * w;  // this wave's hidden units h0 .. h0 + 16 GT - 1
  const int c = p.g_chunk;
  const size_t tok0 = static_cast<size_t>(head) * p.T + static_cast<size_t>(c) * p.chunk;
  const WRef in = wref(p, c, head);
  GSmem& S = sm.g;
  if (tid < D) S.scale[tid] = col_scale(in, tid);
  const int rows = p.chunk % ST == 0 ? ST : ST / 2;  // tokens per stage
  const int nst = p.chunk / rows;
  GLoad ld = g_load(p, tok0, rows, tid);
  g_store(S.st[0], rows, tid, ld);
  __syncthreads();

  // B operands [k = d, n = h]: lane (g, c16) holds d = 32 ks + 8 g + j of hidden unit
  // h0 + 16 ht + c16
  bf16x8 W1B[GT][2], W3B[GT][2], W2B[GT][2];
#pragma unroll
  for (int ht = 0; ht < GT; ++ht) {
    const int h = h0 + 16 * ht + c16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float* w2r = in.w2 + static_cast<size_t>(h) * D + 32 * ks + 8 * g;
      const float4 a = *reinterpret_cast<const float4*>(w2r);
      const float4 b = *reinterpret_cast<const float4*>(w2r + 4);
      const float w2v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = 32 * ks + 8 * g + j;
        W1B[ht][ks][j] = (__bf16)in.w1[d * LH + h];
        W3B[ht][ks][j] = (__bf16)in.w3[d * LH + h];
        W2B[ht][ks][j] = (__bf16)(w2v[j] * S.scale[d]);
      }
    }
  }

  f4 gW1[4][GT], gW3[4][GT], gW2[GT][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < GT; ++j) {
      gW1[i][j] = zero4();
      gW3[i][j] = zero4();
      gW2[j][i] = zero4();
    }

  // K W1, K W3 and V W2^T of one 32-token sub-step: [token][this wave's hidden units] tiles
  auto fwd = [&](const __bf16* Kt, const __bf16* Vt, f4 (&A)[2][GT], f4 (&C)[2][GT], f4 (&P)[2][GT]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      bf16x8 kr[2], vr[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        kr[ks] = *reinterpret_cast<const bf16x8*>(&Kt[(16 * tt + c16) * KRS + 32 * ks + 8 * g]);
        vr[ks] = *reinterpret_cast<const bf16x8*>(&Vt[(16 * tt + c16) * KRS + 32 * ks + 8 * g]);
      }
#pragma unroll
      for (int ht = 0; ht < GT; ++ht) {
        A[tt][ht] = mfma32(kr[1], W1B[ht][1], mfma32(kr[0], W1B[ht][0], zero4()));
        C[tt][ht] = mfma32(kr[1], W3B[ht][1], mfma32(kr[0], W3B[ht][0], zero4()));
        P[tt][ht] = mfma32(vr[1], W2B[ht][1], mfma32(vr[0], W2B[ht][0], zero4()));
      }
    }
  };
  for (int sg = 0; sg < nst; ++sg) {
    const GStage& st = S.st[sg & 1];
    if (sg + 1 < nst) ld = g_load(p, tok0 + static_cast<size_t>(sg + 1) * rows, rows, tid);
    // the forward products of sub-step s + 1 are issued before the element-wise work and the
    // gradient sums of sub-step s, which do not depend on them
    const int nsub = rows / SS;
    f4 A[2][GT], C[2][GT], P[2][GT];
    fwd(st.K, st.V, A, C, P);
    for (int sub = 0; sub < nsub; ++sub) {
      const __bf16* Kt = st.K + sub * SS * KRS;
      const __bf16* Vt = st.V + sub * SS * KRS;
      const float* et = st.eta + sub * SS;
      f4 A2[2][GT], C2[2][GT], P2[2][GT];
      if (sub + 1 < nsub) fwd(Kt + SS * KRS, Vt + SS * KRS, A2, C2, P2);
      bf16x4 gAb[2][GT], gCb[2][GT], ueb[2][GT];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = et[16 * tt + 4 * g + r];
#pragma unroll
        for (int ht = 0; ht < GT; ++ht) {
          f4 ga, gc, ue;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = A[tt][ht][r], cc = C[tt][ht][r];
            const float sg = sigmoid(a);
            const float si = a * sg;
            const float gu = -e[r] * P[tt][ht][r];
            ga[r] = gu * cc * (sg + si * (1.f - sg));
            gc[r] = gu * si;
            ue[r] = -e[r] * si * cc;
          }
          gAb[tt][ht] = cvt4(ga);
          gCb[tt][ht] = cvt4(gc);
          ueb[tt][ht] = cvt4(ue);
        }
      }
      // sums over the 32 tokens (k = token: the two 16-token tiles stacked)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 KT = cat(tgroup(Kt, KRS, dt, g, c16), tgroup(Kt + 16 * KRS, KRS, dt, g, c16));
        const bf16x8 VT = cat(tgroup(Vt, KRS, dt, g, c16), tgroup(Vt + 16 * KRS, KRS, dt, g, c16));
#pragma unroll
        for (int ht = 0; ht < GT; ++ht) {
          gW1[dt][ht] = mfma32(KT, cat(gAb[0][ht], gAb[1][ht]), gW1[dt][ht]);
          gW3[dt][ht] = mfma32(KT, cat(gCb[0][ht], gCb[1][ht]), gW3[dt][ht]);
          gW2[ht][dt] = mfma32(cat(ueb[0][ht], ueb[1][ht]), VT, gW2[ht][dt]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int ht = 0; ht < GT; ++ht) {
          A[tt][ht] = A2[tt][ht];
          C[tt][ht] = C2[tt][ht];
          P[tt][ht] = P2[tt][ht];
        }
    }
    if (sg + 1 < nst) g_store(S.st[(sg + 1) & 1], rows, tid, ld);
    __syncthreads();
  }

  float sc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) sc[dt] = S.scale[16 * dt + c16];
  float part[4] = {0.f, 0.f, 0.f, 0.f};
  {
    float* out = p.state + (static_cast<size_t>((c + 1) & 1) * p.nheads + head) * W_FLOATS;
    // W1 and W3: hidden unit h = h0 + 16 ht + c16 holds d = 16 dt + 4 g + r in this lane;
    // its column norm over d sums the lane's 16 values and the 3 other lanes of that unit
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float* wi = m == 0 ? in.w1 : in.w3;
      float* wo = out + m * D * LH;
#pragma unroll
      for (int ht = 0; ht < GT; ++ht) {
        const int h = h0 + 16 * ht + c16;
        float v[4][4], ssq = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = 16 * dt + 4 * g + r;
            const float gr = m == 0 ? gW1[dt][ht][r] : gW3[dt][ht][r];
            v[dt][r] = wi[d * LH + h] - gr;
            ssq += v[dt][r] * v[dt][r];
          }
        ssq += __shfl_xor(ssq, 16);
        ssq += __shfl_xor(ssq, 32);
        if (c16 == 0 && g == 0) flag_nonfinite(p.status, ssq);
        const float inv = __builtin_amdgcn_rsqf(ssq);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) wo[(16 * dt + 4 * g + r) * LH + h] = v[dt][r] * inv;
      }
    }
    // W2: hidden unit h = h0 + 16 ht + 4 g + r, output unit d = 16 dt + c16
    float* w2o = out + 2 * D * LH;
#pragma unroll
    for (int ht = 0; ht < GT; ++ht)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = h0 + 16 * ht + 4 * g + r, d = 16 * dt + c16;
          const float v = in.w2[h * D + d] * sc[dt] - gW2[ht][dt][r];
          w2o[h * D + d] = v;
          part[dt] += v * v;
        }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      part[dt] += __shfl_xor(part[dt], 16);
      part[dt] += __shfl_xor(part[dt], 32);
    }
  }
  if (g == 0) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) S.part[w][16 * dt + c16] = part[dt];
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += S.part[ww][tid];
    flag_nonfinite(p.status, s);
    p.part[(static_cast<size_t>((c + 1) & 1) * p.nheads + head) * NHB * D + hb * D + tid] = s;
  }
}

// ---------------------------------------------------------------------------------------
// read-out role
// ---------------------------------------------------------------------------------------
__device__ void o_role(const LactParams& p, int head, int tb, LSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  OSmem& S = sm.o;
  const WRef in = wref(p, p.o_state, head);
  if (tid < D) S.scale[tid] = col_scale(in, tid);
  __syncthreads();
  // operand tiles: W1^T / W3^T [m = h, k = d]: lane (g, c16) holds h = 16 ht + c16,
  // d = 32 ks + 8 g + j; W2^T [m = d, k = h]: lane holds d = 16 dt + c16 and, for the pair of h
  // tiles 2 q and 2 q + 1, h = 32 q + 4 g + j (j < 4) and 32 q + 16 + 4 g + (j - 4).
  // Each thread gathers eight float4s (eight d rows of four hidden units of W1 / W3; eight h
  // rows of four output units of W2, coalesced across threads) and writes four whole tiles'
  // slots (16 bytes each).
  {
    const int o8 = tid >> 6, q64 = tid & 63;  // W1 / W3: d = 8 o8 + j, h = 4 q64 + u
    float4 a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = *reinterpret_cast<const float4*>(in.w1 + (8 * o8 + j) * LH + 4 * q64);
      b[j] = *reinterpret_cast<const float4*>(in.w3 + (8 * o8 + j) * LH + 4 * q64);
    }
    const int q = tid >> 6, lg = (tid >> 4) & 3, dq = tid & 15;  // W2: h_j of (q, lg), d = 4 dq + u
    float4 c2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int h = 32 * q + (j < 4 ? 4 * lg + j : 16 + 4 * lg + (j - 4));
      c2[j] = *reinterpret_cast<const float4*>(in.w2 + h * D + 4 * dq);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int h = 4 * q64 + u;
      bf16x8 x, y, z;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = (__bf16)(u == 0 ? a[j].x : u == 1 ? a[j].y : u == 2 ? a[j].z : a[j].w);
        y[j] = (__bf16)(u == 0 ? b[j].x : u == 1 ? b[j].y : u == 2 ? b[j].z : b[j].w);
      }
      S.w1[h >> 4][o8 >> 2][(o8 & 3) * 16 + (h & 15)] = x;
      S.w3[h >> 4][o8 >> 2][(o8 & 3) * 16 + (h & 15)] = y;
      const int d = 4 * dq + u;
      const float sc = S.scale[d];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        z[j] = (__bf16)(sc * (u == 0 ? c2[j].x : u == 1 ? c2[j].y : u == 2 ? c2[j].z : c2[j].w));
      S.w2[d >> 4][q][lg * 16 + (d & 15)] = z;
    }
  }
  __syncthreads();

  const size_t tok_base = static_cast<size_t>(head) * p.T + static_cast<size_t>(p.o_chunk) * p.chunk +
                          static_cast<size_t>(tb) * p.tbo;
  const int rounds = p.tbo / OR;
  for (int rd = w; rd < rounds; rd += NW) {
    const size_t t0 = tok_base + static_cast<size_t>(rd) * OR;
    // Q^T operands [k = d, n = token]: lane (g, c16) holds token 16 tt + c16, d = 32 ks + 8 g + j
    bf16x8 QB[4][2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        QB[tt][ks] = *reinterpret_cast<const bf16x8*>(p.Q + (t0 + 16 * tt + c16) * D + 32 * ks + 8 * g);
    f4 ZT[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) ZT[tt][dt] = zero4();
    for (int q = 0; q < 8; ++q) {
      bf16x4 U[2][4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ht = 2 * q + hh;
        const bf16x8 a0 = S.w1[ht][0][lane], a1 = S.w1[ht][1][lane];
        const bf16x8 b0 = S.w3[ht][0][lane], b1 = S.w3[ht][1][lane];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const f4 A = mfma32(a1, QB[tt][1], mfma32(a0, QB[tt][0], zero4()));
          const f4 C = mfma32(b1, QB[tt][1], mfma32(b0, QB[tt][0], zero4()));
          f4 u;
#pragma unroll
          for (int r = 0; r < 4; ++r) u[r] = A[r] * sigmoid(A[r]) * C[r];
          U[hh][tt] = cvt4(u);
        }
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 w2 = S.w2[dt][q][lane];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) ZT[tt][dt] = mfma32(w2, cat(U[0][tt], U[1][tt]), ZT[tt][dt]);
      }
    }
    // z^T tile: lane (g, c16) holds d = 16 dt + 4 g + r of token 16 tt + c16
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<bf16x4*>(p.Z + (t0 + 16 * tt + c16) * D + 16 * dt + 4 * g) = cvt4(ZT[tt][dt]);
  }
}

// ---------------------------------------------------------------------------------------
// copy-out role: W_T from the last state (W1, W3 as stored, W2 scaled by its column norms);
// block (head, part) copies an eighth of each matrix as float4s
// ---------------------------------------------------------------------------------------
__device__ void f_role(const LactParams& p, int head, int part) {
  const WRef in = wref(p, p.f_state, head);
  const int f = part * NT + threadIdx.x;  // float4 index, D * LH / 4 = 4096 per matrix
  const size_t o = static_cast<size_t>(head) * D * LH / 4 + f;
  reinterpret_cast<float4*>(p.wt1)[o] = reinterpret_cast<const float4*>(in.w1)[f];
  reinterpret_cast<float4*>(p.wt3)[o] = reinterpret_cast<const float4*>(in.w3)[f];
  float4 v = reinterpret_cast<const float4*>(in.w2)[f];
  const int d = (f & 15) * 4;  // W2 [h][d]: float4 f covers d .. d + 3 of row f / 16
  v.x *= col_scale(in, d);
  v.y *= col_scale(in, d + 1);
  v.z *= col_scale(in, d + 2);
  v.w *= col_scale(in, d + 3);
  reinterpret_cast<float4*>(p.wt2)[o] = v;
}

__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
lact_step_kernel(LactParams p) {
  __shared__ LSmem sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  const int b = blockIdx.x;
  int head, sub;
  if (b < p.nG) {
    xcd_map(b, NHB, head, sub);
    if (head < p.nheads) g_role(p, head, sub, sm);
  } else if (b < p.nG + p.nO) {
    xcd_map(b - p.nG, p.chunk / p.tbo, head, sub);
    if (head < p.nheads) o_role(p, head, sub, sm);
  } else {
    const int f = b - p.nG - p.nO;
    f_role(p, f / FP, f % FP);
  }
}

// Tokens per read-out block: the largest power-of-two multiple of 64 up to 512 that divides the
// chunk (512 balances the read-out blocks against the gradient blocks they share a launch with)
int read_tokens(int chunk) {
  int t = 64;
  while (t < 512 && chunk % (2 * t) == 0) t *= 2;
  return t;
}

}  // namespace

bool lact_supported(int d, int hid, int io, int chunk) {
  return d == D && hid == LH && io == TTT_BF16 && chunk >= SS && chunk % SS == 0;
}

size_t lact_workspace_bytes(int nheads) {
  return 2 * static_cast<size_t>(nheads) * W_FLOATS * sizeof(float) +
         2 * static_cast<size_t>(nheads) * NHB * D * sizeof(float);
}

hipError_t launch_lact_fwd(const LactLaunch& L, hipStream_t stream) {
  LactParams p{};
  p.B = L.B;
  p.H = L.H;
  p.T = L.T;
  p.chunk = L.chunk;
  p.flags = L.flags;
  p.nheads = L.B * L.H;
  p.eta_scale = L.eta_scale;
  p.Q = static_cast<const __bf16*>(L.Q);
  p.K = static_cast<const __bf16*>(L.K);
  p.V = static_cast<const __bf16*>(L.V);
  p.eta = L.eta;
  p.w0_1 = L.w0_1;
  p.w0_2 = L.w0_2;
  p.w0_3 = L.w0_3;
  p.Z = static_cast<__bf16*>(L.Z);
  p.status = L.status;
  p.state = L.work;
  p.part = L.work + 2 * static_cast<size_t>(p.nheads) * W_FLOATS;
  p.tbo = read_tokens(L.chunk);
  p.wt1 = L.wt_1;
  p.wt2 = L.wt_2;
  p.wt3 = L.wt_3;
  const int nchunks = L.T / L.chunk;
  const int hpad = (p.nheads + 7) / 8 * 8;
  const bool before = (L.flags & TTT_LACT_READ_BEFORE) != 0;
  const int steps = before ? nchunks : nchunks + 1;
  // the copy-out of W_T joins the launch that reads out the last chunk after its update; when
  // the read-out comes first, the last state is written by the last launch and the copy-out
  // takes a launch of its own
  const int nF = L.wt_1 ? p.nheads * FP : 0;
  for (int s = 0; s < steps; ++s) {
    p.g_chunk = s < nchunks ? s : -1;
    p.o_chunk = before ? s : s - 1;
    p.o_state = s;  // chunk s read before its update, or chunk s - 1 after it: state s
    p.nG = p.g_chunk >= 0 ? hpad * NHB : 0;
    p.nO = p.o_chunk >= 0 ? hpad * (L.chunk / p.tbo) : 0;
    const bool copy = !before && s == steps - 1 && nF > 0;
    p.f_state = copy ? nchunks : -1;
    hipLaunchKernelGGL(lact_step_kernel, dim3(p.nG + p.nO + (copy ? nF : 0)), dim3(NT), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (before && nF > 0) {
    p.g_chunk = p.o_chunk = -1;
    p.nG = p.nO = 0;
    p.f_state = nchunks;
    hipLaunchKernelGGL(lact_step_kernel, dim3(nF), dim3(NT), 0, stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace ttt
