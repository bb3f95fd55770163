// Forward scan with momentum and a forget gate for the TTT-MLP head shape d = 64, hidden = 256,
// chunk 16, bf16 Q/K/V/Z, fp32 memory M and momentum S (gfx950, bf16 MFMA with fp32
// accumulation).
//
// The rule ("Test-Time Training(TTT)과 LLM 메모리", section "Titans와 Miras", Eq. 14 and 13, with
// the mini-batch rule of the base scan: inside a chunk every gradient is taken at the memory
// the chunk started from):
//   S_t = mom_t S_{t-1} - theta_t grad l_t(M_start),   M_t = (1 - alpha_t) M_{t-1} + S_t,
//   z_t = f(Q_t; M_t).
// Inside a chunk the two recurrences unroll into per-token scalars (computed per chunk from the
// gates, in LDS):
//   M_t = A_t M + B_t S - sum_{s<=t} C_ts theta_s grad_s,   S_t = P_t S - sum_{s<=t} D_ts theta_s grad_s,
//   A_t = prod_{u<=t} (1 - alpha_u), P_t = prod_{u<=t} mom_u, B_t = (1 - alpha_t) B_{t-1} + P_t,
//   D_ts = prod_{s<u<=t} mom_u, C_ts = (1 - alpha_t) C_{t-1,s} + D_ts (C_ss = D_ss = 1).
// So with E1n = -theta (.) delta1 and En2 = -theta (.) delta2 (the K side of the base scan with
// theta in place of eta):
//   H^Q_t = A_t (Q M1)_t + B_t (Q S1)_t + sum_s C_ts (Q_t . K_s) E1n_s
//   Z^Q_t = A_t (A^Q M2)_t + B_t (A^Q S2)_t + sum_s C_ts (A^Q_t . A^K_s) En2_s
//   M <- A_b M + B_b S + K^T (c (.) E1n) (and A^K^T (c (.) En2)),  c_s = C_bs
//   S <- P_b S + K^T (e (.) E1n) (and A^K^T (e (.) En2)),         e_s = D_bs
// i.e. the base scan's dual form with per-token scales on the chunk-start products and the
// causal masks weighted by C instead of 0/1.
//
// The memory and the momentum together are 256 KiB of fp32 per head, twice what one CU's
// registers can hold next to the rest, so a head is split by hidden units over S = 2
// workgroups of 8 waves, two per SIMD: wave w of part s holds hidden units 128 s + 16 w .. + 16
// of both M and S as MFMA accumulator tiles (its products over hidden units are 16 deep, one
// half of the 32-deep instruction's operands zero; the matrix cores have room, and two waves
// per SIMD hide each other's VALU latencies). Waves 0-3 also run the per-token phases, 16 lanes
// per token. The two sums over all hidden units, Z^K and Z^Q, are formed from
// the parts' [16 x 64] partials, exchanged through the L2 of the XCD both parts sit on as
// (value, chunk tag) pairs that the reader polls; each part adds the partials in the same
// order, so both compute the same Z^K, En2 and outputs. Across XCDs the exchange falls back
// to counters with device-scope fences. Every wait is bounded and reports TTT_ERR_TIMEOUT.
#include "ttt_mfma_common.hpp"

namespace ttt {
namespace {

using mfma::bf16x4;
using mfma::bf16x8;
using mfma::cat;
using mfma::cvt4;
using mfma::f4;
using mfma::lds4;
using mfma::mfma16;
using mfma::mfma32;
using mfma::sum16;
using mfma::zero4;

constexpr int D = 64;
constexpr int HID = 256;
constexpr int BC = 16;
constexpr int NDT = D / 16;          // d tiles
constexpr int S = 2;                 // workgroups per head
constexpr int NW = 8;                // waves per workgroup (two per SIMD)
constexpr int NT = 64 * NW;
constexpr int HS = HID / (S * NW);   // hidden units per wave (16)
constexpr int NHT = HS / 16;         // h tiles per wave (1)
constexpr int NLN = 4;               // waves 0..3 run the per-token phases, 16 lanes per token
constexpr int NKD = D / 32;          // 32-wide k-steps over d (2)
constexpr int RS = D + 8;            // row stride (bf16) of [token][d] arrays
constexpr int DPL = D / 16;          // d values per LayerNorm lane
constexpr int kSpinLimit = 1 << 20;
static_assert(NHT == 1 && NLN * 4 == BC, "tile split");

// Workspace per head: two exchange areas (Z^K, Z^Q) of two chunk-parity slots of S partial
// [16 x 64] sums, each element a (value, chunk index + 1) pair of 32-bit words; then (after
// all heads) 32 counter words per head. Cleared before every launch.
constexpr size_t kPartFloats = static_cast<size_t>(BC) * D;
constexpr size_t kHeadXFloats = 2 * 2 * S * kPartFloats * 2;
constexpr int kFlagWords = 32;  // [0, S): Z^K counters, [8, 8 + S): Z^Q, [16, 16 + S): XCD ids
constexpr int kLoadL2 = 16;     // exchange loads on one XCD: device scope (sc1), L1 skipped

struct Stage {
  alignas(16) __bf16 K[BC * RS];
  alignas(16) __bf16 Q[BC * RS];
  alignas(16) __bf16 V[BC * RS];
  float theta[BC], mom[BC], alpha[BC];
};

// Per-chunk recurrence coefficients (row t, column s).
struct Coef {
  float C[BC][BC], Dm[BC][BC];
  float A[BC], B[BC], P[BC];
};

struct Smem {
  Stage st[3];                       // chunk c lives in st[c % 3]
  alignas(16) __bf16 E2[BC * RS];    // En2 = -theta delta2, [token][d]
  alignas(16) __bf16 E2c[BC * RS];   // C_bt En2_t (the memory's update)
  alignas(16) __bf16 E2d[BC * RS];   // D_bt En2_t (the momentum's update)
  Coef cf[2];                        // chunk c uses cf[c & 1]
  // per-wave [token x d] partial tiles (lane-rotated rows): [0] Z^K, [1] Z^Q. Separate
  // buffers, so that a chunk's Z^K partials are never written while the previous chunk's Z^Q
  // partials are still being read (no barrier lies between those reads and these writes).
  // Last, so that the small arrays stay within the LDS instructions' 16-bit offsets.
  float red[2][NW][NDT][4][64];
};

__device__ __forceinline__ int prot(int r, int lane) { return (lane + 16 * r) & 63; }

struct Split {
  float* xbuf;        // exchange areas, kHeadXFloats per head
  unsigned* flags;    // kFlagWords per head
  int nheads;
  int head0;          // first head of this launch
};

// fp32 tiles of one wave: X1[:, hb:hb+32] as [d tile][h tile] and X2[hb:hb+32, :] as
// [h tile][d tile] (accumulator layout), through buffer instructions. A null source gives zeros.
__device__ __forceinline__ void t_load(const float* x1, const float* x2, int g, int c16, int hb,
                                       f4 (&A1)[NDT][NHT], f4 (&A2)[NHT][NDT]) {
  if (!x1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        A1[dt][ht] = zero4();
        A2[ht][dt] = zero4();
      }
    return;
  }
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x1), 0, D * HID * 4, mfma::kBufFlags);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x2), 0, D * HID * 4, mfma::kBufFlags);
  const int v1 = (4 * g * HID + hb + c16) * 4, v2 = ((hb + 4 * g) * D + c16) * 4;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        A1[dt][ht][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, v1, ((16 * dt + r) * HID + 16 * ht) * 4, 0));
        A2[ht][dt][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r2, v2, ((16 * ht + r) * D + 16 * dt) * 4, 0));
      }
}
__device__ __forceinline__ void t_store(float* x1, float* x2, int g, int c16, int hb,
                                        const f4 (&A1)[NDT][NHT], const f4 (&A2)[NHT][NDT]) {
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(x1, 0, D * HID * 4, mfma::kBufFlags);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(x2, 0, D * HID * 4, mfma::kBufFlags);
  const int v1 = (4 * g * HID + hb + c16) * 4, v2 = ((hb + 4 * g) * D + c16) * 4;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = A1[dt][ht][r], b = A2[ht][dt][r];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r1, v1, ((16 * dt + r) * HID + 16 * ht) * 4, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(b), r2, v2, ((16 * ht + r) * D + 16 * dt) * 4, 0);
      }
}

// The exchange memory of one head.
struct XMem {
  unsigned* cnt;
  float* xz;
  float* xq;
  __amdgpu_buffer_rsrc_t fr, zr, qr;
  bool local;  // both parts on one XCD
};

__device__ __forceinline__ unsigned cnt_load(const XMem& m, int i) {
  if (m.local) return __builtin_amdgcn_raw_buffer_load_b32(m.fr, 0, 4 * i, kLoadL2);
  return __hip_atomic_load(m.cnt + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Across XCDs: publish the partial every thread has just stored as chunk c (counter := c + 1)
// after a release fence, and wait for the other part's counter after an acquire fence.
__device__ __forceinline__ void publish(const XMem& m, int base, int s, unsigned c1) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(m.cnt + base + s, c1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_all(const XMem& m, int base, int s, unsigned c1, unsigned* status) {
  if (threadIdx.x == 0) {
    bool late = (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout) != 0;
    for (int o = 0; o < S && !late; ++o) {
      if (o == s) continue;
      int it = 0;
      while (cnt_load(m, base + o) < c1) {
        if (++it >= kSpinLimit) {
          late = true;
          atomicOr(status, kStatusTimeout);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 part_load_tagged(const XMem& m, bool zq, int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(zq ? m.qr : m.zr, 8 * off, 0, kLoadL2));
}
__device__ __forceinline__ float part_load(const XMem& m, bool zq, int off) { return (zq ? m.xq : m.xz)[2 * off]; }
__device__ __forceinline__ void part_store(const XMem& m, bool zq, int off, float v, unsigned tag) {
  if (m.local) {
    const u32x2 pv = {__float_as_uint(v), tag};
    __builtin_amdgcn_raw_buffer_store_b64(pv, zq ? m.qr : m.zr, 8 * off, 0, 0);
  } else {
    (zq ? m.xq : m.xz)[2 * off] = v;
  }
}

// Coefficients of one chunk from its staged gates: lane s < 16 of the calling wave fills
// column s of C and D, lane 0 the prefix products A, P and the sum B.
__device__ __forceinline__ void coef_fill(const Stage& st, Coef& cf, int lane) {
  if (lane < BC) {
    const int s = lane;
    float dd = 1.f, cc = 0.f;
    for (int t = 0; t < BC; ++t) {
      if (t > s) dd *= st.mom[t];
      cc = t >= s ? (1.f - st.alpha[t]) * cc + dd : 0.f;
      cf.C[t][s] = cc;
      cf.Dm[t][s] = t >= s ? dd : 0.f;
    }
    if (s == 0) {
      float a = 1.f, b = 0.f, pp = 1.f;
      for (int t = 0; t < BC; ++t) {
        const float keep = 1.f - st.alpha[t];
        pp *= st.mom[t];
        a *= keep;
        b = keep * b + pp;
        cf.A[t] = a;
        cf.B[t] = b;
        cf.P[t] = pp;
      }
    }
  }
}

// The same coefficients from gates held in registers (lane t < 16: mom_t, alpha_t), for a
// wave with nothing else to do: the values travel between lanes by readlane instead of being
// read from LDS inside the recurrence, and the operations are those of coef_fill in the same
// order.
__device__ __forceinline__ void coef_regs(float mo, float al, Coef& cf, int lane) {
  const int s = lane & 15;
  float dd = 1.f, cc = 0.f, a = 1.f, b = 0.f, pp = 1.f;
#pragma unroll
  for (int t = 0; t < BC; ++t) {
    const float mt = __shfl(mo, t, 64), at = __shfl(al, t, 64);
    if (t > s) dd *= mt;
    cc = t >= s ? (1.f - at) * cc + dd : 0.f;
    if (lane < BC) {
      cf.C[t][s] = cc;
      cf.Dm[t][s] = t >= s ? dd : 0.f;
    }
    const float keep = 1.f - at;
    pp *= mt;
    a *= keep;
    b = keep * b + pp;
    if (lane == 0) {
      cf.A[t] = a;
      cf.B[t] = b;
      cf.P[t] = pp;
    }
  }
}

template <int GELU_KIND>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_mom_kernel(ScanParams p, Split x) {
  __shared__ Smem sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  // block -> (head, part): the S parts of a head are 8 blocks apart (same XCD)
  const int b = blockIdx.x;
  const int s = (b >> 3) % S;
  const int bh = x.head0 + ((b >> 3) / S) * 8 + (b & 7);
  if (bh >= x.nheads) return;  // both parts of a missing head leave together
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int hidx = bh % p.H;
  const int hb = s * (HID / S) + w * HS;
  const int T = p.T, nchunks = T / BC;
  const bool per_seq = (p.flags & TTT_W0_PER_SEQ) != 0;
  __shared__ unsigned sh_local;
  TTT_POISON(sh_local);
  TTT_POISON_DONE();
  XMem m;
  m.xz = x.xbuf + static_cast<size_t>(bh) * kHeadXFloats;
  m.xq = m.xz + 2 * 2 * S * kPartFloats;
  m.cnt = x.flags + static_cast<size_t>(bh) * kFlagWords;
  m.fr = __builtin_amdgcn_make_buffer_rsrc(m.cnt, 0, kFlagWords * 4, mfma::kBufFlags);
  m.zr = __builtin_amdgcn_make_buffer_rsrc(m.xz, 0, 2 * S * kPartFloats * 8, mfma::kBufFlags);
  m.qr = __builtin_amdgcn_make_buffer_rsrc(m.xq, 0, 2 * S * kPartFloats * 8, mfma::kBufFlags);
  {
    // placement: every part publishes its XCD id + 1 (device scope) and reads the other's
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (threadIdx.x == 0) {
      __hip_atomic_store(m.cnt + 16 + s, xcc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool same = true;
      for (int o = 0; o < S; ++o) {
        unsigned v = 0;
        for (int it = 0; it < kSpinLimit && v == 0; ++it) {
          v = __hip_atomic_load(m.cnt + 16 + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (v == 0) __builtin_amdgcn_s_sleep(1);
        }
        if (v == 0) atomicOr(p.status, kStatusTimeout);
        same = same && v == xcc + 1;
      }
      sh_local = same && !(p.flags & TTT_FORCE_DEVICE_SCOPE) ? 1u : 0u;
    }
    __syncthreads();
    m.local = sh_local != 0;
  }

  // memory M and momentum S of this wave's hidden units
  f4 M1c[NDT][NHT], M2c[NHT][NDT], S1c[NDT][NHT], S2c[NHT][NDT];
  {
    const size_t wh = per_seq ? static_cast<size_t>(bh) : static_cast<size_t>(hidx);
    t_load(p.w0_1 + wh * D * HID, p.w0_2 + wh * HID * D, g, c16, hb, M1c, M2c);
    const size_t sh = static_cast<size_t>(bh);
    t_load(p.s0_1 ? p.s0_1 + sh * D * HID : nullptr, p.s0_2 ? p.s0_2 + sh * HID * D : nullptr, g, c16, hb, S1c, S2c);
  }
  const bf16x4 I4 = mfma::make_ident(g, c16).i4;

  // LayerNorm lanes: token 4 w + lane/16, 16 lanes per token, d = 16 i + lane%16
  const int ln_t = 4 * w + g;
  float gam[DPL], bet[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    gam[i] = p.gamma[hidx * D + 16 * i + c16];
    bet[i] = p.beta[hidx * D + 16 * i + c16];
  }

  const size_t io_off = static_cast<size_t>(bh) * T * D;
  const __bf16* Qg = static_cast<const __bf16*>(p.Q) + io_off;
  const __bf16* Kg = static_cast<const __bf16*>(p.K) + io_off;
  const __bf16* Vg = static_cast<const __bf16*>(p.V) + io_off;
  __bf16* Zg = static_cast<__bf16*>(p.Z) + io_off;
  const float* thg = p.eta + static_cast<size_t>(bh) * T;
  const float* mog = p.mom + static_cast<size_t>(bh) * T;
  const float* alg = p.alpha + static_cast<size_t>(bh) * T;

  // staging: thread -> token st_t, 4 consecutive d from st_d; threads 0..15 the gates
  const int st_t = tid >> 4, st_d = (tid & 15) * 4;
  struct Ld {
    uint2 k, q, v;
    float th, mo, al;
  };
  auto gload = [&](int chunk) {
    Ld r{};
    if (tid >= NLN * 64) return r;
    const size_t off = (static_cast<size_t>(chunk) * BC + st_t) * D + st_d;
    r.k = *reinterpret_cast<const uint2*>(Kg + off);
    r.q = *reinterpret_cast<const uint2*>(Qg + off);
    r.v = *reinterpret_cast<const uint2*>(Vg + off);
    const int ti = chunk * BC + (tid & 15);
    r.th = tid < BC ? thg[ti] : 0.f;
    r.mo = tid < BC ? mog[ti] : 0.f;
    r.al = tid < BC ? alg[ti] : 0.f;
    return r;
  };
  auto stage_write = [&](Stage& St, const Ld& r) {
    if (tid >= NLN * 64) return;
    *reinterpret_cast<uint2*>(&St.K[st_t * RS + st_d]) = r.k;
    *reinterpret_cast<uint2*>(&St.Q[st_t * RS + st_d]) = r.q;
    *reinterpret_cast<uint2*>(&St.V[st_t * RS + st_d]) = r.v;
    if (tid < BC) {
      St.theta[tid] = r.th * p.eta_scale;
      St.mom[tid] = r.mo;
      St.alpha[tid] = r.al;
    }
  };
  // this part's [16 x 64] partial for the LayerNorm lanes' elements (fixed wave order)
  auto own_partial = [&](bool zq, float (&o)[DPL]) {
    const int t = ln_t;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      float a = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) a += sm.red[zq][ww][i][t & 3][prot(t & 3, 16 * (t >> 2) + c16)];
      o[i] = a;
    }
  };
  auto ln_stats = [&](const float (&z)[DPL], float& mu, float& rs) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) a += z[i];
    mu = sum16(a) * (1.0f / D);
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) v += (z[i] - mu) * (z[i] - mu);
    rs = __builtin_amdgcn_rsqf(sum16(v) * (1.0f / D) + p.eps);
  };
  auto put_own = [&](bool zq, int slot, unsigned tag, float (&own)[DPL]) {
    own_partial(zq, own);
#pragma unroll
    for (int i = 0; i < DPL; ++i)
      part_store(m, zq, (slot * S + s) * kPartFloats + ln_t * D + 16 * i + c16, own[i], tag);
  };
  // the head's total from the S partials of a slot (fixed part order; this part's own from
  // registers); on one XCD each lane polls its elements until every tag reads `tag` (bounded)
  auto total = [&](bool zq, int slot, unsigned tag, const float (&own)[DPL], float (&z)[DPL]) {
    float v[S][DPL];
    if (m.local) {
      for (int it = 0;; ++it) {
        bool all = true;
#pragma unroll
        for (int o = 0; o < S; ++o) {
          if (o == s) continue;
#pragma unroll
          for (int i = 0; i < DPL; ++i) {
            const u32x2 pv = part_load_tagged(m, zq, (slot * S + o) * kPartFloats + ln_t * D + 16 * i + c16);
            v[o][i] = __uint_as_float(pv[0]);
            all = all && pv[1] == tag;
          }
        }
        if (all) break;
        if (it + 1 >= kSpinLimit) {
          atomicOr(p.status, kStatusTimeout);
          break;
        }
        if ((it & 63) == 63 &&
            (__hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout))
          break;
        __builtin_amdgcn_s_sleep(1);
      }
    } else {
#pragma unroll
      for (int o = 0; o < S; ++o)
#pragma unroll
        for (int i = 0; i < DPL; ++i) v[o][i] = part_load(m, zq, (slot * S + o) * kPartFloats + ln_t * D + 16 * i + c16);
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      float a = 0.f;
#pragma unroll
      for (int o = 0; o < S; ++o) a += o == s ? own[i] : v[o][i];
      z[i] = a;
    }
  };
  // output z = Q + LN(Z^Q) of chunk cc for this part's tokens (wave s: tokens 4 s .. 4 s + 3,
  // and wave s + 2: tokens 4 (s + 2) ..; between them the two parts cover the 16 tokens)
  float ownQ[DPL];
  auto ln_out = [&](int cc) {
    const Stage& So = sm.st[cc % 3];
    const int t = ln_t;
    float z[DPL];
    total(true, cc & 1, static_cast<unsigned>(cc) + 1u, ownQ, z);
    float mu, rs;
    ln_stats(z, mu, rs);
    float chk = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int d = 16 * i + c16;
      const float o = mfma::bf(So.Q[t * RS + d]) + gam[i] * (z[i] - mu) * rs + bet[i];
      chk += o;
      Zg[static_cast<size_t>(cc * BC + t) * D + d] = (__bf16)o;
    }
    chk = sum16(chk);
    if (c16 == 0) flag_nonfinite(p.status, chk);
  };
  const bool ln_wave = w < NLN;                 // waves with per-token lanes
  const bool out_wave = ln_wave && (w & 1) == s;  // waves that write outputs: 2 per part, 4 tokens each

  stage_write(sm.st[0], gload(0));
  __syncthreads();
  if (w == 0) coef_fill(sm.st[0], sm.cf[0], lane);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    Stage& St = sm.st[c % 3];
    const Coef& cf = sm.cf[c & 1];
    const int t0 = c * BC;
    const unsigned c1 = static_cast<unsigned>(c) + 1u;
    const int slot = c & 1;
    const bool has_next = c + 1 < nchunks;
    Ld nx{};
    if (has_next) nx = gload(c + 1);
    // the next chunk's gates for its coefficients, computed by wave NLN during the per-token
    // phase below (it has no per-token lanes)
    float mo_n = 0.f, al_n = 0.f;
    if (w == NLN && has_next && lane < BC) {
      mo_n = mog[(c + 1) * BC + lane];
      al_n = alg[(c + 1) * BC + lane];
    }

    bf16x8 aK[NKD], aQ[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      aK[ks] = cat(lds4(&St.K[c16 * RS + 32 * ks + 4 * g]), lds4(&St.K[c16 * RS + 32 * ks + 16 + 4 * g]));
      aQ[ks] = cat(lds4(&St.Q[c16 * RS + 32 * ks + 4 * g]), lds4(&St.Q[c16 * RS + 32 * ks + 16 + 4 * g]));
    }
    bf16x4 M1b[NDT][NHT], M2b[NHT][NDT], S1b[NDT][NHT], S2b[NHT][NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        M1b[dt][ht] = cvt4(M1c[dt][ht]);
        M2b[ht][dt] = cvt4(M2c[ht][dt]);
        S1b[dt][ht] = cvt4(S1c[dt][ht]);
        S2b[ht][dt] = cvt4(S2c[ht][dt]);
      }
    // per-token scales of this lane's accumulator rows (token 4 g + r)
    float rA[4], rB[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rA[r] = cf.A[4 * g + r];
      rB[r] = cf.B[4 * g + r];
    }

    // ---- K side at the chunk-start memory: H^K = K M1, A^K, G; Z^K partial; the query's
    // chunk-start products A_t (Q M1) + B_t (Q S1) ----
    bf16x4 akR[NHT], akT[NHT];
    f4 gk[NHT], hq[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 acc = zero4(), accq = zero4(), accs = zero4();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        acc = mfma32(aK[ks], cat(M1b[2 * ks][ht], M1b[2 * ks + 1][ht]), acc);
        accq = mfma32(aQ[ks], cat(M1b[2 * ks][ht], M1b[2 * ks + 1][ht]), accq);
        accs = mfma32(aQ[ks], cat(S1b[2 * ks][ht], S1b[2 * ks + 1][ht]), accs);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) hq[ht][r] = rA[r] * accq[r] + rB[r] * accs[r];
      f4 a, gd;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v, d1;
        mfma::act_d_fwd<GELU_KIND>(acc[r], v, d1);
        a[r] = v;
        gd[r] = d1;
      }
      gk[ht] = gd;
      akR[ht] = cvt4(a);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) akT[ht] = cvt4(mfma16(akR[ht], I4, zero4()));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const f4 acc = mfma16(akT[0], M2b[0][dt], zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[0][w][dt][r][prot(r, lane)] = acc[r];
    }
    f4 s1t = zero4();  // C[s][t] = K_s . Q_t
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) s1t = mfma32(aK[ks], aQ[ks], s1t);
    __syncthreads();

    // ---- Z^K over all hidden units (this wait also covers the Z^Q partials of chunk c - 1,
    // whose output is written now), LayerNorm forward/backward -> En2 and its two weighted
    // copies for the chunk-end updates ----
    float ownK[DPL];
    if (ln_wave) put_own(false, slot, c1, ownK);
    if (!m.local) {
      publish(m, 0, s, c1);
      wait_all(m, 0, s, c1, p.status);
    }
    if (c > 0 && out_wave) ln_out(c - 1);
    // the chunk-end state before this chunk's gradients: M <- A_b M + B_b S, S <- P_b S (the
    // bf16 operand copies of the chunk-start state were taken above), while the other part's
    // Z^K partial is on its way
    {
      const float Ab = cf.A[BC - 1], Bb = cf.B[BC - 1], Pb = cf.P[BC - 1];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          M1c[dt][ht] = Ab * M1c[dt][ht] + Bb * S1c[dt][ht];
          S1c[dt][ht] = Pb * S1c[dt][ht];
          M2c[ht][dt] = Ab * M2c[ht][dt] + Bb * S2c[ht][dt];
          S2c[ht][dt] = Pb * S2c[ht][dt];
        }
    }
    if (ln_wave) {
      const int t = ln_t;
      float z[DPL];
      total(false, slot, c1, ownK, z);
      float mu, rs;
      ln_stats(z, mu, rs);
      float xh[DPL], gg[DPL], l2 = 0.f, sg = 0.f, sgx = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = 16 * i + c16;
        xh[i] = (z[i] - mu) * rs;
        const float r = mfma::bf(St.K[t * RS + d]) + gam[i] * xh[i] + bet[i] - mfma::bf(St.V[t * RS + d]);
        l2 += r * r;
        gg[i] = 2.f * r * gam[i];
        sg += gg[i];
        sgx += gg[i] * xh[i];
      }
      const float loss = sum16(l2);
      const float mg = sum16(sg) * (1.0f / D), mgx = sum16(sgx) * (1.0f / D);
      const float ne2 = -St.theta[t] * rs;
      const float wc = cf.C[BC - 1][t], wd = cf.Dm[BC - 1][t];
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = 16 * i + c16;
        const float e = ne2 * (gg[i] - mg - xh[i] * mgx);
        sm.E2[t * RS + d] = (__bf16)e;
        sm.E2c[t * RS + d] = (__bf16)(wc * e);
        sm.E2d[t * RS + d] = (__bf16)(wd * e);
      }
      if (c16 == 0 && s == 0) {
        if (p.loss) p.loss[static_cast<size_t>(bh) * T + t0 + t] = loss;
        flag_nonfinite(p.status, loss);
      }
    }
    if (has_next) stage_write(sm.st[(c + 1) % 3], nx);
    // coefficients of chunk c + 1 (chunk c uses the other buffer)
    if (w == NLN && has_next) coef_regs(mo_n, al_n, sm.cf[(c + 1) & 1], lane);
    __syncthreads();

    // ---- E1n = (En2 M2^T) (.) G and its weighted copies; H^Q; A^Q; Z^Q partial ----
    bf16x8 aE[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks)
      aE[ks] = cat(lds4(&sm.E2[c16 * RS + 32 * ks + 4 * g]), lds4(&sm.E2[c16 * RS + 32 * ks + 16 + 4 * g]));
    float rC[4], rD[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rC[r] = cf.C[BC - 1][4 * g + r];
      rD[r] = cf.Dm[BC - 1][4 * g + r];
    }
    bf16x4 e1[NHT], e1c[NHT], e1d[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks)
        acc = mfma32(aE[ks], cat(cvt4(mfma16(M2b[ht][2 * ks], I4, zero4())),
                                 cvt4(mfma16(M2b[ht][2 * ks + 1], I4, zero4()))), acc);
      const f4 v = acc * gk[ht];
      e1[ht] = cvt4(v);
      f4 vc, vd;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vc[r] = rC[r] * v[r];
        vd[r] = rD[r] * v[r];
      }
      e1c[ht] = cvt4(vc);
      e1d[ht] = cvt4(vd);
    }
    // causal masks weighted by C_ts (row s = 4 g + r of the score tile, column t = lane % 16)
    float wmask[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) wmask[r] = cf.C[c16][4 * g + r];
    f4 s1m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s1m[r] = wmask[r] * s1t[r];
    const bf16x4 s1a = cvt4(s1m);
    bf16x4 aqT[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const f4 h = mfma16(s1a, e1[ht], hq[ht]);
      f4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = mfma::act_fwd<GELU_KIND>(h[r]);
      aqT[ht] = cvt4(mfma16(cvt4(a), I4, zero4()));
    }
    f4 s2t = mfma16(akT[0], aqT[0], zero4());  // this wave's share of C[s][t] = A^K_s . A^Q_t
    f4 s2m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s2m[r] = wmask[r] * s2t[r];
    const bf16x4 s2a = cvt4(s2m);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x4 be = mfma::tgroup(sm.E2, RS, dt, g, c16);
      f4 accm = mfma16(aqT[0], M2b[0][dt], zero4());
      const f4 accs = mfma16(aqT[0], S2b[0][dt], zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) accm[r] = rA[r] * accm[r] + rB[r] * accs[r];
      accm = mfma16(s2a, be, accm);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[1][w][dt][r][prot(r, lane)] = accm[r];
      // chunk-end updates of this wave's fp32 memory and momentum
      const bf16x4 kt = mfma::tgroup(St.K, RS, dt, g, c16);
      const bf16x4 bc = mfma::tgroup(sm.E2c, RS, dt, g, c16);
      const bf16x4 bd = mfma::tgroup(sm.E2d, RS, dt, g, c16);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        M1c[dt][ht] = mfma16(kt, e1c[ht], M1c[dt][ht]);
        S1c[dt][ht] = mfma16(kt, e1d[ht], S1c[dt][ht]);
        M2c[ht][dt] = mfma16(akR[ht], bc, M2c[ht][dt]);
        S2c[ht][dt] = mfma16(akR[ht], bd, S2c[ht][dt]);
      }
    }
    __syncthreads();

    // ---- publish this part's Z^Q partial of chunk c (its output is written next chunk) ----
    if (ln_wave) put_own(true, slot, c1, ownQ);
    if (!m.local) publish(m, 8, s, c1);
  }
  if (!m.local) wait_all(m, 8, s, static_cast<unsigned>(nchunks), p.status);
  if (out_wave) ln_out(nchunks - 1);

  if (p.wt_1)
    t_store(p.wt_1 + static_cast<size_t>(bh) * D * HID, p.wt_2 + static_cast<size_t>(bh) * HID * D, g, c16, hb,
            M1c, M2c);
  if (p.st_1)
    t_store(p.st_1 + static_cast<size_t>(bh) * D * HID, p.st_2 + static_cast<size_t>(bh) * HID * D, g, c16, hb,
            S1c, S2c);
}

// Clears the exchange areas (their tags) and the counter words of every head.
__global__ void mom_reset_kernel(uint4* w, size_t n4) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    w[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

bool fwd_mom_supported(const ScanParams& p) {
  return p.kind == TTT_MLP && p.d == D && p.hid == HID && p.chunk == BC && p.io == TTT_BF16;
}

size_t fwd_mom_workspace_bytes(int nheads) {
  return static_cast<size_t>(nheads) * (kHeadXFloats * sizeof(float) + kFlagWords * sizeof(unsigned));
}

static int mom_blocks(int nheads) { return (nheads + 7) / 8 * 8 * S; }

// Resident workgroups of the kernel on the current device (0 when it cannot launch
// cooperatively); the parts of a head wait for each other, so a launch holds at most this
// many. Cached per device ordinal.
static int mom_capacity() {
  constexpr int kMaxDev = 64;
  static int cap[kMaxDev];  // 0 = unknown, else 1 + resident workgroups on the device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  if (cap[dev] == 0) {
    int coop = 0, ncu = 0, per_cu = 0;
    const bool ok =
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(fwd_mom_kernel<TTT_GELU_ERF>), NT, 0) == hipSuccess;
    cap[dev] = 1 + ((ok && coop) ? ncu * per_cu : 0);
  }
  return cap[dev] - 1;
}

// Heads per launch: whole groups of eight heads whose parts all fit on the device at once.
static int mom_heads_per_launch() { return mom_capacity() / (8 * S) * 8; }

bool fwd_mom_fits() { return mom_heads_per_launch() > 0; }

hipError_t launch_fwd_mfma_mom(const ScanParams& p, hipStream_t stream) {
  const int nheads = p.B * p.H;
  const int per = mom_heads_per_launch();
  if (per <= 0) return hipErrorCooperativeLaunchTooLarge;
  Split x;
  x.xbuf = p.wbuf;
  x.flags = reinterpret_cast<unsigned*>(p.wbuf + static_cast<size_t>(nheads) * kHeadXFloats);
  x.nheads = nheads;
  const size_t n4 = static_cast<size_t>(nheads) * (kHeadXFloats + kFlagWords) / 4;
  const unsigned rblocks = static_cast<unsigned>(n4 / 256 + 1 < 2048 ? n4 / 256 + 1 : 2048);
  hipLaunchKernelGGL(mom_reset_kernel, dim3(rblocks), dim3(256), 0, stream, reinterpret_cast<uint4*>(p.wbuf), n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* fn = p.gelu == TTT_GELU_TANH ? reinterpret_cast<const void*>(fwd_mom_kernel<TTT_GELU_TANH>)
                                           : reinterpret_cast<const void*>(fwd_mom_kernel<TTT_GELU_ERF>);
  for (int h0 = 0; h0 < nheads; h0 += per) {
    ScanParams pc = p;
    x.head0 = h0;
    void* args[] = {&pc, &x};
    const int n = nheads - h0 < per ? nheads - h0 : per;
    e = hipLaunchCooperativeKernel(fn, dim3(mom_blocks(n)), dim3(NT), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ttt
