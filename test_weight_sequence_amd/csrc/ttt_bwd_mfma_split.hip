// Tuned outer-loop backward for the TTT-MLP head shape d = 64, hidden = 256, chunk 16, bf16
// Q/K/V/dZ/dQ/dK/dV, fp32 weights, with every head spread over two workgroups: the gradients
// of the scan's outputs with respect to its inputs through the inner updates (gradients of
// gradients; the outer loop of "LLM : 빠른 논문 리뷰 : End-to-End Test-Time Training for Long
// Context", section 2.2, applied to the layer of "Test-Time Training(TTT)과 LLM 메모리",
// section "TTT layer", Eq. 2/4/5 with the mini-batch rule of the review's Eq. 5).
//
// The chunk's forward and adjoint equations are those of the one-workgroup kernel
// (ttt_bwd_mfma.hip). Here part s of a head owns hidden units [128 s, 128 s + 128), wave w of
// the part [128 s + 32 w, + 32), one wave per SIMD with the SIMD's whole register file. Every
// product per hidden unit is local to a part; the sums over hidden units are formed from the
// parts' partials:
//   Z^K, Z^Q and the dE2 partial (P2^T dZQ + dgA W2 + AK dW2'), on the chain: each part stores
//   its [16 x 64] partial to the exchange area and both add the two in part order, so they
//   compute the same LayerNorm statistics, E2, dZQ and dZK;
//   dQ and dK (outputs): part 0 writes dQ and part 1 writes dK, each adding the other part's
//   partial, sent one chunk ahead of its use. P1 = tril(Q K^T) is a sum over d (computed by
//   both); P2 and dP1 are sums over hidden units that enter only linear terms (P2 E2, P2^T dZQ,
//   dP1 K, dP1^T Q), so each part applies its own partial and the exchanges add them.
// The two parts are numbered 8 blocks apart, so that the hardware's round-robin placement puts
// them on one XCD; they check it at start (HW_REG_XCC_ID). On one XCD a partial element travels
// as a (value, tag) pair in one 8-byte store that the reader polls in the XCD's L2; across XCDs
// (or with TTT_FORCE_DEVICE_SCOPE) the parts publish counters with device-scope fences. Waits
// are bounded and report TTT_ERR_TIMEOUT.
#include "ttt_mfma_common.hpp"

namespace ttt {
namespace {

using namespace mfma;

constexpr int S = 2;                  // workgroups (parts) per head
constexpr int NW = 4;                 // waves per workgroup (one per SIMD)
constexpr int NT = 64 * NW;
constexpr int HS = HID / (S * NW);    // hidden units per wave
constexpr int NHT = HS / 16;          // h tiles per wave
constexpr int NKH = NHT / 2;          // 32-wide k-steps over a wave's hidden slice
constexpr int TS = BC + 8;            // padded row stride of the [16 x 16] dP1 arrays
constexpr int PL = D / 16;            // per-token phases: 16 lanes per token, 4 values per lane
constexpr int kSpinLimit = 1 << 20;
constexpr int kLoadL2 = 16;           // exchange loads on one XCD: device scope (sc1), L1 skipped
static_assert(NW * 4 == BC && NHT == 2 && NDT == NW, "part shape");

// Exchange memory per head: five areas (Z^K, Z^Q, dE2 partials of both parts; dQ partial sent
// by part 1; dK partial sent by part 0), each with two chunk-parity slots of S [16 x 64] partials
// whose elements are (value, tag) pairs of 32-bit words; then (after all heads) 32 counter words
// per head: [2 a + s] for area a and part s, [16 + s] the XCD ids. Cleared before every launch.
enum { kXZK = 0, kXZQ = 1, kXDE2 = 2, kXDQ = 3, kXDK = 4, kAreas = 5 };
constexpr size_t kPart = static_cast<size_t>(BC) * D;
constexpr size_t kHeadElems = static_cast<size_t>(kAreas) * 2 * S * kPart;
constexpr size_t kHeadXFloats = 2 * kHeadElems;
constexpr int kFlagWords = 32;

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
// lanes) and the per-token reads (four tokens of 16 lanes) touch 64 distinct banks.
struct Partials {
  float v[NW][NDT][4][64];
};
__device__ __forceinline__ int prot(int r, int lane) { return (lane + 16 * r) & 63; }

struct BSmem {
  BStage st[2];                       // chunk c lives in st[c & 1]
  alignas(16) __bf16 E2[BC * RS];     // E2 (= -eta d2): [token][d]
  alignas(16) __bf16 dZQ[BC * RS];
  alignas(16) __bf16 dZK[BC * RS];
  alignas(16) __bf16 dP1r[BC * TS];   // this part's dP1 partial [t][u]
  alignas(16) __bf16 dP1c[BC * TS];   // the same, [u][t]
  float dKres[BC * D];                // residual part of dK, [t][d]
  float dp1p[NW][4][64];              // per-wave dP1 partials (accumulator-tile order)
  Partials red[3];                    // [0]: ZK, ZQ, dE2;  [1]: dQ;  [2]: dK
  float dgb[NW][2][D];                // per-wave dgamma / dbeta partials
  unsigned local;
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
__device__ __forceinline__ bf16x8 hcat(const bf16x4 (&x)[NHT], int ks) { return cat(x[2 * ks], x[2 * ks + 1]); }

// The chunk-start weights of one wave in the transposed tile orientations: W1^T tiles
// (C[h][d]: lane holds W1[d][h .. h+3]) and W2^T tiles (C[d][h]: lane holds W2[h][d .. d+3]),
// 16 contiguous bytes per lane per tile from the row-major saved copy. Each part reads its own
// hidden units once, so the loads are non-temporal (cache policy nt): the 4 GB stream of saved
// weights then does not push the exchange areas' lines out of the L2.
constexpr int kLoadNT = 2;
__device__ __forceinline__ void wT_load(const float* w1, const float* w2, int g, int c16, int hs,
                                        f4 (&W1T)[NHT][NDT], f4 (&W2T)[NDT][NHT]) {
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w1), 0, D * HID * 4, kBufFlags);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w2), 0, D * HID * 4, kBufFlags);
  const int v1 = (c16 * HID + hs + 4 * g) * 4, v2 = ((hs + c16) * D + 4 * g) * 4;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      W1T[ht][dt] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r1, v1, (16 * dt * HID + 16 * ht) * 4, kLoadNT));
      W2T[dt][ht] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r2, v2, (16 * ht * D + 16 * dt) * 4, kLoadNT));
    }
}

// rows of a [token][d] LDS array as the A operand of a contraction over d (permuted k order)
__device__ __forceinline__ void rows2(const __bf16* a, int c16, int g, bf16x8 (&o)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    o[ks] = cat(lds4(&a[c16 * RS + 32 * ks + 4 * g]), lds4(&a[c16 * RS + 32 * ks + 16 + 4 * g]));
}
// [token][d] LDS array as the B operand of a contraction over tokens (k = token, n = d)
__device__ __forceinline__ bf16x4 colsT(const __bf16* a, int dt, int c16, int g) {
  return tgroup(a, RS, dt, g, c16);
}
// this part's sum over its waves of element (t, 16 i + c16)
__device__ __forceinline__ float red_sum(const Partials& P, int i, int t, int c16) {
  float s = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) s += P.v[ww][i][t & 3][prot(t & 3, 16 * (t >> 2) + c16)];
  return s;
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

// The exchange memory of one head.
struct XMem {
  unsigned* cnt;
  float* x;
  __amdgpu_buffer_rsrc_t fr, xr;
  bool local;  // both parts on one XCD
};
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
// element index of (area, slot, part, element within the [16 x 64] partial)
__device__ __forceinline__ int xel(int area, int slot, int part, int e) {
  return static_cast<int>(((area * 2 + slot) * S + part) * kPart) + e;
}
__device__ __forceinline__ void x_store(const XMem& m, int el, float v, unsigned tag) {
  if (m.local) {
    const u32x2 pv = {__float_as_uint(v), tag};
    __builtin_amdgcn_raw_buffer_store_b64(pv, m.xr, 8 * el, 0, 0);
  } else {
    m.x[2 * el] = v;
  }
}
__device__ __forceinline__ u32x2 x_load_tagged(const XMem& m, int el) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(m.xr, 8 * el, 0, kLoadL2));
}
__device__ __forceinline__ unsigned cnt_load(const XMem& m, int i) {
  return __hip_atomic_load(m.cnt + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-scope path: publish what every thread has just stored for area `a` (counter word
// 2 a + s := tag; the stores are released first), and wait for the other part's counter.
__device__ __forceinline__ void publish(const XMem& m, int a, int s, unsigned tag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(m.cnt + 2 * a + s, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_other(const XMem& m, int a, int s, unsigned tag, unsigned* status) {
  if (threadIdx.x == 0) {
    const int o = 1 - s;
    bool late = (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout) != 0;
    for (int it = 0; !late && cnt_load(m, 2 * a + o) < tag; ++it) {
      if (it + 1 >= kSpinLimit) {
        atomicOr(status, kStatusTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
// The other part's values of the listed elements (polled until their tags read `tag` on one
// XCD, bounded; plain loads after wait_other across XCDs).
template <int N>
__device__ __forceinline__ void x_read(const XMem& m, const int (&el)[N], unsigned tag, float (&v)[N],
                                       unsigned* status) {
  if (m.local) {
    for (int it = 0;; ++it) {
      bool all = true;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const u32x2 pv = x_load_tagged(m, el[i]);
        v[i] = __uint_as_float(pv[0]);
        all = all && pv[1] == tag;
      }
      if (all) break;
      if (it + 1 >= kSpinLimit) {
        atomicOr(status, kStatusTimeout);
        break;
      }
      if ((it & 63) == 63 &&
          (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout))
        break;
      __builtin_amdgcn_s_sleep(1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = m.x[2 * el[i]];
  }
}

struct BSplit {
  float* xbuf;       // B*H heads x kHeadXFloats
  unsigned* flags;   // B*H heads x kFlagWords
  int head0, nheads;
};

template <int GELU_KIND>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_split_kernel(BwdParams p, BSplit x) {
  __shared__ BSmem sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  // block -> (head, part): the parts of a head are 8 blocks apart (same XCD)
  const int b = blockIdx.x;
  const int s = (b >> 3) % S;
  const int bh = x.head0 + ((b >> 3) / S) * 8 + (b & 7);
  if (bh >= x.nheads) return;  // both parts of a missing head leave together
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int hidx = bh % p.H;
  const int hs = s * (HID / S) + w * HS;
  const int T = p.T, nchunks = T / BC;
  bf16x4 I4 = make_ident(g, c16).i4;

  XMem m;
  m.x = x.xbuf + static_cast<size_t>(bh) * kHeadXFloats;
  m.cnt = x.flags + static_cast<size_t>(bh) * kFlagWords;
  m.fr = __builtin_amdgcn_make_buffer_rsrc(m.cnt, 0, kFlagWords * 4, kBufFlags);
  m.xr = __builtin_amdgcn_make_buffer_rsrc(m.x, 0, static_cast<int>(kHeadElems * 8), kBufFlags);
  {
    // placement: every part publishes its XCD id + 1 (device scope) and reads the other's
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (tid == 0) {
      __hip_atomic_store(m.cnt + 16 + s, xcc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool same = true;
      for (int o = 0; o < S; ++o) {
        unsigned v = 0;
        for (int it = 0; it < kSpinLimit && v == 0; ++it) {
          v = cnt_load(m, 16 + o);
          if (v == 0) __builtin_amdgcn_s_sleep(1);
        }
        if (v == 0) atomicOr(p.status, kStatusTimeout);
        same = same && v == xcc + 1;
      }
      sm.local = same && !(p.flags & TTT_FORCE_DEVICE_SCOPE) ? 1u : 0u;
    }
    __syncthreads();
    m.local = sm.local != 0;
  }

  float* work = p.work + static_cast<size_t>(bh) * bwd_work_floats_per_head(TTT_MLP, D, HID, BC);

  // ---- carried adjoint of the chunk-end weights (this wave's hidden units) ----
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

  // per-token lane mapping: token 4 w + lane / 16, 16 lanes per token, d = 16 i + lane % 16
  const int ln_t = 4 * w + g;
  float gam[PL], bet[PL], dgam[PL], dbet[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    gam[i] = p.gamma[hidx * D + 16 * i + c16];
    bet[i] = p.beta[hidx * D + 16 * i + c16];
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
  // chunk cc's exchange tag: 1, 2, ... in the order the chunks are processed (last first)
  auto tag_of = [&](int cc) { return static_cast<unsigned>(nchunks - cc); };

  // Row staging: thread -> token st_t, four consecutive d from st_d.
  const int st_t = tid >> 4, st_d = (tid & 15) * 4;
  auto gload = [&](int chunk, uint2& kk, uint2& qq, uint2& vv, uint2& zz, float& e) {
    const size_t off = (static_cast<size_t>(chunk) * BC + st_t) * D + st_d;
    kk = *reinterpret_cast<const uint2*>(Kg + off);
    qq = *reinterpret_cast<const uint2*>(Qg + off);
    vv = *reinterpret_cast<const uint2*>(Vg + off);
    zz = *reinterpret_cast<const uint2*>(dZg + off);
    e = tid < BC ? etag[chunk * BC + tid] : 0.f;
  };
  auto stage_write = [&](BStage& St, uint2 kk, uint2 qq, uint2 vv, uint2 zz, float e) {
    *reinterpret_cast<uint2*>(&St.K[st_t * RS + st_d]) = kk;
    *reinterpret_cast<uint2*>(&St.Q[st_t * RS + st_d]) = qq;
    *reinterpret_cast<uint2*>(&St.V[st_t * RS + st_d]) = vv;
    *reinterpret_cast<uint2*>(&St.dZ[st_t * RS + st_d]) = zz;
    if (tid < BC) St.eta[tid] = e * p.eta_scale;
  };
  // This part's sum over its waves of the dQ (red[1]) or dK (red[2]) partial of four elements
  // of a thread (token st_t, d = st_d .. st_d + 3).
  auto own_out = [&](int which, float (&o)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = st_t, d = st_d + k;
      const int dt = d >> 4, n = d & 15, r = t & 3, l = 16 * (t >> 2) + n;
      float a = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) a += sm.red[which].v[ww][dt][r][prot(r, l)];
      o[k] = a;
    }
  };
  // Send the partial of chunk cc that the other part finalizes: part 1 sends dQ, part 0 dK.
  auto send_out = [&](int cc) {
    float o[4];
    own_out(s == 1 ? 1 : 2, o);
    const int area = s == 1 ? kXDQ : kXDK;
#pragma unroll
    for (int k = 0; k < 4; ++k) x_store(m, xel(area, cc & 1, s, st_t * D + st_d + k), o[k], tag_of(cc));
    if (!m.local) publish(m, area, s, tag_of(cc));
  };
  // Write the output this part finalizes for chunk cc (part 0: dQ, part 1: dK): its own
  // partial plus the other part's, in part order.
  auto emit_out = [&](int cc) {
    const int area = s == 0 ? kXDQ : kXDK;
    if (!m.local) wait_other(m, area, s, tag_of(cc), p.status);
    float own[4], oth[4];
    own_out(s == 0 ? 1 : 2, own);
    int el[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) el[k] = xel(area, cc & 1, 1 - s, st_t * D + st_d + k);
    x_read(m, el, tag_of(cc), oth, p.status);
    __bf16* out = s == 0 ? dQg : dKg;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = s == 0 ? own[k] + oth[k] : oth[k] + own[k];
      out[static_cast<size_t>(cc * BC + st_t) * D + st_d + k] = (__bf16)v;
    }
  };
  // The head's total of a [16 x 64] sum over hidden units for the per-token lanes' elements:
  // this part's partial (sum over its waves of red[0]) is stored to the area's slot, the other
  // part's is read, and the two are added in part order.
  auto total = [&](int area, int cc, float (&z)[PL]) {
    const int t = ln_t;
    const unsigned tag = tag_of(cc);
    float own[PL], oth[PL];
    int el[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      own[i] = red_sum(sm.red[0], i, t, c16);
      x_store(m, xel(area, cc & 1, s, t * D + 16 * i + c16), own[i], tag);
      el[i] = xel(area, cc & 1, 1 - s, t * D + 16 * i + c16);
    }
    if (!m.local) {
      publish(m, area, s, tag);
      wait_other(m, area, s, tag, p.status);
    }
    x_read(m, el, tag, oth, p.status);
#pragma unroll
    for (int i = 0; i < PL; ++i) z[i] = s == 0 ? own[i] + oth[i] : oth[i] + own[i];
  };
  auto ln_stats16 = [&](const float (&z)[PL], float eps) {
    const float mu = sum16(z[0] + z[1] + z[2] + z[3]) * (1.0f / D);
    float var = 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) var += (z[i] - mu) * (z[i] - mu);
    var = sum16(var) * (1.0f / D);
    return LnStats{mu, __builtin_amdgcn_rsqf(var + eps)};
  };

  {
    uint2 kk, qq, vv, zz;
    float e;
    gload(nchunks - 1, kk, qq, vv, zz, e);
    stage_write(sm.st[(nchunks - 1) & 1], kk, qq, vv, zz, e);
  }
  // the start weights of the chunk to process next, loaded one chunk ahead (issued after the
  // chunk's last exchange, so that no poll of the exchange waits for them)
  f4 Wn1[NHT][NDT], Wn2[NDT][NHT];
  wT_load(saved + static_cast<size_t>(nchunks - 1) * 2 * D * HID,
          saved + static_cast<size_t>(nchunks - 1) * 2 * D * HID + D * HID, g, c16, hs, Wn1, Wn2);
  __syncthreads();

  for (int c = nchunks - 1; c >= 0; --c) {
    BStage& St = sm.st[c & 1];
    const int t0 = c * BC;
    const bool has_next = c > 0;
    // the dQ / dK partial of chunk c + 1 (from the last barrier) for the other part
    if (c + 1 < nchunks) send_out(c + 1);
    // next (earlier) chunk's rows, staged after the first LayerNorm
    uint2 nk{}, nq{}, nv{}, nz{};
    float ne = 0.f;
    if (has_next) gload(c - 1, nk, nq, nv, nz, ne);

    // this chunk's start weights, as bf16 operand tiles in both orientations
    bf16x4 W1b[NDT][NHT], W2b[NHT][NDT], W1T[NHT][NDT], W2T[NDT][NHT];
    {
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
    rows2(St.K, c16, g, aK);
    rows2(St.Q, c16, g, aQ);

    // ================= A: K side and Q W1 =================
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

    // ================= B: inner-gradient LayerNorm of Z^K; the output of chunk c + 1;
    // staging of chunk c - 1 =================
    float xk[PL], rk_[PL], d2k[PL], rsk, mgxk, etak;
    {
      const int t = ln_t;
      float z[PL];
      total(kXZK, c, z);
      const LnStats ls = ln_stats16(z, p.eps);
      float sg = 0.f, sgx = 0.f, gg[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 16 * i + c16;
        xk[i] = (z[i] - ls.mu) * ls.rs;
        rk_[i] = bf(St.K[t * RS + d]) + gam[i] * xk[i] + bet[i] - bf(St.V[t * RS + d]);
        gg[i] = 2.f * rk_[i] * gam[i];
        sg += gg[i];
        sgx += gg[i] * xk[i];
      }
      const float mg = sum16(sg) * (1.0f / D);
      mgxk = sum16(sgx) * (1.0f / D);
      rsk = ls.rs;
      etak = St.eta[t];
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 16 * i + c16;
        d2k[i] = (gg[i] - mg - xk[i] * mgxk) * rsk;
        sm.E2[t * RS + d] = (__bf16)(-etak * d2k[i]);
      }
    }
    if (c + 1 < nchunks) emit_out(c + 1);
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
    // P2 over this wave's hidden slice, both ways (this part's share of a sum over hidden
    // units: it enters only linear terms, which the exchanges add up)
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
      total(kXZQ, c, z);
      const LnStats ls = ln_stats16(z, p.eps);
      float xo[PL], v[PL], sv = 0.f, svx = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 16 * i + c16;
        xo[i] = (z[i] - ls.mu) * ls.rs;
        const float o = bf(St.dZ[t * RS + d]);
        dgam[i] += o * xo[i];
        dbet[i] += o;
        v[i] = o * gam[i];
        sv += v[i];
        svx += v[i] * xo[i];
      }
      const float mv = sum16(sv) * (1.0f / D), mvx = sum16(svx) * (1.0f / D);
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 16 * i + c16;
        sm.dZQ[t * RS + d] = (__bf16)((v[i] - mv - xo[i] * mvx) * ls.rs);
      }
    }
    __syncthreads();  // ---- 4

    // ================= E: Q-side adjoints, dE1, dE2 partial, dW terms =================
    I4 = fresh(I4);
    rows2(sm.E2, c16, g, aE);
    rows2(St.K, c16, g, aK);
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
      const bf16x4 qt = colsT(St.Q, dt, c16, g);
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

    // ================= F: inner-gradient backward per token; this part's dP1 =================
    {
      const int t = ln_t;
      float de[PL];
      total(kXDE2, c, de);
#pragma unroll
      for (int i = 0; i < PL; ++i) de[i] = -de[i];  // adjoint of eta d2
      float sq = 0.f, su = 0.f, sux = 0.f, u[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        sq += de[i] * d2k[i];
        u[i] = etak * de[i];
        su += u[i];
        sux += u[i] * xk[i];
      }
      const float deta = sum16(sq) * p.eta_scale;
      const float mu = sum16(su) * (1.0f / D), mux = sum16(sux) * (1.0f / D);
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
      const float ds = -rsk * sum16(suq);
      float sdx = 0.f, sdxx = 0.f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        sdx += dx[i];
        sdxx += dx[i] * xk[i];
      }
      const float mdx = sum16(sdx) * (1.0f / D), mdxx = sum16(sdxx) * (1.0f / D);
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int d = 16 * i + c16;
        sm.dZK[t * RS + d] = (__bf16)(rsk * (dx[i] - mdx - xk[i] * mdxx) + ds * xk[i] * (1.0f / D));
        sm.dKres[t * D + d] = dr[i];
        if (s == 0) dVg[static_cast<size_t>(t0 + t) * D + d] = (__bf16)(-dr[i]);
      }
      if (c16 == 0 && s == 0) {
        p.deta[static_cast<size_t>(bh) * T + t0 + t] = deta;
        flag_nonfinite(p.status, deta);
      }
    }
    {
      // this part's dP1 = sum of its waves' partials, as two bf16 operand layouts
      const int t = tid >> 4, u = tid & 15;
      const int r = t & 3, l = 16 * (t >> 2) + u;
      float a = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) a += sm.dp1p[ww][r][l];
      const __bf16 e = (__bf16)a;
      sm.dP1r[t * TS + u] = e;
      sm.dP1c[u * TS + t] = e;
    }
    __syncthreads();  // ---- 6

    // ================= G: dAK, dHK, dK, remaining dW terms =================
    if (has_next)
      wT_load(saved + static_cast<size_t>(c - 1) * 2 * D * HID,
              saved + static_cast<size_t>(c - 1) * 2 * D * HID + D * HID, g, c16, hs, Wn1, Wn2);
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
        // the terms not split over hidden units, one d tile per wave: this part's dP1 into
        // both (dP1^T Q into dK, dP1 K into dQ); the residual into dK on the part that writes
        // dK, dz into dQ on the part that writes dQ
        dk = mfma16(lds4(&sm.dP1c[c16 * TS + 4 * g]), colsT(St.Q, dt, c16, g), dk);
        if (s == 1) {
#pragma unroll
          for (int r = 0; r < 4; ++r) dk[r] += sm.dKres[(4 * g + r) * D + 16 * dt + c16];
        }
        f4 dq = get_tile(sm.red[1], w, dt, lane);
        dq = mfma16(lds4(&sm.dP1r[c16 * TS + 4 * g]), colsT(St.K, dt, c16, g), dq);
        if (s == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) dq[r] += bf(St.dZ[(4 * g + r) * RS + 16 * dt + c16]);
        }
        put_tile(sm.red[1], w, dt, lane, dq);
      }
      put_tile(sm.red[2], w, dt, lane, dk);
      const bf16x4 kt = colsT(St.K, dt, c16, g);
      const bf16x4 zkt = colsT(sm.dZK, dt, c16, g);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        dW1c[dt][ht] = mfma16(kt, dhkR[ht], dW1c[dt][ht]);
        dW2c[ht][dt] = mfma16(akR[ht], zkt, dW2c[ht][dt]);
      }
    }
    __syncthreads();  // ---- 7
  }
  send_out(0);
  emit_out(0);

  // dW of the first chunk's start = dW0 of this head (this part's hidden units); dgamma /
  // dbeta partials (both parts hold the same per-token values: part 0 writes them)
  wtiles_store<NHT>(work, work + D * HID, g, c16, hs, dW1c, dW2c);
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    // sum over the four tokens of this wave (lanes with equal lane % 16)
    float a = dgam[i], bb = dbet[i];
    a += __shfl_xor(a, 16, 64);
    bb += __shfl_xor(bb, 16, 64);
    a += __shfl_xor(a, 32, 64);
    bb += __shfl_xor(bb, 32, 64);
    if (lane < 16) {
      sm.dgb[w][0][16 * i + c16] = a;
      sm.dgb[w][1][16 * i + c16] = bb;
    }
  }
  __syncthreads();
  if (s == 0 && tid < 2 * D) {
    const int k = tid >> 6, d = tid & 63;
    float a = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) a += sm.dgb[ww][k][d];
    p.dgb[static_cast<size_t>(bh) * 2 * D + k * D + d] = a;
  }
}

// Clears the exchange areas (their tags) and the counter words of every head.
__global__ void bwd_split_reset_kernel(uint4* wp, size_t n4) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    wp[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

size_t bwd_split_workspace_bytes(int nheads) {
  return static_cast<size_t>(nheads) * (kHeadXFloats * sizeof(float) + kFlagWords * sizeof(unsigned));
}

// Resident workgroups of the split backward on the current device (0 when it cannot launch
// cooperatively), cached per device ordinal.
static int bwd_split_capacity() {
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
            &per_cu, reinterpret_cast<const void*>(bwd_split_kernel<TTT_GELU_ERF>), NT, 0) == hipSuccess;
    cap[dev] = 1 + ((ok && coop) ? ncu * per_cu : 0);
  }
  return cap[dev] - 1;
}

// Heads per launch: whole groups of eight heads whose two parts all fit on the device at once.
static int bwd_split_heads_per_launch() { return bwd_split_capacity() / (8 * S) * 8; }

bool bwd_split_fits() { return bwd_split_heads_per_launch() > 0; }

hipError_t launch_bwd_mfma_split(const BwdParams& p, float* xbuf, hipStream_t stream) {
  const int nheads = p.B * p.H;
  const int per = bwd_split_heads_per_launch();
  if (per <= 0) return hipErrorCooperativeLaunchTooLarge;
  BSplit x;
  x.xbuf = xbuf;
  x.flags = reinterpret_cast<unsigned*>(xbuf + static_cast<size_t>(nheads) * kHeadXFloats);
  x.nheads = nheads;
  const size_t n4 = static_cast<size_t>(nheads) * (kHeadXFloats + kFlagWords) / 4;
  const unsigned rblocks = static_cast<unsigned>(n4 / 256 + 1 < 2048 ? n4 / 256 + 1 : 2048);
  hipLaunchKernelGGL(bwd_split_reset_kernel, dim3(rblocks), dim3(256), 0, stream, reinterpret_cast<uint4*>(xbuf), n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* fn = p.gelu == TTT_GELU_TANH ? reinterpret_cast<const void*>(bwd_split_kernel<TTT_GELU_TANH>)
                                           : reinterpret_cast<const void*>(bwd_split_kernel<TTT_GELU_ERF>);
  for (int h0 = 0; h0 < nheads; h0 += per) {
    BwdParams pc = p;
    x.head0 = h0;
    void* args[] = {&pc, &x};
    const int n = nheads - h0 < per ? nheads - h0 : per;
    e = hipLaunchCooperativeKernel(fn, dim3((n + 7) / 8 * 8 * S), dim3(NT), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ttt
