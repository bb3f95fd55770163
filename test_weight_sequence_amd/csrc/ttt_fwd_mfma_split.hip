// Tuned forward scan for the long-context TTT-MLP head shape d = 128, hidden = 512, chunk 16,
// bf16 Q/K/V/Z, fp32 fast weights (gfx950, bf16 MFMA with fp32 accumulation).
//
// A head's fp32 fast weights (W1 128 x 512 and W2 512 x 128, 512 KiB) are as large as one
// CU's whole register file, so the head is split by hidden units over S = 4 workgroups of 4
// waves (one wave per SIMD): workgroup s holds hidden units [128 s, 128 s + 128) and its
// wave w the 32 units from 128 s + 32 w, as fp32 MFMA accumulator tiles that stay in
// registers for the whole scan. Everything that is per hidden unit (H^K, A^K, E1, H^Q,
// A^Q, the weight update) is local to a workgroup. The two sums over all hidden units that
// every chunk needs, Z^K = A^K W2 (for the inner-loss LayerNorm) and
// Z^Q = A^Q W2 + tril(A^Q A^K^T) E2 (for the output), are formed from the four
// workgroups' [16 x 128] partial sums: each workgroup writes its partial to a slot in the
// workspace, raises its counter, waits for the other three and adds the four partials in the
// same fixed order, so all four compute bit-identical sums and therefore the same E2. Only
// Z^K is waited for: a workgroup publishes its Z^Q partial of chunk c before its Z^K partial
// of chunk c + 1, so once the Z^K wait of chunk c + 1 is over, the Z^Q partials of chunk c
// are all in place, and the output of chunk c is written then.
//
// Per chunk (E = eta-scaled, negated rows; all at the chunk-start weights): the dual form
// of the per-token rule on the page "Test-Time Training(TTT)과 LLM 메모리", section
// "TTT layer", Eq. 2/4/5, with the mini-batch rule of the E2E paper review, section 2.3,
// Eq. 5:
//   H^K = K W1, A^K = GELU, G = GELU';  Z^K = A^K W2 (summed over the workgroups)
//   LN fwd/bwd of Z^K per token -> En2 = -eta * delta2;  E1n = (En2 W2^T) (.) G
//   H^Q = Q W1 + tril(Q K^T) E1n, A^Q = GELU;  Z^Q = A^Q W2 + tril(A^Q A^K^T) En2 (summed)
//   z = Q + LN(Z^Q);  W1 += K^T E1n, W2 += A^K^T En2
// The four workgroups of a head are numbered so that the hardware's round-robin placement
// puts them on one XCD. They check that at start (HW_REG_XCC_ID): on one XCD the exchange
// goes through that XCD's L2 with plain stores and loads that skip the CU's L1; otherwise it
// uses device-scope release/acquire fences.
//
// Two forms share this code. In the first (fwd_split_kernel) every workgroup runs both sides
// of the chunk. In the producer/consumer form (fwd_split_pair_kernel, below), used when all
// heads fit in one launch of it, four more workgroups per head take the query side, so the
// chunk-to-chunk chain through the Z^K exchange carries only the key side.
#include "ttt_mfma_common.hpp"

namespace ttt {
namespace {

using mfma::bf16x4;
using mfma::bf16x8;
using mfma::f4;
using mfma::cat;
using mfma::cvt4;
using mfma::lds4;
using mfma::mfma16;
using mfma::mfma32;
using mfma::sum16;
using mfma::zero4;

constexpr int D = 128;
constexpr int HID = 512;
constexpr int BC = 16;
constexpr int NDT = D / 16;          // d tiles
constexpr int S = 4;                 // workgroups per head
constexpr int NW = 4;                // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int HS = HID / (S * NW);   // hidden units per wave
constexpr int NHT = HS / 16;         // h tiles per wave
constexpr int NKD = D / 32;          // 32-wide k-steps over d
constexpr int RS = D + 8;            // row stride (bf16) of [token][d] arrays
constexpr int DPL = D / 16;          // d values per LayerNorm lane
constexpr int kSpinLimit = 1 << 20;
static_assert(NHT == 2 && NW * 4 == BC, "tile split");

// Workspace per head: two exchange areas (Z^K, Z^Q) of two chunk-parity slots of S partial
// [16 x 128] fp32 sums, then (after all heads) 32 counter words per head. On one XCD the
// partials carry their own readiness: each element is stored with the chunk's tag in one
// 8-byte store, and a reader polls its elements until the tags match (the area is cleared
// before every launch). Across XCDs the parts exchange counters with device-scope fences.
constexpr size_t kPartFloats = static_cast<size_t>(BC) * D;
// Each element travels as a (value, tag) pair of 32-bit words, the tag being the chunk index + 1.
constexpr size_t kHeadXFloats = 2 * 2 * S * kPartFloats * 2;
// [0, S): Z^K counters, [8, 8 + S): Z^Q, [16, 16 + 2 S): XCD ids, [32, 52): the hand-off counters
// of the producer/consumer form
constexpr int kFlagWords = 64;
constexpr int kLoadL2 = 16;     // cache policy of exchange loads on one XCD: device scope (sc1)

struct Stage {
  alignas(16) __bf16 K[BC * RS];
  alignas(16) __bf16 Q[BC * RS];
  alignas(16) __bf16 V[BC * RS];
  float eta[BC];
};

struct Smem {
  Stage st[3];                        // chunk c lives in st[c % 3]
  // per-wave [token x d] partial tiles (lane-rotated rows): [0] Z^K, [1] Z^Q. Separate
  // buffers, so that a chunk's Z^K partials are never written while the previous chunk's Z^Q
  // partials are still being read (no barrier lies between those reads and these writes).
  float red[2][NW][NDT][4][64];
  alignas(16) __bf16 E2[BC * RS];     // En2, [token][d]
};

__device__ __forceinline__ int prot(int r, int lane) { return (lane + 16 * r) & 63; }

struct Split {
  float* xbuf;        // exchange areas, kHeadXFloats per head
  unsigned* flags;    // kFlagWords per head
  char* ring;         // hand-off rings of the producer/consumer form, kRingBytes per head
  int nheads;         // heads in the whole call
  int head0;          // first head of this launch (heads are launched in groups the device holds)
};

// fp32 weight tiles of one wave: W1[:, hb:hb+32] as [d tile][h tile], W2[hb:hb+32, :] as
// [h tile][d tile] (accumulator layout: row 4 (lane/16) + r, column lane % 16), moved with
// buffer instructions: one per-lane offset register plus a scalar offset per element.
__device__ __forceinline__ void w_load(const float* w1, const float* w2, int g, int c16, int hb,
                                       f4 (&W1c)[NDT][NHT], f4 (&W2c)[NHT][NDT]) {
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w1), 0, D * HID * 4, mfma::kBufFlags);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w2), 0, D * HID * 4, mfma::kBufFlags);
  const int v1 = (4 * g * HID + hb + c16) * 4, v2 = ((hb + 4 * g) * D + c16) * 4;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        W1c[dt][ht][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, v1, ((16 * dt + r) * HID + 16 * ht) * 4, 0));
        W2c[ht][dt][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r2, v2, ((16 * ht + r) * D + 16 * dt) * 4, 0));
      }
}
// (each element is copied to a scalar float before the store: a bit_cast applied directly
// to a vector element was compiled as a read of element 0)
__device__ __forceinline__ void w_store(float* w1, float* w2, int g, int c16, int hb,
                                        const f4 (&W1c)[NDT][NHT], const f4 (&W2c)[NHT][NDT]) {
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(w1, 0, D * HID * 4, mfma::kBufFlags);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(w2, 0, D * HID * 4, mfma::kBufFlags);
  const int v1 = (4 * g * HID + hb + c16) * 4, v2 = ((hb + 4 * g) * D + c16) * 4;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = W1c[dt][ht][r], b = W2c[ht][dt][r];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r1, v1, ((16 * dt + r) * HID + 16 * ht) * 4, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(b), r2, v2, ((16 * ht + r) * D + 16 * dt) * 4, 0);
      }
}

// The exchange memory of one head: counter words and the Z^K / Z^Q partial slots.
struct XMem {
  unsigned* cnt;
  float* xz;
  float* xq;
  __amdgpu_buffer_rsrc_t fr, zr, qr;
  bool local;  // all parts on one XCD
};

__device__ __forceinline__ unsigned cnt_load(const XMem& m, int i) {
  if (m.local) return __builtin_amdgcn_raw_buffer_load_b32(m.fr, 0, 4 * i, kLoadL2);
  return __hip_atomic_load(m.cnt + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish the partial that every thread has just stored as chunk c (counter word base + s
// := c + 1): the stores are complete before the counter store.
__device__ __forceinline__ void publish(const XMem& m, int base, int s, unsigned c1) {
  if (m.local)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    if (m.local)
      __builtin_amdgcn_raw_buffer_store_b32(c1, m.fr, 0, 4 * (base + s), 0);
    else
      __hip_atomic_store(m.cnt + base + s, c1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait until the other parts' counters base + o reach c1. Bounded: an expired wait sets the
// timeout bit, and once that bit is set no later wait spins, so a lost partner costs one
// bound in total.
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
  if (!m.local) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// one element of a partial slot area (element offset; elements are (value, tag) pairs)
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;
typedef u64 u64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 part_load_tagged(const XMem& m, bool zq, int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(zq ? m.qr : m.zr, 8 * off, 0, kLoadL2));
}
__device__ __forceinline__ float part_load(const XMem& m, bool zq, int off) {
  return (zq ? m.xq : m.xz)[2 * off];
}
__device__ __forceinline__ void part_store(const XMem& m, bool zq, int off, float v, unsigned tag) {
  if (m.local) {
    const u32x2 pv = {__float_as_uint(v), tag};
    __builtin_amdgcn_raw_buffer_store_b64(pv, zq ? m.qr : m.zr, 8 * off, 0, 0);
  } else {
    (zq ? m.xq : m.xz)[2 * off] = v;
  }
}

template <int GELU_KIND>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
fwd_split_kernel(ScanParams p, Split x) {
  __shared__ Smem sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  // block -> (head, part): the S parts of a head are 8 blocks apart (same XCD)
  const int b = blockIdx.x;
  const int s = (b >> 3) % S;
  const int bh = x.head0 + ((b >> 3) / S) * 8 + (b & 7);
  if (bh >= x.nheads) return;  // all parts of a missing head leave together
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
  m.xz = x.xbuf + static_cast<size_t>(bh) * kHeadXFloats;  // [slot][S][16 x 128]
  m.xq = m.xz + 2 * 2 * S * kPartFloats;
  m.cnt = x.flags + static_cast<size_t>(bh) * kFlagWords;
  m.fr = __builtin_amdgcn_make_buffer_rsrc(m.cnt, 0, kFlagWords * 4, mfma::kBufFlags);
  m.zr = __builtin_amdgcn_make_buffer_rsrc(m.xz, 0, 2 * S * kPartFloats * 8, mfma::kBufFlags);
  m.qr = __builtin_amdgcn_make_buffer_rsrc(m.xq, 0, 2 * S * kPartFloats * 8, mfma::kBufFlags);
  {
    // placement: every part publishes its XCD id + 1 (device scope) and reads the others'
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

  f4 W1c[NDT][NHT], W2c[NHT][NDT];
  {
    const size_t wh = per_seq ? static_cast<size_t>(bh) : static_cast<size_t>(hidx);
    w_load(p.w0_1 + wh * D * HID, p.w0_2 + wh * HID * D, g, c16, hb, W1c, W2c);
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
  const float* etag = p.eta + static_cast<size_t>(bh) * T;

  // staging: thread -> token st_t, 8 consecutive d from st_d
  const int st_t = tid >> 4, st_d = (tid & 15) * 8;
  auto gload = [&](int chunk, uint4& kk, uint4& qq, uint4& vv, float& e) {
    const size_t off = (static_cast<size_t>(chunk) * BC + st_t) * D + st_d;
    kk = *reinterpret_cast<const uint4*>(Kg + off);
    qq = *reinterpret_cast<const uint4*>(Qg + off);
    vv = *reinterpret_cast<const uint4*>(Vg + off);
    e = tid < BC ? etag[chunk * BC + tid] : 0.f;
  };
  auto stage_write = [&](Stage& St, uint4 kk, uint4 qq, uint4 vv, float e) {
    *reinterpret_cast<uint4*>(&St.K[st_t * RS + st_d]) = kk;
    *reinterpret_cast<uint4*>(&St.Q[st_t * RS + st_d]) = qq;
    *reinterpret_cast<uint4*>(&St.V[st_t * RS + st_d]) = vv;
    if (tid < BC) St.eta[tid] = e * p.eta_scale;
  };
  // this workgroup's [16 x 128] partial for the LayerNorm lanes' elements, from the waves'
  // tiles in red (fixed wave order)
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
  auto ln_stats8 = [&](const float (&z)[DPL], float& mu, float& rs) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) a += z[i];
    mu = sum16(a) * (1.0f / D);
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) v += (z[i] - mu) * (z[i] - mu);
    rs = __builtin_amdgcn_rsqf(sum16(v) * (1.0f / D) + p.eps);
  };
  // store this part's partial of chunk parity `slot` (the LayerNorm lanes' elements)
  auto put_own = [&](bool zq, int slot, unsigned tag, float (&own)[DPL]) {
    own_partial(zq, own);
#pragma unroll
    for (int i = 0; i < DPL; ++i)
      part_store(m, zq, (slot * S + s) * kPartFloats + ln_t * D + 16 * i + c16, own[i], tag);
  };
  // the head's total from the S partials of a slot (fixed part order; this part's own from
  // registers). On one XCD each lane polls its elements until every tag reads `tag` (bounded;
  // on expiry the timeout bit is set and the values are whatever was read).
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
  // output z = Q + LN(Z^Q) of chunk cc for this part's tokens (wave s: tokens 4 s .. 4 s + 3)
  float ownQ[DPL];  // this part's Z^Q partial of the chunk whose output is still to be written
  auto ln_out = [&](int cc) {
    const Stage& So = sm.st[cc % 3];
    const int t = ln_t;
    float z[DPL];
    total(true, cc & 1, static_cast<unsigned>(cc) + 1u, ownQ, z);
    float mu, rs;
    ln_stats8(z, mu, rs);
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

  {
    uint4 kk, qq, vv;
    float e;
    gload(0, kk, qq, vv, e);
    stage_write(sm.st[0], kk, qq, vv, e);
  }
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    Stage& St = sm.st[c % 3];
    const int t0 = c * BC;
    const unsigned c1 = static_cast<unsigned>(c) + 1u;
    const int slot = c & 1;
    uint4 nk{}, nq{}, nv{};
    float ne = 0.f;
    const bool has_next = c + 1 < nchunks;
    if (has_next) gload(c + 1, nk, nq, nv, ne);
    if (p.saved) {
      float* sv = p.saved + (static_cast<size_t>(bh) * nchunks + c) * (2 * D * HID);
      w_store(sv, sv + D * HID, g, c16, hb, W1c, W2c);
    }

    bf16x8 aK[NKD], aQ[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      aK[ks] = cat(lds4(&St.K[c16 * RS + 32 * ks + 4 * g]), lds4(&St.K[c16 * RS + 32 * ks + 16 + 4 * g]));
      aQ[ks] = cat(lds4(&St.Q[c16 * RS + 32 * ks + 4 * g]), lds4(&St.Q[c16 * RS + 32 * ks + 16 + 4 * g]));
    }
    bf16x4 W1b[NDT][NHT], W2b[NHT][NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        W1b[dt][ht] = cvt4(W1c[dt][ht]);
        W2b[ht][dt] = cvt4(W2c[ht][dt]);
      }

    // ---- K side: H^K = K W1, A^K, G; Z^K partial over this wave's hidden units ----
    bf16x4 akR[NHT], akT[NHT];
    f4 gk[NHT], hq[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 acc = zero4(), accq = zero4();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        const bf16x8 wb = cat(W1b[2 * ks][ht], W1b[2 * ks + 1][ht]);
        acc = mfma32(aK[ks], wb, acc);
        accq = mfma32(aQ[ks], wb, accq);
      }
      hq[ht] = accq;
      f4 a, gd;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v, d1;
        mfma::act_d<GELU_KIND>(acc[r], v, d1);
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
      const f4 acc = mfma32(cat(akT[0], akT[1]), cat(W2b[0][dt], W2b[1][dt]), zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[0][w][dt][r][prot(r, lane)] = acc[r];
    }
    f4 s1t = zero4();  // C[s][t] = K_s . Q_t
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) s1t = mfma32(aK[ks], aQ[ks], s1t);
    __syncthreads();

    // ---- Z^K over all hidden units (this wait also covers the Z^Q partials of chunk c - 1,
    // whose output is written now), LayerNorm forward/backward -> En2 ----
    float ownK[DPL];
    put_own(false, slot, c1, ownK);
    if (!m.local) {
      publish(m, 0, s, c1);
      wait_all(m, 0, s, c1, p.status);
    }
    if (c > 0 && w == s) ln_out(c - 1);
    {
      const int t = ln_t;
      float z[DPL];
      total(false, slot, c1, ownK, z);
      float mu, rs;
      ln_stats8(z, mu, rs);
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
      const float ne2 = -St.eta[t] * rs;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = 16 * i + c16;
        const __bf16 e = (__bf16)(ne2 * (gg[i] - mg - xh[i] * mgx));
        sm.E2[t * RS + d] = e;
      }
      if (c16 == 0 && s == 0) {
        if (p.loss) p.loss[static_cast<size_t>(bh) * T + t0 + t] = loss;
        flag_nonfinite(p.status, loss);
      }
    }
    if (has_next) stage_write(sm.st[(c + 1) % 3], nk, nq, nv, ne);
    __syncthreads();

    // ---- E1n = (En2 W2^T) (.) G ; H^Q ; A^Q ; Z^Q partial ----
    bf16x8 aE[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks)
      aE[ks] = cat(lds4(&sm.E2[c16 * RS + 32 * ks + 4 * g]), lds4(&sm.E2[c16 * RS + 32 * ks + 16 + 4 * g]));
    bf16x4 e1[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks)
        acc = mfma32(aE[ks], cat(cvt4(mfma16(W2b[ht][2 * ks], I4, zero4())),
                                 cvt4(mfma16(W2b[ht][2 * ks + 1], I4, zero4()))), acc);
      e1[ht] = cvt4(acc * gk[ht]);
    }
    f4 s1m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s1m[r] = (4 * g + r) <= c16 ? s1t[r] : 0.f;
    const bf16x4 s1a = cvt4(s1m);
    bf16x4 aqT[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const f4 h = mfma16(s1a, e1[ht], hq[ht]);
      f4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = mfma::act<GELU_KIND>(h[r]);
      aqT[ht] = cvt4(mfma16(cvt4(a), I4, zero4()));
    }
    f4 s2t = mfma32(cat(akT[0], akT[1]), cat(aqT[0], aqT[1]), zero4());  // C[s][t] = A^K_s . A^Q_t
    f4 s2m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s2m[r] = (4 * g + r) <= c16 ? s2t[r] : 0.f;
    const bf16x4 s2a = cvt4(s2m);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x4 be = mfma::tgroup(sm.E2, RS, dt, g, c16);
      f4 acc = mfma32(cat(aqT[0], aqT[1]), cat(W2b[0][dt], W2b[1][dt]), zero4());
      acc = mfma16(s2a, be, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[1][w][dt][r][prot(r, lane)] = acc[r];
      // chunk-end update of this wave's fp32 weights
      const bf16x4 kt = mfma::tgroup(St.K, RS, dt, g, c16);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        W1c[dt][ht] = mfma16(kt, e1[ht], W1c[dt][ht]);
        W2c[ht][dt] = mfma16(akR[ht], be, W2c[ht][dt]);
      }
    }
    __syncthreads();

    // ---- publish this part's Z^Q partial of chunk c (its output is written next chunk) ----
    put_own(true, slot, c1, ownQ);
    if (!m.local) publish(m, 8, s, c1);
  }
  if (!m.local) wait_all(m, 8, s, static_cast<unsigned>(nchunks), p.status);
  if (w == s) ln_out(nchunks - 1);

  if (p.wt_1)
    w_store(p.wt_1 + static_cast<size_t>(bh) * D * HID, p.wt_2 + static_cast<size_t>(bh) * HID * D,
            g, c16, hb, W1c, W2c);
}

// ---------------------------------------------------------------------------------------
// Producer/consumer form, eight workgroups per head. Parts 0..3 (producers) hold the hidden
// slices of the weights exactly as above and run the key side of every chunk: H^K, A^K, G,
// the Z^K exchange among themselves, the LayerNorm forward/backward and E1n. Parts 4..7
// (consumers; consumer s + 4 holds the same hidden units as producer s) replay the same
// weight update from the same bf16 operands, so their fp32 weights stay bitwise equal, and run
// the query side: H^Q, A^Q, the Z^Q exchange among themselves and the output. Producer s hands
// each chunk's E1n and A^K of its units and the chunk's En2 rows to consumer s through a ring
// of chunk slots in the workspace, wave by wave: producer wave w raises its counter once its
// stores of the slot have completed, consumer wave w loads its part of the slot only after it
// has seen that counter, and the consumer workgroup raises a counter of chunks it is done
// reading. Nothing flows back from the query side, so it is off the chunk-to-chunk chain.
// ---------------------------------------------------------------------------------------
constexpr int RINGD = 4;                         // chunk slots per producer/consumer pair
constexpr int SLOT_E1 = 0;                        // E1n: producer wave w, lane l: 16 bytes at (w * 64 + l) * 16
constexpr int SLOT_AK = NW * 64 * 16;             // A^K, the same layout
constexpr int SLOT_E2 = 2 * NW * 64 * 16;         // En2 rows 4 w .. 4 w + 3: lane l holds row 4 w + l / 16, d = 8 (l % 16) ..
constexpr int SLOT_BYTES = 3 * NW * 64 * 16;      // 12 KiB
constexpr size_t kRingBytes = static_cast<size_t>(S) * RINGD * SLOT_BYTES;  // per head
constexpr int kCntReady = 32;                     // + 4 s + w: chunks published by producer s's wave w
constexpr int kCntRead = 48;                      // + s: chunks consumer s has finished reading

struct SplitRing {
  char* ring;                  // this pair's RINGD slots
  __amdgpu_buffer_rsrc_t rr;
};

template <int GELU_KIND>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
fwd_split_pair_kernel(ScanParams p, Split x) {
  __shared__ Smem sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  // block -> (head, role, part): the 2 S workgroups of a head are 8 blocks apart (same XCD)
  const int b = blockIdx.x;
  const int q = (b >> 3) % (2 * S);
  const int s = q % S;
  const bool consumer = q >= S;
  const int bh = x.head0 + ((b >> 3) / (2 * S)) * 8 + (b & 7);
  if (bh >= x.nheads) return;  // all workgroups of a missing head leave together
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
  m.xz = x.xbuf + static_cast<size_t>(bh) * kHeadXFloats;  // [slot][S][16 x 128]
  m.xq = m.xz + 2 * 2 * S * kPartFloats;
  m.cnt = x.flags + static_cast<size_t>(bh) * kFlagWords;
  m.fr = __builtin_amdgcn_make_buffer_rsrc(m.cnt, 0, kFlagWords * 4, mfma::kBufFlags);
  m.zr = __builtin_amdgcn_make_buffer_rsrc(m.xz, 0, 2 * S * kPartFloats * 8, mfma::kBufFlags);
  m.qr = __builtin_amdgcn_make_buffer_rsrc(m.xq, 0, 2 * S * kPartFloats * 8, mfma::kBufFlags);
  SplitRing rg;
  rg.ring = x.ring + static_cast<size_t>(bh) * kRingBytes + static_cast<size_t>(s) * RINGD * SLOT_BYTES;
  rg.rr = __builtin_amdgcn_make_buffer_rsrc(rg.ring, 0, RINGD * SLOT_BYTES, mfma::kBufFlags);
  {
    // placement: every workgroup publishes its XCD id + 1 (device scope) and reads the others'
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (threadIdx.x == 0) {
      __hip_atomic_store(m.cnt + 16 + q, xcc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool same = true;
      for (int o = 0; o < 2 * S; ++o) {
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
  // hand-off accesses: on one XCD plain stores and device-scope (L1-skipping) loads that meet
  // in the L2; otherwise agent-scope atomics
  auto ring_st = [&](int off, bf16x8 v) {
    if (m.local) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rg.rr, off, 0, 0);
    } else {
      const u64x2 xv = __builtin_bit_cast(u64x2, v);
      u64* qp = reinterpret_cast<u64*>(rg.ring + off);
      __hip_atomic_store(qp, xv[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(qp + 1, xv[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto ring_ld = [&](int off) {
    if (m.local) return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rg.rr, off, 0, kLoadL2));
    const u64* qp = reinterpret_cast<const u64*>(rg.ring + off);
    const u64x2 v = {__hip_atomic_load(qp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     __hip_atomic_load(qp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
    return __builtin_bit_cast(bf16x8, v);
  };
  auto cnt_st = [&](int i, unsigned v) {
    if (m.local)
      __builtin_amdgcn_raw_buffer_store_b32(v, m.fr, 0, 4 * i, 0);
    else
      __hip_atomic_store(m.cnt + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // wait until counter word i >= target (bounded; gives up at once after any timeout)
  auto cnt_wait = [&](int i, unsigned target) {
    for (int it = 0; it < kSpinLimit; ++it) {
      if (cnt_load(m, i) >= target) return;
      if ((it & 63) == 0 && (__hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout))
        return;
      __builtin_amdgcn_s_sleep(2);
    }
    atomicOr(p.status, kStatusTimeout);
  };

  f4 W1c[NDT][NHT], W2c[NHT][NDT];
  {
    const size_t wh = per_seq ? static_cast<size_t>(bh) : static_cast<size_t>(hidx);
    w_load(p.w0_1 + wh * D * HID, p.w0_2 + wh * HID * D, g, c16, hb, W1c, W2c);
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
  const float* etag = p.eta + static_cast<size_t>(bh) * T;

  // staging: thread -> token st_t, 8 consecutive d from st_d; a producer stages K, V and eta,
  // a consumer K and Q
  const int st_t = tid >> 4, st_d = (tid & 15) * 8;
  auto gload = [&](int chunk, uint4& kk, uint4& xx, float& e) {
    const size_t off = (static_cast<size_t>(chunk) * BC + st_t) * D + st_d;
    kk = *reinterpret_cast<const uint4*>(Kg + off);
    xx = *reinterpret_cast<const uint4*>((consumer ? Qg : Vg) + off);
    e = (!consumer && tid < BC) ? etag[chunk * BC + tid] : 0.f;
  };
  auto stage_write = [&](Stage& St, uint4 kk, uint4 xx, float e) {
    *reinterpret_cast<uint4*>(&St.K[st_t * RS + st_d]) = kk;
    *reinterpret_cast<uint4*>(&(consumer ? St.Q : St.V)[st_t * RS + st_d]) = xx;
    if (!consumer && tid < BC) St.eta[tid] = e * p.eta_scale;
  };
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
  auto ln_stats8 = [&](const float (&z)[DPL], float& mu, float& rs) {
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

  {
    uint4 kk, xx;
    float e;
    gload(0, kk, xx, e);
    stage_write(sm.st[0], kk, xx, e);
  }
  __syncthreads();

  if (!consumer) {
    // ===================================== producer =====================================
    for (int c = 0; c < nchunks; ++c) {
      Stage& St = sm.st[c % 3];
      const int t0 = c * BC;
      const unsigned c1 = static_cast<unsigned>(c) + 1u;
      const int slot = c & 1;
      uint4 nk{}, nx{};
      float ne = 0.f;
      const bool has_next = c + 1 < nchunks;
      if (has_next) gload(c + 1, nk, nx, ne);
      if (p.saved) {
        float* sv = p.saved + (static_cast<size_t>(bh) * nchunks + c) * (2 * D * HID);
        w_store(sv, sv + D * HID, g, c16, hb, W1c, W2c);
      }
      bf16x8 aK[NKD];
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks)
        aK[ks] = cat(lds4(&St.K[c16 * RS + 32 * ks + 4 * g]), lds4(&St.K[c16 * RS + 32 * ks + 16 + 4 * g]));
      bf16x4 W1b[NDT][NHT], W2b[NHT][NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          W1b[dt][ht] = cvt4(W1c[dt][ht]);
          W2b[ht][dt] = cvt4(W2c[ht][dt]);
        }
      // ---- H^K = K W1, A^K, G; Z^K partial over this wave's hidden units ----
      bf16x4 akR[NHT], akT[NHT];
      f4 gk[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        f4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) acc = mfma32(aK[ks], cat(W1b[2 * ks][ht], W1b[2 * ks + 1][ht]), acc);
        f4 a, gd;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v, d1;
          mfma::act_d<GELU_KIND>(acc[r], v, d1);
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
        const f4 acc = mfma32(cat(akT[0], akT[1]), cat(W2b[0][dt], W2b[1][dt]), zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.red[0][w][dt][r][prot(r, lane)] = acc[r];
      }
      __syncthreads();
      // ---- Z^K over all hidden units, LayerNorm forward/backward -> En2 ----
      float ownK[DPL];
      put_own(false, slot, c1, ownK);
      if (!m.local) {
        publish(m, 0, s, c1);
        wait_all(m, 0, s, c1, p.status);
      }
      {
        const int t = ln_t;
        float z[DPL];
        total(false, slot, c1, ownK, z);
        float mu, rs;
        ln_stats8(z, mu, rs);
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
        const float ne2 = -St.eta[t] * rs;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          const int d = 16 * i + c16;
          sm.E2[t * RS + d] = (__bf16)(ne2 * (gg[i] - mg - xh[i] * mgx));
        }
        if (c16 == 0 && s == 0) {
          if (p.loss) p.loss[static_cast<size_t>(bh) * T + t0 + t] = loss;
          flag_nonfinite(p.status, loss);
        }
      }
      if (has_next) stage_write(sm.st[(c + 1) % 3], nk, nx, ne);
      __syncthreads();
      // ---- E1n = (En2 W2^T) (.) G ----
      bf16x8 aE[NKD];
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks)
        aE[ks] = cat(lds4(&sm.E2[c16 * RS + 32 * ks + 4 * g]), lds4(&sm.E2[c16 * RS + 32 * ks + 16 + 4 * g]));
      bf16x4 e1[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        f4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks)
          acc = mfma32(aE[ks], cat(cvt4(mfma16(W2b[ht][2 * ks], I4, zero4())),
                                   cvt4(mfma16(W2b[ht][2 * ks + 1], I4, zero4()))), acc);
        e1[ht] = cvt4(acc * gk[ht]);
      }
      // ---- hand chunk c to the consumer: slot c % RINGD must have been read (chunk c - RINGD) ----
      if (c >= RINGD) cnt_wait(kCntRead + s, static_cast<unsigned>(c - RINGD + 1));
      const int base = (c % RINGD) * SLOT_BYTES;
      ring_st(base + SLOT_E1 + (w * 64 + lane) * 16, cat(e1[0], e1[1]));
      ring_st(base + SLOT_AK + (w * 64 + lane) * 16, cat(akR[0], akR[1]));
      ring_st(base + SLOT_E2 + (w * 64 + lane) * 16,
              *reinterpret_cast<const bf16x8*>(&sm.E2[(4 * w + g) * RS + 8 * c16]));
      // ---- chunk-end update of this wave's fp32 weights ----
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x4 be = mfma::tgroup(sm.E2, RS, dt, g, c16);
        const bf16x4 kt = mfma::tgroup(St.K, RS, dt, g, c16);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          W1c[dt][ht] = mfma16(kt, e1[ht], W1c[dt][ht]);
          W2c[ht][dt] = mfma16(akR[ht], be, W2c[ht][dt]);
        }
      }
      // publish chunk c once this wave's slot stores have completed
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (lane == 0) cnt_st(kCntReady + 4 * s + w, c1);
      // the E2 rows and the staged K of this chunk are read above; the next chunk overwrites
      // E2 only after its first barrier
    }
    if (p.wt_1)
      w_store(p.wt_1 + static_cast<size_t>(bh) * D * HID, p.wt_2 + static_cast<size_t>(bh) * HID * D,
              g, c16, hb, W1c, W2c);
    return;
  }

  // ===================================== consumer =====================================
  float ownQ[DPL];  // this part's Z^Q partial of the chunk whose output is still to be written
  // output z = Q + LN(Z^Q) of chunk cc for this part's tokens (wave s: tokens 4 s .. 4 s + 3)
  auto ln_out = [&](int cc) {
    const Stage& So = sm.st[cc % 3];
    const int t = ln_t;
    float z[DPL];
    total(true, cc & 1, static_cast<unsigned>(cc) + 1u, ownQ, z);
    float mu, rs;
    ln_stats8(z, mu, rs);
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
  for (int c = 0; c < nchunks; ++c) {
    Stage& St = sm.st[c % 3];
    const unsigned c1 = static_cast<unsigned>(c) + 1u;
    const int slot = c & 1;
    const bool has_next = c + 1 < nchunks;
    // ---- this wave's part of slot c: E1n and A^K of its units, En2 rows 4 w .. 4 w + 3 ----
    cnt_wait(kCntReady + 4 * s + w, c1);
    const int base = (c % RINGD) * SLOT_BYTES;
    const bf16x8 e1v = ring_ld(base + SLOT_E1 + (w * 64 + lane) * 16);
    const bf16x8 akv = ring_ld(base + SLOT_AK + (w * 64 + lane) * 16);
    const bf16x8 e2v = ring_ld(base + SLOT_E2 + (w * 64 + lane) * 16);
    *reinterpret_cast<bf16x8*>(&sm.E2[(4 * w + g) * RS + 8 * c16]) = e2v;
    const bf16x4 e1[NHT] = {mfma::lo4(e1v), mfma::hi4(e1v)};
    const bf16x4 akR[NHT] = {mfma::lo4(akv), mfma::hi4(akv)};
    // the output of chunk c - 1 (its Z^Q partials were published at the end of chunk c - 1)
    if (!m.local) wait_all(m, 8, s, static_cast<unsigned>(c), p.status);
    if (c > 0 && w == s) ln_out(c - 1);
    // every wave's slot loads have returned before the slot is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) cnt_st(kCntRead + s, c1);
    uint4 nk{}, nx{};
    float ne = 0.f;
    if (has_next) gload(c + 1, nk, nx, ne);
    bf16x8 aK[NKD], aQ[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      aK[ks] = cat(lds4(&St.K[c16 * RS + 32 * ks + 4 * g]), lds4(&St.K[c16 * RS + 32 * ks + 16 + 4 * g]));
      aQ[ks] = cat(lds4(&St.Q[c16 * RS + 32 * ks + 4 * g]), lds4(&St.Q[c16 * RS + 32 * ks + 16 + 4 * g]));
    }
    bf16x4 W1b[NDT][NHT], W2b[NHT][NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        W1b[dt][ht] = cvt4(W1c[dt][ht]);
        W2b[ht][dt] = cvt4(W2c[ht][dt]);
      }
    // ---- H^Q = Q W1 + tril(Q K^T) E1n, A^Q; Z^Q = A^Q W2 + tril(A^Q A^K^T) En2 (partial) ----
    f4 s1t = zero4();  // C[s][t] = K_s . Q_t
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) s1t = mfma32(aK[ks], aQ[ks], s1t);
    f4 s1m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s1m[r] = (4 * g + r) <= c16 ? s1t[r] : 0.f;
    const bf16x4 s1a = cvt4(s1m);
    bf16x4 akT[NHT], aqT[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 accq = zero4();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) accq = mfma32(aQ[ks], cat(W1b[2 * ks][ht], W1b[2 * ks + 1][ht]), accq);
      const f4 h = mfma16(s1a, e1[ht], accq);
      f4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = mfma::act<GELU_KIND>(h[r]);
      aqT[ht] = cvt4(mfma16(cvt4(a), I4, zero4()));
      akT[ht] = cvt4(mfma16(akR[ht], I4, zero4()));
    }
    const f4 s2t = mfma32(cat(akT[0], akT[1]), cat(aqT[0], aqT[1]), zero4());  // C[s][t] = A^K_s . A^Q_t
    f4 s2m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s2m[r] = (4 * g + r) <= c16 ? s2t[r] : 0.f;
    const bf16x4 s2a = cvt4(s2m);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x4 be = mfma::tgroup(sm.E2, RS, dt, g, c16);
      f4 acc = mfma32(cat(aqT[0], aqT[1]), cat(W2b[0][dt], W2b[1][dt]), zero4());
      acc = mfma16(s2a, be, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[1][w][dt][r][prot(r, lane)] = acc[r];
      // the same chunk-end update as the producer's, from the same bf16 operands
      const bf16x4 kt = mfma::tgroup(St.K, RS, dt, g, c16);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        W1c[dt][ht] = mfma16(kt, e1[ht], W1c[dt][ht]);
        W2c[ht][dt] = mfma16(akR[ht], be, W2c[ht][dt]);
      }
    }
    if (has_next) stage_write(sm.st[(c + 1) % 3], nk, nx, ne);
    __syncthreads();
    // ---- publish this part's Z^Q partial of chunk c (its output is written next chunk) ----
    put_own(true, slot, c1, ownQ);
    if (!m.local) publish(m, 8, s, c1);
  }
  if (!m.local) wait_all(m, 8, s, static_cast<unsigned>(nchunks), p.status);
  if (w == s) ln_out(nchunks - 1);
}

// Clears the exchange areas (their tags) and the counter words of every head.
__global__ void split_reset_kernel(uint4* w, size_t n4) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    w[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

bool fwd_split_supported(const ScanParams& p) {
  return p.kind == TTT_MLP && p.d == D && p.hid == HID && p.chunk == BC && p.io == TTT_BF16;
}

// Workspace: the exchange areas of every head, then their counter words, then the hand-off
// rings of the producer/consumer form.
size_t fwd_split_workspace_bytes(int nheads) {
  return static_cast<size_t>(nheads) * (kHeadXFloats * sizeof(float) + kFlagWords * sizeof(unsigned) + kRingBytes);
}

// Workgroups per head of the two forms.
constexpr int kBlocksOne = S;       // every workgroup runs both sides
constexpr int kBlocksPair = 2 * S;  // producers and consumers

// Resident workgroups of a form's kernel on the current device (0 when it cannot launch
// cooperatively). The workgroups of a head wait for each other, so one launch may hold at most
// this many. Cached per device ordinal and form.
static int split_capacity(bool paired) {
  constexpr int kMaxDev = 64;
  static int cap[2][kMaxDev];  // 0 = unknown, else 1 + resident workgroups on the device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int& c = cap[paired ? 1 : 0][dev];
  if (c == 0) {
    int coop = 0, ncu = 0, per_cu = 0;
    const void* fn = paired ? reinterpret_cast<const void*>(fwd_split_pair_kernel<TTT_GELU_ERF>)
                            : reinterpret_cast<const void*>(fwd_split_kernel<TTT_GELU_ERF>);
    const bool ok =
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, 0) == hipSuccess;
    c = 1 + ((ok && coop) ? ncu * per_cu : 0);
  }
  return c - 1;
}

// Heads per launch of a form: whole groups of eight heads whose workgroups all fit at once.
static int split_heads_per_launch(bool paired) {
  return split_capacity(paired) / (8 * (paired ? kBlocksPair : kBlocksOne)) * 8;
}

// The producer/consumer form when all heads fit in one of its launches (32 heads on 256 CUs);
// above that the form with both sides in every workgroup, whose launches hold twice as many
// heads, needs fewer launches and finishes first.
static bool split_paired(int nheads) { return nheads <= split_heads_per_launch(true); }

// Whether the split kernel can run at all here (at least one group of eight heads fits).
bool fwd_split_fits(int) { return split_heads_per_launch(false) > 0; }

hipError_t launch_fwd_mfma_split(const ScanParams& p, hipStream_t stream) {
  const int nheads = p.B * p.H;
  const bool paired = split_paired(nheads);
  const int per = split_heads_per_launch(paired);
  if (per <= 0) return hipErrorCooperativeLaunchTooLarge;
  Split x;
  x.xbuf = p.wbuf;
  x.flags = reinterpret_cast<unsigned*>(p.wbuf + static_cast<size_t>(nheads) * kHeadXFloats);
  x.ring = reinterpret_cast<char*>(x.flags + static_cast<size_t>(nheads) * kFlagWords);
  x.nheads = nheads;
  const size_t n4 = static_cast<size_t>(nheads) * (kHeadXFloats + kFlagWords) / 4;
  const unsigned rblocks = static_cast<unsigned>(n4 / 256 + 1 < 2048 ? n4 / 256 + 1 : 2048);
  hipLaunchKernelGGL(split_reset_kernel, dim3(rblocks), dim3(256), 0, stream, reinterpret_cast<uint4*>(p.wbuf), n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* fn =
      paired ? (p.gelu == TTT_GELU_TANH ? reinterpret_cast<const void*>(fwd_split_pair_kernel<TTT_GELU_TANH>)
                                        : reinterpret_cast<const void*>(fwd_split_pair_kernel<TTT_GELU_ERF>))
             : (p.gelu == TTT_GELU_TANH ? reinterpret_cast<const void*>(fwd_split_kernel<TTT_GELU_TANH>)
                                        : reinterpret_cast<const void*>(fwd_split_kernel<TTT_GELU_ERF>));
  // heads are independent: launch them in groups the device holds at once, in order
  for (int h0 = 0; h0 < nheads; h0 += per) {
    ScanParams pc = p;
    x.head0 = h0;
    void* args[] = {&pc, &x};
    const int n = nheads - h0 < per ? nheads - h0 : per;
    const int blocks = (n + 7) / 8 * 8 * (paired ? kBlocksPair : kBlocksOne);
    e = hipLaunchCooperativeKernel(fn, dim3(blocks), dim3(NT), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ttt
