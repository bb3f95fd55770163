// Decode step for the TTT-MLP head shape d = 64, hidden = 256 with every head spread over
// four workgroups: one token per (batch, head), the mini-batch rule of decoding in "LLM : 빠른
// 논문 리뷰 : End-to-End Test-Time Training for Long Context", section 2.3.2 (the gradient
// step is taken only when the decoded tokens fill a mini-batch), on the layer of "Test-Time
// Training(TTT)과 LLM 메모리", section "TTT layer", Eq. 2/4/5.
//
// The step is bound by HBM traffic: per head it reads W_start and acc (256 KiB) and writes acc
// (or W_start at the chunk's last token). With one workgroup per head a call of 96 heads pulls
// 24 MiB through 96 CUs; here part s of a head owns hidden units 64 s .. 64 s + 63 (its
// columns of W1 and acc1, its rows of W2 and acc2: 64 KiB), so four times as many CUs load.
// Everything per hidden unit is local to a part:
//   HK = k W1, AK = GELU, G = GELU';  E1 = (E2 W2^T) (.) G;  acc1 += k^T E1;  acc2 += AK^T E2;
//   HQ = q (W1 - acc1), AQ = GELU
// and the two sums over hidden units are formed from the parts' [64] partials:
//   ZK = sum_s AK_s W2_s  (every part needs it: E2 = eta' LN-backward(ZK))
//   ZQ = sum_s AQ_s (W2 - acc2)_s  (only part 0 needs it: z = q + LN(ZQ))
// All parts add the partials in the same order, so they compute the same E2. HQ is formed as
// q (W1 - acc1_before) - (q . k) E1, so its reduction runs before E1 is known, and acc2 and
// acc1 are stored as soon as they are final.
//
// The four parts of a head are numbered 8 blocks apart, so that the hardware's round-robin
// placement puts them on one XCD; they check it at start (HW_REG_XCC_ID). On one XCD each
// partial element travels as a (value, 1) pair in one 8-byte store and the reader polls the
// pair in that XCD's L2 until its tag is 1. Across XCDs (or with TTT_FORCE_DEVICE_SCOPE) the
// parts publish counters with device-scope release/acquire fences. Part 0 is the last to use
// the exchange area of its head (it waits for every other part's ZQ partial, which each part
// sends after it has read all it needs), and it clears the area's tags and counters before it
// ends, so every call finds them zero, as in a zero-filled workspace. Waits are bounded; an
// expired wait sets the timeout bit of the status word (the area must then be zero-filled
// again).
#include "ttt_device.hpp"

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int HID = 256;
constexpr int SP = 4;             // workgroups (parts) per head
constexpr int NT = 256;           // threads per workgroup
constexpr int NWV = NT / 64;      // waves per workgroup
constexpr int HP = HID / SP;      // hidden units per part
constexpr int kSpinLimit = 1 << 20;
constexpr unsigned kBufFlags = 0x00020000u;
constexpr int kLoadL2 = 16;       // exchange loads on one XCD: device scope (sc1), L1 skipped
static_assert(HP == 64 && NWV * 16 == D, "part shape");

// Exchange words per head: XCD ids (one 8-byte word per part: xcc + 1 | 1 << 32), the
// device-scope counters (Z^K at kXCnt + s, Z^Q at kXCnt + 8 + s), then the Z^K and Z^Q
// partials, SP x 64 (value, tag) pairs each.
constexpr int kXIds = 0;
constexpr int kXCnt = 16;
constexpr int kXZk = 64;
constexpr int kXZq = kXZk + SP * D * 2;
constexpr int kXWords = kXZq + SP * D * 2;
static_assert((kXWords * 4) % 256 == 0, "exchange area alignment");

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int GELU_KIND>
__device__ __forceinline__ void act_dv(float x, float& v, float& d1) {
  if (GELU_KIND == TTT_GELU_ERF)
    ttt_gelu::gelu_d(x, v, d1);
  else
    gelu_d(x, GELU_KIND, v, d1);
}

__device__ __forceinline__ float4 sub4(float4 a, float4 b) {
  return float4{a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w};
}

__device__ __forceinline__ void fma4(float x, float4 m, float4& acc) {
  acc.x = fmaf(x, m.x, acc.x);
  acc.y = fmaf(x, m.y, acc.y);
  acc.z = fmaf(x, m.z, acc.z);
  acc.w = fmaf(x, m.w, acc.w);
}

// sum over the four lanes 16 apart (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float4 sum_rows4(float4 z) {
#pragma unroll
  for (int m = 16; m <= 32; m <<= 1) {
    z.x += __shfl_xor(z.x, m, 64);
    z.y += __shfl_xor(z.y, m, 64);
    z.z += __shfl_xor(z.z, m, 64);
    z.w += __shfl_xor(z.w, m, 64);
  }
  return z;
}

struct XArea {
  unsigned* w;                 // the head's exchange words
  __amdgpu_buffer_rsrc_t r;    // the same, as a buffer
  bool local;
};

__device__ __forceinline__ bool status_timed_out(unsigned* status) {
  return (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout) != 0;
}

// Part s publishes its partial `own` (element `lane` of area `area`, counter word `cnt`).
// Wave 0 only.
__device__ __forceinline__ void publish(const XArea& x, int area, int cnt, int s, int lane, float own) {
  const int off = area + 2 * (s * D + lane);
  if (x.local) {
    const u32x2 pv = {__float_as_uint(own), 1u};
    __builtin_amdgcn_raw_buffer_store_b64(pv, x.r, 4 * off, 0, 0);
  } else {
    reinterpret_cast<float*>(x.w)[off] = own;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) __hip_atomic_store(x.w + cnt + s, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The head's total of an area: the partials of every part but `s` are read (polled until
// published, bounded), own is this part's, and the sum runs in part order. Wave 0 only.
__device__ __forceinline__ float gather(const XArea& x, int area, int cnt, int s, int lane, float own,
                                        unsigned* status) {
  float v[SP];
  if (x.local) {
    for (int it = 0;; ++it) {
      bool all = true;
#pragma unroll
      for (int o = 0; o < SP; ++o) {
        if (o == s) continue;
        const u32x2 pv = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(x.r, 4 * (area + 2 * (o * D + lane)), 0, kLoadL2));
        v[o] = __uint_as_float(pv[0]);
        all = all && pv[1] == 1u;
      }
      if (all) break;
      if (it + 1 >= kSpinLimit) {
        atomicOr(status, kStatusTimeout);
        break;
      }
      if ((it & 63) == 63 && status_timed_out(status)) break;
      __builtin_amdgcn_s_sleep(1);
    }
  } else {
    if (lane == 0) {
      bool late = status_timed_out(status);
      for (int o = 0; o < SP && !late; ++o) {
        if (o == s) continue;
        int it = 0;
        while (__hip_atomic_load(x.w + cnt + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 1u) {
          if (++it >= kSpinLimit) {
            late = true;
            atomicOr(status, kStatusTimeout);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
    for (int o = 0; o < SP; ++o)
      if (o != s) v[o] = __hip_atomic_load(reinterpret_cast<float*>(x.w) + area + 2 * (o * D + lane),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  v[s] = own;
  float t = v[0];
#pragma unroll
  for (int o = 1; o < SP; ++o) t += v[o];
  return t;
}

template <typename IO, int GELU_KIND>
__global__ void __launch_bounds__(NT) decode_split_kernel(DecodeParams p, unsigned* xbuf, int nheads) {
  __shared__ float sq[D], sk[D], sv[D], sE2[D];
  __shared__ float sA[HP], sG[HP], sE1[HP], sPQ[HP], sAQ[HP];
  __shared__ float4 red1[NWV][HP / 4];  // [wave][hidden/4]: k W1 partials
  __shared__ float4 redq[NWV][HP / 4];  // [wave][hidden/4]: q (W1 - acc1) partials (acc1 before this token)
  __shared__ float4 red2[NWV][D / 4];   // [wave][d/4]: A W2 partials
  __shared__ float sEta, sQK;
  __shared__ unsigned sh_local;
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
  TTT_POISON(sh_local);
  TTT_POISON_DONE();
  // block -> (head, part): the parts of a head are 8 blocks apart (same XCD)
  const int blk = blockIdx.x;
  const int s = (blk >> 3) % SP;
  const int bh = ((blk >> 3) / SP) * 8 + (blk & 7);
  if (bh >= nheads) return;  // all parts of a missing head leave together
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hidx = bh % p.H;
  const bool commit = p.pos == p.chunk - 1;

  // W1 / acc1 of this part: thread holds columns 64 s + 4 c1 .. + 3 of rows 16 wv + 4 r1 + i
  const int c1 = lane & 15, r1 = lane >> 4;
  const size_t head1 = static_cast<size_t>(bh) * D * HID + HP * s + 4 * c1;
  float* W1 = p.ws_1 + head1;
  float* A1 = p.acc_1 + head1;
  // W2 / acc2 of this part: thread holds rows 64 s + 4 rb + i, columns 4 cg .. 4 cg + 3
  const int cg = tid & 15, rb = tid >> 4;
  const size_t head2 = static_cast<size_t>(bh) * HID * D + static_cast<size_t>(HP * s) * D + 4 * cg;
  float* W2 = p.ws_2 + head2;
  float* A2 = p.acc_2 + head2;
  // loads in the order of first use (W1, W2, acc1, acc2)
  float4 w1[4], a1[4], w2[4], a2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w1[i] = *reinterpret_cast<const float4*>(W1 + (16 * wv + 4 * r1 + i) * HID);
#pragma unroll
  for (int i = 0; i < 4; ++i) w2[i] = *reinterpret_cast<const float4*>(W2 + (4 * rb + i) * D);
#pragma unroll
  for (int i = 0; i < 4; ++i) a1[i] = *reinterpret_cast<const float4*>(A1 + (16 * wv + 4 * r1 + i) * HID);
#pragma unroll
  for (int i = 0; i < 4; ++i) a2[i] = *reinterpret_cast<const float4*>(A2 + (4 * rb + i) * D);
  if (tid < D) {
    const size_t o = static_cast<size_t>(bh) * D + tid;
    sq[tid] = to_f32(static_cast<const IO*>(p.q)[o]);
    sk[tid] = to_f32(static_cast<const IO*>(p.k)[o]);
    sv[tid] = to_f32(static_cast<const IO*>(p.v)[o]);
  }
  if (tid == 0) sEta = p.eta[bh] * p.eta_scale;

  XArea x;
  x.w = xbuf + static_cast<size_t>(bh) * kXWords;
  x.r = __builtin_amdgcn_make_buffer_rsrc(x.w, 0, kXWords * 4, kBufFlags);
  {
    // placement: every part publishes its XCD id + 1 (device scope) and reads the others'
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (tid == 0) {
      uint64_t* ids = reinterpret_cast<uint64_t*>(x.w + kXIds);
      __hip_atomic_store(ids + s, (static_cast<uint64_t>(1) << 32) | (xcc + 1), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      bool same = true;
      for (int o = 0; o < SP; ++o) {
        uint64_t v = 0;
        for (int it = 0; it < kSpinLimit && (v >> 32) != 1u; ++it) {
          v = __hip_atomic_load(ids + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((v >> 32) != 1u) __builtin_amdgcn_s_sleep(1);
        }
        if ((v >> 32) != 1u) atomicOr(p.status, kStatusTimeout);
        same = same && static_cast<unsigned>(v) == xcc + 1;
      }
      sh_local = same && !(p.flags & TTT_FORCE_DEVICE_SCOPE) ? 1u : 0u;
    }
  }
  __syncthreads();
  x.local = sh_local != 0;

  // ---- H^K = k W1 for this part's hidden units ----
  {
    float4 h = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) fma4(sk[16 * wv + 4 * r1 + i], w1[i], h);
    h = sum_rows4(h);
    if (lane < 16) red1[wv][c1] = h;
  }
  __syncthreads();
  if (tid < HP) {
    const float* r = reinterpret_cast<const float*>(red1);
    float hs = r[tid];
#pragma unroll
    for (int w = 1; w < NWV; ++w) hs += r[w * HP + tid];
    float v, d1;
    act_dv<GELU_KIND>(hs, v, d1);
    sA[tid] = v;
    sG[tid] = d1;
  } else if (wv == 1) {
    const float qk = wave_sum(sq[lane] * sk[lane]);
    if (lane == 0) sQK = qk;
  }
  __syncthreads();

  // partial of x W2 (or x (W2 - acc2)) over this thread's four hidden rows, summed over the
  // wave's 16 rows, then (wave 0, one d per lane) over the waves
  auto w2_partial = [&](const float* xs, bool minus_acc) {
    float4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) fma4(xs[4 * rb + i], minus_acc ? sub4(w2[i], a2[i]) : w2[i], z);
    z = sum_rows4(z);
    if (lane < 16) red2[wv][cg] = z;
  };
  auto own_partial = [&]() {
    const float* r = reinterpret_cast<const float*>(red2);
    float z = r[lane];
#pragma unroll
    for (int w = 1; w < NWV; ++w) z += r[w * D + lane];
    return z;
  };

  // ---- this part's Z^K partial; the part of H^Q that does not depend on this token's
  //      gradient: q (W1 - acc1), acc1 before this token (H^Q = that - (q . k) E1) ----
  w2_partial(sA, false);
  {
    float4 h = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) fma4(sq[16 * wv + 4 * r1 + i], sub4(w1[i], a1[i]), h);
    h = sum_rows4(h);
    if (lane < 16) redq[wv][c1] = h;
  }
  __syncthreads();
  // ---- Z^K over all parts; LayerNorm forward/backward: E2 = eta' delta2 (wave 0); meanwhile
  //      wave 1 sums the q (W1 - acc1) partials ----
  if (wv == 0) {
    const float own = own_partial();
    publish(x, kXZk, kXCnt, s, lane, own);
    const float z = gather(x, kXZk, kXCnt, s, lane, own, p.status);
    const float mu = wave_sum(z) * (1.0f / D);
    const float c = z - mu;
    const float rs = 1.0f / sqrtf(wave_sum(c * c) * (1.0f / D) + p.eps);
    const float xh = c * rs;
    const float gam = p.gamma[hidx * D + lane], bet = p.beta[hidx * D + lane];
    const float res = sk[lane] + gam * xh + bet - sv[lane];
    const float gg = 2.f * res * gam;
    const float mg = wave_sum(gg) * (1.0f / D), mgx = wave_sum(gg * xh) * (1.0f / D);
    sE2[lane] = sEta * (gg - mg - xh * mgx) * rs;
    if (s == 0) {
      const float loss = wave_sum(res * res);
      if (lane == 0) flag_nonfinite(p.status, loss);
    }
  } else if (wv == 1) {
    const float* r = reinterpret_cast<const float*>(redq);
    float hs = r[lane];
#pragma unroll
    for (int w = 1; w < NWV; ++w) hs += r[w * HP + lane];
    sPQ[lane] = hs;
  }
  __syncthreads();

  // ---- E1 = (E2 W2^T) (.) G for this thread's four hidden rows; acc2 += A^K^T E2 (stored
  //      now: nothing after this changes it) ----
  {
    const float4 e = reinterpret_cast<const float4*>(sE2)[cg];
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float u = w2[i].x * e.x;
      u = fmaf(w2[i].y, e.y, u);
      u = fmaf(w2[i].z, e.z, u);
      t[i] = fmaf(w2[i].w, e.w, u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // sum over the 16 lanes holding the columns of these rows (aligned lane groups)
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) t[i] += __shfl_xor(t[i], m, 64);
    }
    if (cg == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sE1[4 * rb + i] = t[i] * sG[4 * rb + i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fma4(sA[4 * rb + i], e, a2[i]);
      const size_t o2 = static_cast<size_t>(4 * rb + i) * D;
      if (commit) {
        *reinterpret_cast<float4*>(W2 + o2) = sub4(w2[i], a2[i]);
        *reinterpret_cast<float4*>(A2 + o2) = float4{0.f, 0.f, 0.f, 0.f};
      } else {
        *reinterpret_cast<float4*>(A2 + o2) = a2[i];
      }
    }
  }
  __syncthreads();

  // ---- H^Q = q (W1 - acc1) - (q . k) E1, A^Q = GELU;  acc1 += k^T E1 (stored) ----
  if (tid < HP) {
    const float hq = fmaf(-sQK, sE1[tid], sPQ[tid]);
    sAQ[tid] = GELU_KIND == TTT_GELU_ERF ? ttt_gelu::gelu(hq) : gelu(hq, GELU_KIND);
  }
  {
    const float4 e1 = reinterpret_cast<const float4*>(sE1)[c1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fma4(sk[16 * wv + 4 * r1 + i], e1, a1[i]);
      const size_t o1 = static_cast<size_t>(16 * wv + 4 * r1 + i) * HID;
      if (commit) {
        *reinterpret_cast<float4*>(W1 + o1) = sub4(w1[i], a1[i]);
        *reinterpret_cast<float4*>(A1 + o1) = float4{0.f, 0.f, 0.f, 0.f};
      } else {
        *reinterpret_cast<float4*>(A1 + o1) = a1[i];
      }
    }
  }
  __syncthreads();

  // ---- Z^Q = A^Q (W2 - acc2) over all parts (gathered by part 0); z = q + LN(Z^Q) ----
  w2_partial(sAQ, true);
  __syncthreads();
  if (wv != 0) return;
  const float own = own_partial();
  if (s != 0) {
    publish(x, kXZq, kXCnt + 8, s, lane, own);
    return;
  }
  const float z = gather(x, kXZq, kXCnt + 8, 0, lane, own, p.status);
  const float mu = wave_sum(z) * (1.0f / D);
  const float c = z - mu;
  const float rs = 1.0f / sqrtf(wave_sum(c * c) * (1.0f / D) + p.eps);
  const float o = sq[lane] + p.gamma[hidx * D + lane] * c * rs + p.beta[hidx * D + lane];
  static_cast<IO*>(p.z)[static_cast<size_t>(bh) * D + lane] = from_f32<IO>(o);
  const float chk = wave_sum(o);
  if (lane == 0) flag_nonfinite(p.status, chk);
  // every other part has read all it needs from the area (it sent its Z^Q partial after
  // reading the Z^K partials and the ids): clear the tags and counters for the next call
  const u32x2 zero2 = {0u, 0u};
#pragma unroll
  for (int q = 0; q < SP; ++q) {
    __builtin_amdgcn_raw_buffer_store_b64(zero2, x.r, 4 * (kXZk + 2 * (q * D + lane)), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b64(zero2, x.r, 4 * (kXZq + 2 * (q * D + lane)), 0, 0);
  }
  if (lane < kXZk) __builtin_amdgcn_raw_buffer_store_b32(0u, x.r, 4 * lane, 0, 0);
}

}  // namespace

bool decode_split_supported(const DecodeParams& p) {
  return p.kind == TTT_MLP && p.d == D && p.hid == HID;
}

size_t decode_split_workspace_bytes(int heads) {
  return static_cast<size_t>((heads + 7) / 8) * 8 * kXWords * sizeof(unsigned);
}

// Progress needs only the 32 blocks of one group of eight heads resident at once: blocks are
// dispatched in order, and a head's parts wait only for each other.
hipError_t launch_decode_split(const DecodeParams& p, void* xbuf, hipStream_t stream) {
  const int nheads = p.B * p.H;
  const dim3 grid(((nheads + 7) / 8) * 8 * SP), block(NT);
  unsigned* xw = static_cast<unsigned*>(xbuf);
  const bool tanh_form = p.gelu == TTT_GELU_TANH;
  if (p.io == TTT_BF16) {
    if (tanh_form)
      hipLaunchKernelGGL((decode_split_kernel<bf16_t, TTT_GELU_TANH>), grid, block, 0, stream, p, xw, nheads);
    else
      hipLaunchKernelGGL((decode_split_kernel<bf16_t, TTT_GELU_ERF>), grid, block, 0, stream, p, xw, nheads);
  } else {
    if (tanh_form)
      hipLaunchKernelGGL((decode_split_kernel<float, TTT_GELU_TANH>), grid, block, 0, stream, p, xw, nheads);
    else
      hipLaunchKernelGGL((decode_split_kernel<float, TTT_GELU_ERF>), grid, block, 0, stream, p, xw, nheads);
  }
  return hipGetLastError();
}

}  // namespace ttt
