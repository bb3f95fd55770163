// Forward scan for the TTT-MLP head shape d = 64, hidden = 256, chunk 16, bf16 I/O, fp32
// fast weights, on TWO workgroups (two compute units) per (batch, head):
//   producer: the chain that carries the weights from chunk to chunk -- H^K = K W1,
//             A^K = GELU, G = GELU', Z^K = A^K W2, the LayerNorm forward/backward of Z^K
//             (En2 = -eta * delta2), E1n = (En2 W2^T) (.) G, then W1 += K^T E1n and
//             W2 += A^K^T En2. It hands E1n, A^K and En2 of every chunk to its partner.
//   consumer: replays the same weight update from the same bf16 operands (so its fp32
//             weights stay bitwise equal to the producer's) and computes the query side of
//             the dual form: H^Q = Q W1 + tril(Q K^T) E1n, A^Q = GELU(H^Q),
//             Z^Q = A^Q W2 + tril(A^Q A^K^T) En2, z = Q + LN(Z^Q).
// Nothing flows from the consumer to the producer except "slot consumed" counters, so the
// query side is off the chunk-to-chunk critical path. (Dual form of the per-token rule on
// the page "Test-Time Training(TTT)과 LLM 메모리", section "TTT layer", Eq. 2/4/5;
// mini-batch rule of the E2E paper review, section 2.3, Eq. 5.)
//
// The producer's chain is shortened by a look-ahead: with W1(c+1) = W1(c) + K(c)^T E1n(c),
//   H^K(c+1) = K(c+1) W1(c) + (K(c+1) K(c)^T) E1n(c),
// and K(c+1) W1(c) is computed while chunk c is in flight. Between E1n(c) and H^K(c+1) there
// is then one K = 16 product; the fp32 weight update of chunk c is applied at the start of
// chunk c + 1, next to the GELU work, where it is off the chain. (The same identity is the
// dual form's own: the look-ahead term is the next chunk's first dual-form correction.)
//
// Hand-off: a ring of RING chunk slots per head in the workspace, per-wave counters
// ready[w] (chunks published by producer wave w) and one counter of chunks the consumer
// workgroup is done reading (raised by its wave 0 after the barrier that follows the slot
// loads of every wave). A producer wave waits for its slot stores to complete (s_waitcnt vmcnt)
// before it raises its counter, and a consumer wave issues its slot loads only after it has
// seen the counter. Workgroups b and b + 8 of each group of 16 form a pair; workgroups are
// dealt to the 8 XCDs round-robin, so both normally sit on one XCD. Each side reads its XCD
// id at start and the two compare them through device-coherent atomics: on one XCD the
// hand-off meets in the shared L2 (plain stores through the write-through L1, device-scope
// loads that skip the L1); otherwise every hand-off access is an agent-scope atomic.
//
// Every wait is bounded. On expiry the status word gets kStatusTimeout, later waits return
// at once, and the kernel runs to completion with meaningless outputs. The launch is
// cooperative, so the two workgroups of a pair are always co-resident.
//
// Mini-batches larger than 16 tokens (b = 16 m, up to 1024): the kernel still walks the
// sequence in 16-token sub-tiles, and the consumer is unchanged (its running weights are the
// mini-batch start plus the updates of the sub-tiles before, so its query side is the dual
// form of the whole mini-batch evaluated block by block: the tril products inside a sub-tile,
// the earlier sub-tiles through the running weights). The producer takes every gradient of
// the mini-batch at the weights the mini-batch started from, so its bf16 weight copies, their
// transposes and the look-ahead correction are made once per mini-batch instead of once per
// sub-tile; the fp32 weights still take each sub-tile's update in order, bit for bit as in
// the consumer.
//
// Key-side output rule (Eq. 9 of the E2E paper review, section 2.4.2: z_t = f(K_t; W at the
// mini-batch start), 16-token mini-batches): the output is K + LN(Z^K), which the producer's
// LayerNorm lanes already hold, so a separate kernel runs the producer alone, one workgroup
// per head, and writes it there; no consumer, no hand-off.
#include "ttt_mfma_common.hpp"

namespace ttt {

#ifdef TTT_PHASE_CLOCKS
// Opt-in timing build (test_weight_sequence_amd/phase_clocks.py builds it into a separate
// library; the product library is compiled without it): shader-clock stamps at the phase
// boundaries of each chunk of head 0, summed per wave over chunks 16 .. end.
// [side: producer, consumer][wave][slot]: slots 0..7 phase sums, 8 chunk count, 9 last stamp,
// 10 first counted stamp.
__device__ unsigned long long g_phase_clocks[2][8][16];
#define TTT_STAMP(var)        \
  unsigned long long var;     \
  asm volatile("s_memtime %0\n s_waitcnt lgkmcnt(0)" : "=s"(var)::"memory")
#define TTT_DEP(x) asm volatile("" ::"v"(x))
#else
#define TTT_STAMP(var)
#define TTT_DEP(x)
#endif

namespace {

using namespace mfma;

constexpr int NW = 8;                  // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int HS = HID / NW;           // hidden units per wave (32)
constexpr int NHT = HS / 16;           // h tiles per wave (2)
constexpr int RING = 6;                // chunk slots per head
// slot layout (bytes): E1n and A^K of wave w as one 16-byte (two-tile) operand per lane,
// then En2 as four 8-byte (k = token, n = d) operands per lane
constexpr int SLOT_E1 = 0;
constexpr int SLOT_AK = NW * 64 * 16;
constexpr int SLOT_E2 = 2 * NW * 64 * 16;
constexpr int SLOT_BYTES = SLOT_E2 + 64 * 32;
constexpr int FLAG_WORDS = 32;         // per head: ready[0..7], consumed[16], XCD ids
constexpr int FLAG_XCC = 24;           // producer's and consumer's XCD id + 1 (words 24, 25)
constexpr int kSpinLimit = 1 << 20;
static_assert(NHT == 2, "layout assumes 8 waves of 32 hidden units");

struct Pair {
  unsigned* flags;  // [head][FLAG_WORDS]
  char* ring;       // [head][RING][SLOT_BYTES]
  int nheads;
};

struct PStage {
  alignas(16) __bf16 K[BC * RS];
  alignas(16) __bf16 X[BC * RS];  // V (producer) or Q (consumer)
  alignas(16) float eta[BC];
};
struct ProdSmem {
  PStage st[4];   // chunk j in slot j & 3
  float red[NW][NDT][4][PS];
  alignas(16) __bf16 E2[BC * RS];  // En2 [token][d]
  alignas(16) __bf16 zeros[8];
};
struct ConsSmem {
  PStage st[3];   // chunk j in slot j % 3
  float red[2][NW][NDT][4][PS];
  alignas(16) __bf16 zeros[8];
};
union SmemP {
  ProdSmem p;
  ConsSmem c;
};

// Cache policy of hand-off loads on one XCD: device scope (sc1), which skips the CU's L1
// (a plain or sc0 load may return a line the L1 still holds from an earlier read).
constexpr int kLoadL2 = 16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned long long u64;
typedef u64 u64x2 __attribute__((ext_vector_type(2)));

// Hand-off memory of one head: its counter words and its ring of chunk slots.
template <bool LOCAL>
struct HandOff {
  unsigned* flags;
  char* ring;
  __amdgpu_buffer_rsrc_t fr, rr;
  __device__ __forceinline__ HandOff(unsigned* f, char* r) : flags(f), ring(r) {
    fr = __builtin_amdgcn_make_buffer_rsrc(f, 0, FLAG_WORDS * 4, kBufFlags);
    rr = __builtin_amdgcn_make_buffer_rsrc(r, 0, RING * SLOT_BYTES, kBufFlags);
  }
  __device__ __forceinline__ unsigned ld(int i) const {
    if constexpr (LOCAL)
      return __builtin_amdgcn_raw_buffer_load_b32(fr, 0, 4 * i, kLoadL2);
    else
      return __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ void st(int i, unsigned v) const {
    if constexpr (LOCAL)
      __builtin_amdgcn_raw_buffer_store_b32(v, fr, 0, 4 * i, 0);
    else
      __hip_atomic_store(flags + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ bf16x8 ld16(int off) const {
    if constexpr (LOCAL) {
      return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, kLoadL2));
    } else {
      const u64* q = reinterpret_cast<const u64*>(ring + off);
      const u64x2 v = {__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                       __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
      return __builtin_bit_cast(bf16x8, v);
    }
  }
  __device__ __forceinline__ void st16(int off, bf16x8 v) const {
    if constexpr (LOCAL) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rr, off, 0, 0);
    } else {
      const u64x2 x = __builtin_bit_cast(u64x2, v);
      u64* q = reinterpret_cast<u64*>(ring + off);
      __hip_atomic_store(q, x[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(q + 1, x[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
};

// Wait until counter word i >= target, at most kSpinLimit polls; gives up at once once any
// wave of the launch has timed out.
template <bool LOCAL>
__device__ __forceinline__ void spin_geq(const HandOff<LOCAL>& h, int i, unsigned target, unsigned* status) {
  for (int it = 0; it < kSpinLimit; ++it) {
    if (h.ld(i) >= target) return;
    if ((it & 63) == 0 && (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout))
      return;
    __builtin_amdgcn_s_sleep(2);
  }
  atomicOr(status, kStatusTimeout);
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// One chunk's hand-off data as held by a consumer lane.
struct Slot {
  bf16x8 e1, ak;
  bf16x8 e2[2];  // En2 tiles (d tiles 0,1) and (2,3), each 4 values with k = token
};
template <bool LOCAL>
__device__ __forceinline__ void slot_load(const HandOff<LOCAL>& h, Slot& s, int chunk, int w, int lane) {
  const int base = (chunk % RING) * SLOT_BYTES;
  s.e1 = h.ld16(base + SLOT_E1 + (w * 64 + lane) * 16);
  s.ak = h.ld16(base + SLOT_AK + (w * 64 + lane) * 16);
  s.e2[0] = h.ld16(base + SLOT_E2 + lane * 32);
  s.e2[1] = h.ld16(base + SLOT_E2 + lane * 32 + 16);
}
__device__ __forceinline__ bf16x4 slot_e2(const Slot& s, int dt) { return dt & 1 ? hi4(s.e2[dt >> 1]) : lo4(s.e2[dt >> 1]); }
// A value that depends on every register of the slot: the compiler must wait for all its
// loads before computing it.
__device__ __forceinline__ unsigned slot_dep(const Slot& s) {
  const u64x2 a = __builtin_bit_cast(u64x2, s.e1), b = __builtin_bit_cast(u64x2, s.ak);
  const u64x2 c = __builtin_bit_cast(u64x2, s.e2[0]), d = __builtin_bit_cast(u64x2, s.e2[1]);
  const u64 x = a[0] ^ a[1] ^ b[0] ^ b[1] ^ c[0] ^ c[1] ^ d[0] ^ d[1];
  return static_cast<unsigned>(x) ^ static_cast<unsigned>(x >> 32);
}

// What the producer carries from chunk c - 1 into chunk c.
struct Carry {
  f4 P[NHT];       // K(c) W1(c-1) for this wave's h tiles
  bf16x4 sA;       // K(c) K(c-1)^T as an A operand (m = token of c, k = token of c-1)
  bf16x8 e1, ak;   // E1n(c-1), A^K(c-1): k = token (two h tiles)
};

// W1 += K^T E1n, W2 += A^K^T En2 from K^T / En2^T operands that hold two d tiles each
// (k01: d tiles 0 and 1 in the lower and upper half, k23: 2 and 3; likewise e01, e23) and
// E1n / A^K operands holding the two h tiles of the wave (e1, ak).
__device__ __forceinline__ void update_mfmas(f4 (&W1c)[NDT][NHT], f4 (&W2c)[NHT][NDT], bf16x8 k01, bf16x8 k23,
                                             bf16x8 e01, bf16x8 e23, bf16x8 e1, bf16x8 ak, bf16x4 zz) {
  const bf16x8 b_lo[NHT] = {cat(lo4(e1), zz), cat(hi4(e1), zz)};  // E1n of h tile ht, lower half
  const bf16x8 b_hi[NHT] = {cat(zz, lo4(e1)), cat(zz, hi4(e1))};  // upper half
  const bf16x8 a_lo[NHT] = {cat(lo4(ak), zz), cat(hi4(ak), zz)};  // A^K^T of h tile ht
  const bf16x8 a_hi[NHT] = {cat(zz, lo4(ak)), cat(zz, hi4(ak))};
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    W1c[0][ht] = mfma32(k01, b_lo[ht], W1c[0][ht]);
    W1c[1][ht] = mfma32(k01, b_hi[ht], W1c[1][ht]);
    W1c[2][ht] = mfma32(k23, b_lo[ht], W1c[2][ht]);
    W1c[3][ht] = mfma32(k23, b_hi[ht], W1c[3][ht]);
    W2c[ht][0] = mfma32(a_lo[ht], e01, W2c[ht][0]);
    W2c[ht][1] = mfma32(a_hi[ht], e01, W2c[ht][1]);
    W2c[ht][2] = mfma32(a_lo[ht], e23, W2c[ht][2]);
    W2c[ht][3] = mfma32(a_hi[ht], e23, W2c[ht][3]);
  }
}

// The 16 MFMAs of a chunk-end update: W1 += K^T E1n, W2 += A^K^T En2 (K = 16 over the
// chunk's tokens). K^T and En2^T come from the staged [token][d] rows through transposing
// LDS loads, each in one half of a K = 32 operand with zeros in the other.
__device__ __forceinline__ void chunk_update(f4 (&W1c)[NDT][NHT], f4 (&W2c)[NHT][NDT], const __bf16* Krows,
                                             const __bf16* E2rows, bf16x8 e1, bf16x8 ak, int g, int c16,
                                             bf16x4 zz) {
  // K^T and En2^T of d tiles (0, 1) and (2, 3) fill both halves of an operand; the other
  // operand carries its data in one half and zeros in the other, which selects the d tile
  const bf16x8 k01 = cat(tgroup(Krows, RS, 0, g, c16), tgroup(Krows, RS, 1, g, c16));
  const bf16x8 k23 = cat(tgroup(Krows, RS, 2, g, c16), tgroup(Krows, RS, 3, g, c16));
  const bf16x8 e01 = cat(tgroup(E2rows, RS, 0, g, c16), tgroup(E2rows, RS, 1, g, c16));
  const bf16x8 e23 = cat(tgroup(E2rows, RS, 2, g, c16), tgroup(E2rows, RS, 3, g, c16));
  update_mfmas(W1c, W2c, k01, k23, e01, e23, e1, ak, zz);
}

// Operands of a staged [token][d] chunk: rows (token = lane%16), permuted d order.
__device__ __forceinline__ void rows(const __bf16* X, int g, int c16, bf16x8 (&a)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    a[ks] = cat(lds4(&X[c16 * RS + 32 * ks + 4 * g]), lds4(&X[c16 * RS + 32 * ks + 16 + 4 * g]));
}
// bf16 operand copies of the fp32 weight tiles.
__device__ __forceinline__ void cvt_w(const f4 (&W1c)[NDT][NHT], const f4 (&W2c)[NHT][NDT], bf16x4 (&W1b)[NDT][NHT],
                                      bf16x8 (&W2b8)[NDT]) {
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) W1b[dt][ht] = cvt4(W1c[dt][ht]);
    W2b8[dt] = cat(cvt4(W2c[0][dt]), cvt4(W2c[1][dt]));
  }
}
// bf16 operand copy of the fp32 W1 tiles alone.
__device__ __forceinline__ void cvt_w1(const f4 (&W1c)[NDT][NHT], bf16x4 (&W1b)[NDT][NHT]) {
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) W1b[dt][ht] = cvt4(W1c[dt][ht]);
}
// X W1 for this wave's h tiles (X as row operands).
__device__ __forceinline__ void xw1(const bf16x8 (&a)[2], const bf16x4 (&W1b)[NDT][NHT], f4 (&out)[NHT]) {
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    f4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) acc = mfma32(a[ks], cat(W1b[2 * ks][ht], W1b[2 * ks + 1][ht]), acc);
    out[ht] = acc;
  }
}

// Per-workgroup view of one (batch, head).
struct Ctx {
  int tid, lane, w, g, c16, head, hidx, hs, T, nchunks;
  int m;            // 16-token sub-tiles per mini-batch (chunk / 16)
  unsigned* flags;  // counter words of this head
  char* ring;       // ring of this head
  const __bf16* Kg;
  const __bf16* Xg;  // V (producer) or Q (consumer)
  __bf16* Zg;
  const float* etag;
};
// Chunk-start weights of the head, LayerNorm affine parameters and identity operands.
struct HeadState {
  f4 W1c[NDT][NHT], W2c[NHT][NDT];
  float gam[NDT], bet[NDT];
  Ident id;
};
__device__ __forceinline__ void head_init(const ScanParams& p, const Ctx& x, HeadState& h) {
  const bool per_seq = (p.flags & TTT_W0_PER_SEQ) != 0;
  const size_t wh = per_seq ? static_cast<size_t>(x.head) : static_cast<size_t>(x.hidx);
  wtiles_load(p.w0_1 + wh * D * HID, p.w0_2 + wh * HID * D, x.g, x.c16, x.hs, h.W1c, h.W2c);
  h.id = make_ident(x.g, x.c16);
#pragma unroll
  for (int i = 0; i < NDT; ++i) {
    h.gam[i] = p.gamma[x.hidx * D + 16 * i + x.c16];
    h.bet[i] = p.beta[x.hidx * D + 16 * i + x.c16];
  }
}

template <int GELU_KIND, bool LOCAL, bool LARGE, bool KEY = false>
__device__ __forceinline__ void producer_body(const ScanParams& p, const Ctx& x, ProdSmem& S) {
  const int tid = x.tid, lane = x.lane, w = x.w, g = x.g, c16 = x.c16, head = x.head, hs = x.hs;
  const int T = x.T, nchunks = x.nchunks;
  const HandOff<LOCAL> ho(x.flags, x.ring);
  // Output rule z_t = f(K_t; W at the mini-batch start) (TTT_OUTPUT_KEY): the LayerNorm lanes
  // write it from Z^K, and there is no consumer to hand anything to.
  constexpr bool key_out = KEY;
  const __bf16* Kg = x.Kg;
  const __bf16* Xg = x.Xg;
  const float* etag = x.etag;
  HeadState hst;
  head_init(p, x, hst);
  auto& W1c = hst.W1c;
  auto& W2c = hst.W2c;
  const float* gam = hst.gam;
  const float* bet = hst.bet;
  const Ident& id = hst.id;
  // the update applied at chunk 0 (from the zero carry of "chunk -1") reads stage slot 3
  // and the En2 rows before anything is written there: they start at zero (finite)
  {
    uint4* z4 = reinterpret_cast<uint4*>(S.st[3].K);
    for (int i = tid; i < static_cast<int>(sizeof(S.st[3].K)) / 16; i += NT) z4[i] = uint4{0u, 0u, 0u, 0u};
    uint4* e4 = reinterpret_cast<uint4*>(S.E2);
    for (int i = tid; i < static_cast<int>(sizeof(S.E2)) / 16; i += NT) e4[i] = uint4{0u, 0u, 0u, 0u};
  }
  if (tid < 8) S.zeros[tid] = (__bf16)0.f;
  // Streamed rows read for the last time (V, eta here; K and Q in the consumer) and the Z
  // stores are non-temporal, so that they leave the L2 first and the ring lines stay: with
  // plain accesses about a quarter of the ring's stores were evicted to HBM (333 MB written
  // per launch at B=8, H=12, T=8192 against 142 MB with these hints). K stays a plain load:
  // the consumer reads the same rows a few chunks later and finds them in the L2.
  // staging by waves 4..7: thread -> (token, 4 consecutive d). Every wave issues exactly
  // three loads (K, V, eta) per chunk (waves 0..3 load the same addresses as waves 4..7 and
  // drop the data), so the count of memory operations after the slot stores is fixed.
  const int lt = tid & 255;
  const int st_t = lt >> 4, st_d = (lt & 15) * 4;
  struct Ld {
    uint2 k, x;
    float e;
  };
  auto gload = [&](int chunk) {
    Ld r;
    const size_t off = (static_cast<size_t>(chunk) * BC + st_t) * D + st_d;
    r.k = *reinterpret_cast<const uint2*>(Kg + off);
    const u32x2 xv = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(Xg + off));
    r.x = uint2{xv[0], xv[1]};
    r.e = __builtin_nontemporal_load(etag + chunk * BC + (lt & 15));
    return r;
  };
  auto stage_write = [&](int chunk, const Ld& r) {
    PStage& st = S.st[chunk & 3];
    *reinterpret_cast<uint2*>(&st.K[st_t * RS + st_d]) = r.k;
    *reinterpret_cast<uint2*>(&st.X[st_t * RS + st_d]) = r.x;
    if (lt < BC) st.eta[lt] = r.e * p.eta_scale;
  };
  if (w >= 4) {
    stage_write(0, gload(0));
    if (nchunks > 1) stage_write(1, gload(1));
  }
  __syncthreads();
  const bf16x4 zz = lds4(S.zeros);

  // bf16 operand copies of the weights the current mini-batch's gradients are taken at (the
  // mini-batch start): made once per mini-batch. With 16-token mini-batches that is every
  // sub-tile; with larger ones every sub-tile of the mini-batch reuses them.
  // (kept across sub-tiles only for mini-batches above 16 tokens; with 16-token mini-batches
  // each step makes its own, which keeps them out of the registers live across the loop)
  struct WCopies {
    bf16x4 W1b[NDT][NHT];
    bf16x8 W2b8[NDT];
    bf16x4 W2Tb[NDT][NHT];
  };
  WCopies keep;
  const int m = LARGE ? x.m : 1;
  // chunk 0 enters with P = K(0) W0, and zero look-ahead terms
  Carry ca{}, cb{};
  {
    cvt_w(W1c, W2c, keep.W1b, keep.W2b8);
    bf16x8 aK[2];
    rows(S.st[0].K, g, c16, aK);
    xw1(aK, keep.W1b, ca.P);
  }

#ifdef TTT_PHASE_CLOCKS
  unsigned long long pacc[11] = {};
#endif
  auto step = [&](const int c, const Carry& in, Carry& out) {
    TTT_STAMP(s0);
    const PStage& st = S.st[c & 3];
    const int t0 = c * BC;
    const Ld ld = gload(min(c + 2, nchunks - 1));
    // sub-tile c of a mini-batch of m sub-tiles: the first one starts from the weights after
    // every update so far, the others take their gradients at those same weights
    const int sub = LARGE ? c % m : 0;
    const bool first = sub == 0, last = sub == m - 1;
    WCopies local;
    WCopies& wc = LARGE ? keep : local;
    auto& W1b = wc.W1b;
    auto& W2b8 = wc.W2b8;
    auto& W2Tb = wc.W2Tb;
    // first: H^K(c) = K(c) W1(c-1) + (K(c) K(c-1)^T) E1n(c-1) (the look-ahead plus the update
    // of the sub-tile before); otherwise H^K(c) = K(c) W1(start), computed one step ahead
    f4 hk[NHT];
    if (first) {
      hk[0] = mfma32(cat(in.sA, zz), in.e1, in.P[0]);
      hk[1] = mfma32(cat(zz, in.sA), in.e1, in.P[1]);
    } else {
      hk[0] = in.P[0];
      hk[1] = in.P[1];
    }
    // the update of chunk c - 1 (W(c) = W(c-1) + ...), next to the GELU work
    // (at chunk 0 the carry is zero and the operands are zero-filled: an exact no-op)
    chunk_update(W1c, W2c, S.st[(c - 1) & 3].K, S.E2, in.e1, in.ak, g, c16, zz);
    // A^K (R layout: m = h, k = token), G
    bf16x4 akR[NHT];
    f4 gk[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 a, gd;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v, d1;
        act_d_fwd<GELU_KIND>(hk[ht][r], v, d1);
        a[r] = v;
        gd[r] = d1;
      }
      gk[ht] = gd;
      akR[ht] = cvt4(a);
    }
    out.ak = cat(akR[0], akR[1]);
    TTT_DEP(out.ak[0]);
    TTT_DEP(gk[0][0]);
    TTT_STAMP(s1);
    // scheduling hint: issue the 16 update MFMAs one at a time between runs of 4 VALU
    // instructions of the GELU above, so the matrix unit works while the VALU does
    // (runs of 2, 3, 5, 6 or 8 measured slower)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    if (first)
      cvt_w(W1c, W2c, W1b, W2b8);  // the new mini-batch's start weights
    else if (last)
      cvt_w1(W1c, W1b);  // W1 with every update but this sub-tile's, for the next look-ahead
    // look-ahead for sub-tile c + 1: K(c+1) W1 and, when c + 1 starts a mini-batch,
    // K(c+1) K(c)^T for the update of sub-tile c (after the last sub-tile the slot holds
    // other data and the result is not used)
    {
      bf16x8 aK1[2];
      rows(S.st[(c + 1) & 3].K, g, c16, aK1);
      xw1(aK1, W1b, out.P);
      if (last) {
        bf16x8 aK[2];
        rows(st.K, g, c16, aK);
        f4 sT = mfma32(aK[0], aK1[0], zero4());  // C[t][t'] = K(c)_t . K(c+1)_t'
        sT = mfma32(aK[1], aK1[1], sT);
        out.sA = cvt4(sT);
      }
    }
    // Z^K partial over this wave's h slice
    const bf16x8 akT8 = cat(cvt4(mfma32(out.ak, id.ilo, zero4())), cvt4(mfma32(out.ak, id.ihi, zero4())));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const f4 acc = mfma32(akT8, W2b8[dt], zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) S.red[w][dt][r][lane] = acc[r];
    }
    TTT_STAMP(s2);
    // W2^T tiles for E1n (once per mini-batch): waves 0..3 now, waves 4..7 during the LayerNorm
    auto w2t = [&]() {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        W2Tb[dt][0] = cvt4(mfma32(W2b8[dt], id.ilo, zero4()));
        W2Tb[dt][1] = cvt4(mfma32(W2b8[dt], id.ihi, zero4()));
      }
    };
    // LayerNorm inputs that do not depend on Z^K, prepared by the LayerNorm waves ahead of
    // the barrier: K + beta - V and -eta for token 4w + lane/16
    float kvb[NDT] = {0.f, 0.f, 0.f, 0.f}, neta = 0.f;
    if (w < 4) {
      if (first) w2t();
      const int t = 4 * w + g;
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const int d = 16 * i + c16;
        kvb[i] = bf(st.K[t * RS + d]) + bet[i] - bf(st.X[t * RS + d]);
      }
      neta = -st.eta[t];
    }
    // publish chunk c - 1: its slot stores were the last vector-memory operations before
    // this chunk's three input loads
    if (c > 0 && !key_out) {
      asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
      if (lane == 0) ho.st(w, static_cast<unsigned>(c));
      compiler_fence();
    }
    // chunks the consumer is done reading (checked after the barriers)
    const unsigned cons = key_out ? 0u : ho.ld(16);
    if (p.saved && first) {
      float* sv = p.saved + (static_cast<size_t>(head) * (nchunks / m) + c / m) * (2 * D * HID);
      wtiles_store(sv, sv + D * HID, g, c16, hs, W1c, W2c);
    }
    TTT_STAMP(s3);
    __syncthreads();
    TTT_STAMP(s4);

    if (w < 4) {
      // LayerNorm forward/backward of Z^K: token 4w + lane/16, 16 lanes each
      const int t = 4 * w + g;
      float z[NDT];
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += S.red[ww][i][t & 3][16 * (t >> 2) + c16];
        z[i] = s;
      }
      const LnStats ls = ln_stats(z, p.eps);
      float xh[NDT], gg[NDT], l2 = 0.f, sg = 0.f, sgx = 0.f;
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const int d = 16 * i + c16;
        xh[i] = (z[i] - ls.mu) * ls.rs;
        const float r = kvb[i] + gam[i] * xh[i];
        l2 += r * r;
        gg[i] = 2.f * r * gam[i];
        sg += gg[i];
        sgx += gg[i] * xh[i];
      }
      const float mg = sum16(sg) * (1.0f / D), mgx = sum16(sgx) * (1.0f / D);
      const float ne2 = neta * ls.rs;
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const int d = 16 * i + c16;
        const __bf16 e = (__bf16)(ne2 * (gg[i] - mg - xh[i] * mgx));
        S.E2[t * RS + d] = e;
      }
      if (p.loss) {
        const float loss = sum16(l2);
        if (c16 == 0) p.loss[static_cast<size_t>(head) * T + t0 + t] = loss;
      }
      if (key_out) {
        // z = K + gamma xhat + beta = (K + beta - V) + gamma xhat + V
#pragma unroll
        for (int i = 0; i < NDT; ++i) {
          const int d = 16 * i + c16;
          x.Zg[static_cast<size_t>(t0 + t) * D + d] = (__bf16)(kvb[i] + gam[i] * xh[i] + bf(st.X[t * RS + d]));
        }
      }
      // mean(g) is non-finite whenever any residual (inputs, Z^K) is
      if (c16 == 0) flag_nonfinite(p.status, mg);
    } else {
      if (first) w2t();
      if (c + 2 < nchunks) stage_write(c + 2, ld);
    }
    TTT_STAMP(s5);
    __syncthreads();
    TTT_STAMP(s6);

    // E1n(c) = (En2 W2^T) (.) G
    bf16x8 aE[2];
    rows(S.E2, g, c16, aE);
    bf16x4 e1[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma32(aE[ks], cat(W2Tb[2 * ks][ht], W2Tb[2 * ks + 1][ht]), acc);
      e1[ht] = cvt4(acc * gk[ht]);
    }
    out.e1 = cat(e1[0], e1[1]);
    TTT_DEP(out.e1[0]);
    TTT_STAMP(s7);

    // hand chunk c to the consumer: slot c % RING must have been read (chunk c - RING)
    if (!key_out) {
      const unsigned need = c >= RING ? static_cast<unsigned>(c - RING + 1) : 0u;
      if (cons < need) spin_geq(ho, 16, need, p.status);
      compiler_fence();
      const int base = (c % RING) * SLOT_BYTES;
      ho.st16(base + SLOT_E1 + (w * 64 + lane) * 16, out.e1);
      ho.st16(base + SLOT_AK + (w * 64 + lane) * 16, out.ak);
      if (w == 0) {
        ho.st16(base + SLOT_E2 + lane * 32, cat(tgroup(S.E2, RS, 0, g, c16), tgroup(S.E2, RS, 1, g, c16)));
        ho.st16(base + SLOT_E2 + lane * 32 + 16, cat(tgroup(S.E2, RS, 2, g, c16), tgroup(S.E2, RS, 3, g, c16)));
      }
      compiler_fence();
    }
#ifdef TTT_PHASE_CLOCKS
    TTT_STAMP(s8);
    if (c >= 16) {
      const unsigned long long ph[8] = {s1 - s0, s2 - s1, s3 - s2, s4 - s3, s5 - s4, s6 - s5, s7 - s6, s8 - s7};
      for (int k = 0; k < 8; ++k) pacc[k] += ph[k];
      pacc[8] += 1;
      pacc[9] = s8;
    }
    if (c == 16) pacc[10] = s0;
#endif
  };

  // two chunks per trip, so the carried registers alternate without copies
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    step(c, ca, cb);
    step(c + 1, cb, ca);
  }
  if (c < nchunks) step(c, ca, cb);
  const Carry& last = (nchunks & 1) ? cb : ca;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0 && !key_out) ho.st(w, static_cast<unsigned>(nchunks));
  // the last chunk's update (its En2 is still in E2)
  chunk_update(W1c, W2c, S.st[(nchunks - 1) & 3].K, S.E2, last.e1, last.ak, g, c16, zz);
  if (p.wt_1)
    wtiles_store(p.wt_1 + static_cast<size_t>(head) * D * HID, p.wt_2 + static_cast<size_t>(head) * HID * D,
                 g, c16, hs, W1c, W2c);
#ifdef TTT_PHASE_CLOCKS
  if (head == 0 && lane == 0)
    for (int k = 0; k < 11; ++k) g_phase_clocks[0][w][k] = pacc[k];
#endif
  return;
}

template <int GELU_KIND, bool LOCAL>
__device__ __forceinline__ void consumer_body(const ScanParams& p, const Ctx& x, ConsSmem& S) {
  const int tid = x.tid, lane = x.lane, w = x.w, g = x.g, c16 = x.c16;
  const int nchunks = x.nchunks;
  const HandOff<LOCAL> ho(x.flags, x.ring);
  const __bf16* Kg = x.Kg;
  const __bf16* Xg = x.Xg;
  __bf16* Zg = x.Zg;
  HeadState hst;
  head_init(p, x, hst);
  auto& W1c = hst.W1c;
  auto& W2c = hst.W2c;
  const float* gam = hst.gam;
  const float* bet = hst.bet;
  const Ident& id = hst.id;
  if (tid < 8) S.zeros[tid] = (__bf16)0.f;
  // staging by all waves: thread -> (token, 2 consecutive d)
  const int st_t = tid >> 5, st_d = (tid & 31) * 2;
  struct Ld {
    unsigned k, x;
  };
  auto gload = [&](int chunk) {
    Ld r;
    const size_t off = (static_cast<size_t>(chunk) * BC + st_t) * D + st_d;
    r.k = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(Kg + off));
    r.x = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(Xg + off));
    return r;
  };
  auto stage_write = [&](int slot, const Ld& r) {
    PStage& st = S.st[slot];
    *reinterpret_cast<unsigned*>(&st.K[st_t * RS + st_d]) = r.k;
    *reinterpret_cast<unsigned*>(&st.X[st_t * RS + st_d]) = r.x;
  };
  stage_write(0, gload(0));
  __syncthreads();
  const bf16x4 zz = lds4(S.zeros);

  auto ln_out = [&](int cc) {
    const PStage& So = S.st[cc % 3];
    const int t = 4 * w + g;
    float z[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) s += S.red[cc & 1][ww][i][t & 3][16 * (t >> 2) + c16];
      z[i] = s;
    }
    const LnStats ls = ln_stats(z, p.eps);
    float chk = 0.f;
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      const int d = 16 * i + c16;
      const float o = bf(So.X[t * RS + d]) + gam[i] * (z[i] - ls.mu) * ls.rs + bet[i];
      chk += o;
      __builtin_nontemporal_store((__bf16)o, &Zg[static_cast<size_t>(cc * BC + t) * D + d]);
    }
    chk = sum16(chk);
    if (c16 == 0) flag_nonfinite(p.status, chk);
  };

#ifdef TTT_PHASE_CLOCKS
  unsigned long long cacc[11] = {};
#endif
  auto step = [&](const int c, const Slot& cur, Slot& nxt) {
    TTT_STAMP(s0);
    const int sl = c % 3;
    const PStage& st = S.st[sl];
    const bool has_next = c + 1 < nchunks;
    // counters for chunk c + 1, checked late in this chunk
    const unsigned rdy_own = ho.ld(w), rdy_0 = ho.ld(0);
    Ld ld{};
    if (has_next) ld = gload(c + 1);
    bf16x8 aK[2], aQ[2];
    rows(st.K, g, c16, aK);
    rows(st.X, g, c16, aQ);
    bf16x4 W1b[NDT][NHT];
    bf16x8 W2b8[NDT];
    cvt_w(W1c, W2c, W1b, W2b8);
    f4 hq[NHT];
    xw1(aQ, W1b, hq);
    f4 s1t = zero4();  // C[s][t] = K_s . Q_t
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) s1t = mfma32(aK[ks], aQ[ks], s1t);

    // H^Q = Q W1 + tril(Q K^T) E1n ; A^Q = GELU(H^Q)
    f4 s1m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s1m[r] = (4 * g + r) <= c16 ? s1t[r] : 0.f;
    const bf16x4 s1a = cvt4(s1m);
    bf16x4 aqR[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const f4 h = mfma32(ht == 0 ? cat(s1a, zz) : cat(zz, s1a), cur.e1, hq[ht]);
      f4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = act_fwd<GELU_KIND>(h[r]);
      aqR[ht] = cvt4(a);
    }
    const bf16x8 aqR8 = cat(aqR[0], aqR[1]);
    TTT_DEP(aqR8[0]);
    TTT_STAMP(s1);
    const bf16x8 aqT8 = cat(cvt4(mfma32(aqR8, id.ilo, zero4())), cvt4(mfma32(aqR8, id.ihi, zero4())));
    const bf16x8 akT8 = cat(cvt4(mfma32(cur.ak, id.ilo, zero4())), cvt4(mfma32(cur.ak, id.ihi, zero4())));
    // Z^Q partial = A^Q W2 + tril(A^Q A^K^T) En2 over this wave's h slice
    const f4 s2t = mfma32(akT8, aqT8, zero4());  // C[s][t] = A^K_s . A^Q_t (this slice)
    f4 s2m;
#pragma unroll
    for (int r = 0; r < 4; ++r) s2m[r] = (4 * g + r) <= c16 ? s2t[r] : 0.f;
    const bf16x4 s2a = cvt4(s2m);
    const bf16x8 s2lo = cat(s2a, zz), s2hi = cat(zz, s2a);  // select the d tile of the En2 operand
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 acc = mfma32(aqT8, W2b8[dt], zero4());
      acc = mfma32(dt & 1 ? s2hi : s2lo, cur.e2[dt >> 1], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) S.red[c & 1][w][dt][r][lane] = acc[r];
    }
    TTT_STAMP(s2);
    // the producer's chunk-end update, from the same operands
    update_mfmas(W1c, W2c, cat(tgroup(st.K, RS, 0, g, c16), tgroup(st.K, RS, 1, g, c16)),
                 cat(tgroup(st.K, RS, 2, g, c16), tgroup(st.K, RS, 3, g, c16)), cur.e2[0], cur.e2[1], cur.e1,
                 cur.ak, zz);
    // this wave is done with slot c (its loads have returned: the dependency forces the
    // wait); wave 0 releases the slot after the barrier below. Then prefetch chunk c + 1.
    {
      const unsigned dep = slot_dep(cur);
      asm volatile("" ::"v"(dep) : "memory");
      compiler_fence();
    }
    TTT_STAMP(s3);
    if (has_next) {
      const unsigned need = static_cast<unsigned>(c + 2);
      if (min(rdy_own, rdy_0) < need) {
        spin_geq(ho, w, need, p.status);
        if (w != 0) spin_geq(ho, 0, need, p.status);
      }
      compiler_fence();
      slot_load(ho, nxt, c + 1, w, lane);
      stage_write((c + 1) % 3, ld);
    }
    TTT_STAMP(s4);
    __syncthreads();
    TTT_STAMP(s5);
    if (w == 0 && lane == 0) ho.st(16, static_cast<unsigned>(c + 1));
    if (w < 4) ln_out(c);
#ifdef TTT_PHASE_CLOCKS
    TTT_STAMP(s6);
    if (c >= 16) {
      const unsigned long long ph[6] = {s1 - s0, s2 - s1, s3 - s2, s4 - s3, s5 - s4, s6 - s5};
      for (int k = 0; k < 6; ++k) cacc[k] += ph[k];
      cacc[8] += 1;
      cacc[9] = s6;
    }
    if (c == 16) cacc[10] = s0;
#endif
  };

  spin_geq(ho, w, 1u, p.status);
  if (w != 0) spin_geq(ho, 0, 1u, p.status);
  compiler_fence();
  Slot sa, sb;
  slot_load(ho, sa, 0, w, lane);
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    step(c, sa, sb);
    step(c + 1, sb, sa);
  }
  if (c < nchunks) step(c, sa, sb);
#ifdef TTT_PHASE_CLOCKS
  if (x.head == 0 && lane == 0)
    for (int k = 0; k < 11; ++k) g_phase_clocks[1][w][k] = cacc[k];
#endif
}

template <int GELU_KIND, bool LARGE>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_mfma_pair_kernel(ScanParams p, Pair q) {
  __shared__ SmemP sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  Ctx x;
  x.tid = threadIdx.x;
  x.lane = x.tid & 63;
  x.w = x.tid >> 6;
  x.g = x.lane >> 4;
  x.c16 = x.lane & 15;
  const int b = blockIdx.x;
  x.head = (b >> 4) * 8 + (b & 7);
  const bool producer = ((b >> 3) & 1) == 0;
  if (x.head >= q.nheads) return;  // both members of a padding pair leave
  x.hidx = x.head % p.H;
  x.hs = x.w * HS;
  x.T = p.T;
  x.nchunks = p.T / BC;
  x.m = p.chunk / BC;
  x.flags = q.flags + static_cast<size_t>(x.head) * FLAG_WORDS;
  x.ring = q.ring + static_cast<size_t>(x.head) * RING * SLOT_BYTES;
  const size_t io_off = static_cast<size_t>(x.head) * p.T * D;
  x.Kg = static_cast<const __bf16*>(p.K) + io_off;
  x.Xg = static_cast<const __bf16*>(producer ? p.V : p.Q) + io_off;
  x.Zg = static_cast<__bf16*>(p.Z) + io_off;
  x.etag = p.eta + static_cast<size_t>(x.head) * p.T;
  // placement: each side publishes its XCD id + 1 (device-coherent) and reads the partner's
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const int mine = producer ? FLAG_XCC : FLAG_XCC + 1, theirs = producer ? FLAG_XCC + 1 : FLAG_XCC;
  if (x.tid == 0) __hip_atomic_store(x.flags + mine, xcc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  unsigned other = 0;
  for (int it = 0; it < kSpinLimit; ++it) {
    other = __hip_atomic_load(x.flags + theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (other != 0) break;
    __builtin_amdgcn_s_sleep(2);
  }
  if (other == 0 && x.tid == 0) atomicOr(p.status, kStatusTimeout);
  const bool local = other == xcc + 1 && !(p.flags & TTT_FORCE_DEVICE_SCOPE);
  if (producer) {
    if (local)
      producer_body<GELU_KIND, true, LARGE>(p, x, sm.p);
    else
      producer_body<GELU_KIND, false, LARGE>(p, x, sm.p);
  } else {
    if (local)
      consumer_body<GELU_KIND, true>(p, x, sm.c);
    else
      consumer_body<GELU_KIND, false>(p, x, sm.c);
  }
}

// The key-side output rule: one workgroup per (batch, head) running the producer alone (its
// hand-off code is compiled out, so the flags and ring are never touched); LARGE for
// mini-batches above 16 tokens, as in the paired kernel.
template <int GELU_KIND, bool LARGE>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_mfma_key_kernel(ScanParams p) {
  __shared__ ProdSmem sm;
  TTT_POISON(sm);
  TTT_POISON_DONE();
  Ctx x;
  x.tid = threadIdx.x;
  x.lane = x.tid & 63;
  x.w = x.tid >> 6;
  x.g = x.lane >> 4;
  x.c16 = x.lane & 15;
  x.head = blockIdx.x;
  x.hidx = x.head % p.H;
  x.hs = x.w * HS;
  x.T = p.T;
  x.nchunks = p.T / BC;
  x.m = p.chunk / BC;
  x.flags = nullptr;
  x.ring = nullptr;
  const size_t io_off = static_cast<size_t>(x.head) * p.T * D;
  x.Kg = static_cast<const __bf16*>(p.K) + io_off;
  x.Xg = static_cast<const __bf16*>(p.V) + io_off;
  x.Zg = static_cast<__bf16*>(p.Z) + io_off;
  x.etag = p.eta + static_cast<size_t>(x.head) * p.T;
  producer_body<GELU_KIND, true, LARGE, true>(p, x, sm);
}

__global__ void pair_reset_kernel(unsigned* flags, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) flags[i] = 0u;
}

size_t flag_bytes(int nheads) {
  return (static_cast<size_t>(nheads) * FLAG_WORDS * sizeof(unsigned) + 255) / 256 * 256;
}

}  // namespace

bool fwd_pair_supported(const ScanParams& p) {
  return p.kind == TTT_MLP && p.d == D && p.hid == HID && p.io == TTT_BF16 && p.chunk >= BC &&
         p.chunk % BC == 0 && p.chunk <= kMaxPairChunk;
}

size_t fwd_pair_workspace_bytes(int nheads) {
  return flag_bytes(nheads) + static_cast<size_t>(nheads) * RING * SLOT_BYTES;
}

int fwd_pair_blocks(int nheads) { return (nheads + 7) / 8 * 16; }

// Whether the current device can hold every workgroup of the paired launch at once
// (cooperative launch support, and resident workgroups per CU times the CU count). The
// device answers are cached per device ordinal.
bool fwd_pair_fits(int nheads) {
  constexpr int kMaxDev = 64;
  static int cap[kMaxDev];  // 0 = unknown, else 1 + resident workgroups on the device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return false;
  if (cap[dev] == 0) {
    int coop = 0, ncu = 0, per_cu = 0;
    const bool ok =
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(fwd_mfma_pair_kernel<TTT_GELU_ERF, true>), NT, 0) == hipSuccess;
    cap[dev] = 1 + ((ok && coop) ? ncu * per_cu : 0);
  }
  return fwd_pair_blocks(nheads) <= cap[dev] - 1;
}

hipError_t launch_fwd_mfma_pair(const ScanParams& p, hipStream_t stream) {
  const int nheads = p.B * p.H;
  Pair q;
  q.flags = reinterpret_cast<unsigned*>(p.wbuf);
  q.ring = reinterpret_cast<char*>(p.wbuf) + flag_bytes(nheads);
  q.nheads = nheads;
  const int nflags = nheads * FLAG_WORDS;
  hipLaunchKernelGGL(pair_reset_kernel, dim3((nflags + 255) / 256), dim3(256), 0, stream, q.flags, nflags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScanParams pc = p;
  void* args[] = {&pc, &q};
  // one kernel per mini-batch regime, so that the 16-token one keeps its own register allocation
  const bool large = p.chunk > BC;
  const void* fn = p.gelu == TTT_GELU_TANH
                       ? (large ? reinterpret_cast<const void*>(fwd_mfma_pair_kernel<TTT_GELU_TANH, true>)
                                : reinterpret_cast<const void*>(fwd_mfma_pair_kernel<TTT_GELU_TANH, false>))
                       : (large ? reinterpret_cast<const void*>(fwd_mfma_pair_kernel<TTT_GELU_ERF, true>)
                                : reinterpret_cast<const void*>(fwd_mfma_pair_kernel<TTT_GELU_ERF, false>));
  return hipLaunchCooperativeKernel(fn, dim3(fwd_pair_blocks(nheads)), dim3(NT), args, 0, stream);
}

bool fwd_key_supported(const ScanParams& p) {
  return fwd_pair_supported(p) && (p.flags & TTT_OUTPUT_KEY);
}

hipError_t launch_fwd_mfma_key(const ScanParams& p, hipStream_t stream) {
  const int nheads = p.B * p.H;
  const bool large = p.chunk > BC;
  if (p.gelu == TTT_GELU_TANH) {
    if (large)
      hipLaunchKernelGGL((fwd_mfma_key_kernel<TTT_GELU_TANH, true>), dim3(nheads), dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_mfma_key_kernel<TTT_GELU_TANH, false>), dim3(nheads), dim3(NT), 0, stream, p);
  } else {
    if (large)
      hipLaunchKernelGGL((fwd_mfma_key_kernel<TTT_GELU_ERF, true>), dim3(nheads), dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_mfma_key_kernel<TTT_GELU_ERF, false>), dim3(nheads), dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ttt

#ifdef TTT_PHASE_CLOCKS
// Copies the per-phase clock sums of the last launch to host memory (2 * 8 * 16 values).
extern "C" int ttt_phase_clocks_read(unsigned long long* host) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(ttt::g_phase_clocks), sizeof(ttt::g_phase_clocks)) == hipSuccess ? 0 : 1;
}
#endif
