// Shared pieces of the bf16 MFMA scan kernels for the d = 64, hidden = 256, chunk 16 head
// shape: vector types, MFMA wrappers, conversions, LDS staging layout, DPP reductions and
// the activation.
//
// Register-layout rule used by every kernel: a 16x16 MFMA accumulator tile C[m][n] puts m
// on (lane/16)*4 + r and n on lane%16. A tile can feed another MFMA as an operand only
// through its m axis as the contraction index. Two tiles stacked along m give the 8
// k-values of a 16x16x32 operand in a permuted k order, and the other operand is read in
// the same permuted order. An MFMA against an identity operand swaps which index sits on
// lane%16, i.e. transposes bf16 values exactly.
#pragma once

#include "ttt_device.hpp"

namespace ttt {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int D = 64;
constexpr int HID = 256;
constexpr int BC = 16;             // chunk
constexpr int NDT = D / 16;        // d tiles
constexpr int RS = D + 8;          // padded row stride (bf16 elements) of [token][d] arrays
// Row stride (floats) of the cross-wave partial-sum rows. LayerNorm lanes read four rows at
// once (16 lanes each); 80 = 64 + 16 puts the four rows on different banks.
constexpr int PS = 80;

struct Stage {
  alignas(16) __bf16 K[BC * RS];
  alignas(16) __bf16 Q[BC * RS];
  alignas(16) __bf16 V[BC * RS];
  float eta[BC];
};

// Transposing LDS load of four bf16 (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane 4q + e receives element e of the 8-byte chunks addressed by lanes q, q+4, q+8, q+12.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_tr4(const __bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const auto lp = (lds_s16x4*)((__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}
// Four consecutive tokens of one column of a [token][d] LDS array with row stride rs: lane
// (g, c16) gets X[4 g + r][16 dt + c16], r = 0..3 (lane (g, 4q + e) addresses row 4 g + e',
// columns 16 dt + 4 q' .. + 3 with q' = c16 % 4, e' = c16 / 4). As an MFMA operand that is the
// transposed chunk with k = token: K^T or En2^T for the K = 16 update products.
__device__ __forceinline__ bf16x4 tgroup(const __bf16* X, int rs, int dt, int g, int c16) {
  return lds_tr4(&X[(4 * g + (c16 >> 2)) * rs + 16 * dt + 4 * (c16 & 3)]);
}

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f4 mfma32(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// K = 16 product (k = 4*(lane/16) + j, j < 4) issued as a 16x16x32 MFMA whose upper four
// k-slots are zero in both operands. The result is identical; the kernels use only the
// 16x16x32 encoding (the legacy 16x16x16 bf16 encoding read a source register that the
// compiler had already reallocated to a following VALU write).
__device__ __forceinline__ f4 mfma16(bf16x4 a, bf16x4 b, f4 c) {
  const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                 __builtin_shufflevector(b, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 cvt4(f4 v) {
  bf16x4 r = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  return r;
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 lo4(bf16x8 a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x4 hi4(bf16x8 a) { return __builtin_shufflevector(a, a, 4, 5, 6, 7); }
__device__ __forceinline__ bf16x4 lds4(const __bf16* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}
// identity operands for transposes: B[k][n] = [k == n] with k = 4*(lane/16) + j in the
// lower (ilo) or upper (ihi) four k-slots, zero in the other four. Against a pair of tiles
// cat(X0, X1), ilo transposes X0 and ihi transposes X1, with no zero padding of X.
struct Ident {
  bf16x4 i4;
  bf16x8 ilo, ihi;
};
__device__ __forceinline__ Ident make_ident(int g, int c16) {
  Ident id;
#pragma unroll
  for (int j = 0; j < 4; ++j) id.i4[j] = (__bf16)((4 * g + j) == c16 ? 1.0f : 0.0f);
  const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
  id.ilo = cat(id.i4, z);
  id.ihi = cat(z, id.i4);
  return id;
}

// Sum over aligned groups of 16 lanes with DPP moves (no LDS round trip). After the two
// quad permutations every lane of a quad holds the quad sum, so mirroring within 8 lanes
// and then within 16 lanes pairs each lane with the other half; every lane of the group
// ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float bf(__bf16 x) { return static_cast<float>(x); }

// erf-form GELU through the branch-free A&S 7.1.26 evaluation (ttt_gelu.hpp); the tanh
// form through the library tanh.
template <int GELU_KIND>
__device__ __forceinline__ void act_d(float x, float& v, float& d1) {
  if (GELU_KIND == TTT_GELU_ERF)
    ttt_gelu::gelu_d(x, v, d1);
  else
    gelu_d(x, GELU_KIND, v, d1);
}
template <int GELU_KIND>
__device__ __forceinline__ float act(float x) {
  return GELU_KIND == TTT_GELU_ERF ? ttt_gelu::gelu(x) : gelu(x, GELU_KIND);
}
// The d = 64 forward kernels' activations (rounded to bf16 right after): the erf form
// through the lower-order A&S 7.1.25 evaluation of ttt_gelu.hpp. Its error (1.25e-5 in Phi)
// moves a scan's output by about 2e-5 at d = 64, far inside the bf16 rounding of the
// operands; the d = 128 kernel, whose drifting inputs amplify perturbations more, keeps the
// 7.1.26 form.
template <int GELU_KIND>
__device__ __forceinline__ void act_d_fwd(float x, float& v, float& d1) {
  if (GELU_KIND == TTT_GELU_ERF)
    ttt_gelu::gelu_d_fast(x, v, d1);
  else
    gelu_d(x, GELU_KIND, v, d1);
}
template <int GELU_KIND>
__device__ __forceinline__ float act_fwd(float x) {
  return GELU_KIND == TTT_GELU_ERF ? ttt_gelu::gelu_fast(x) : gelu(x, GELU_KIND);
}

// Staged elements per thread and their load type.
template <int EPT>
struct StageVec;
template <>
struct StageVec<4> {
  using T = uint2;
  using B = bf16x4;
};
template <>
struct StageVec<2> {
  using T = unsigned;
  using B = bf16x2;
};

// Per-token LayerNorm statistics over 64 values held 4 per lane by 16 lanes.
struct LnStats {
  float mu, rs;
};
__device__ __forceinline__ LnStats ln_stats(const float z[4], float eps) {
  const float mu = sum16(z[0] + z[1] + z[2] + z[3]) * (1.0f / D);
  float var = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) var += (z[i] - mu) * (z[i] - mu);
  var = sum16(var) * (1.0f / D);
  return LnStats{mu, __builtin_amdgcn_rsqf(var + eps)};  // v_rsq_f32, 1 ulp
}

// One wave's fp32 weight tiles: W1[:, hs:hs+16*NH] as [d tile][h tile] and
// W2[hs:hs+16*NH, :] as [h tile][d tile] accumulator tiles, moved to and from row-major
// [d][HID] / [HID][d] arrays with buffer instructions. Every element address is one
// per-lane register plus a compile-time tile offset, so no per-element 64-bit addresses
// stay live.
constexpr unsigned kBufFlags = 0x00020000u;
template <int NH = 2>
__device__ __forceinline__ void wtiles_load(const float* w1, const float* w2, int g, int c16, int hs,
                                            f4 (&W1c)[NDT][NH], f4 (&W2c)[NH][NDT]) {
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w1), 0, D * HID * 4, kBufFlags);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w2), 0, D * HID * 4, kBufFlags);
  const int v1 = (4 * g * HID + hs + c16) * 4, v2 = ((hs + 4 * g) * D + c16) * 4;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ht = 0; ht < NH; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        W1c[dt][ht][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, v1, ((16 * dt + r) * HID + 16 * ht) * 4, 0));
        W2c[ht][dt][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r2, v2, ((16 * ht + r) * D + 16 * dt) * 4, 0));
      }
}
// The element is copied to a scalar float first: a bit_cast applied directly to a vector
// element was compiled as a read of element 0.
template <int NH = 2>
__device__ __forceinline__ void wtiles_store(float* w1, float* w2, int g, int c16, int hs,
                                             const f4 (&W1c)[NDT][NH], const f4 (&W2c)[NH][NDT]) {
  const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(w1, 0, D * HID * 4, kBufFlags);
  const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(w2, 0, D * HID * 4, kBufFlags);
  const int v1 = (4 * g * HID + hs + c16) * 4, v2 = ((hs + 4 * g) * D + c16) * 4;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ht = 0; ht < NH; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = W1c[dt][ht][r], b = W2c[ht][dt][r];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r1, v1, ((16 * dt + r) * HID + 16 * ht) * 4, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(b), r2, v2, ((16 * ht + r) * D + 16 * dt) * 4, 0);
      }
}

}  // namespace mfma
}  // namespace ttt
