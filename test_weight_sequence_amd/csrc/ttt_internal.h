// Internal interface between the C-ABI host layer (ttt_abi.cpp) and the kernel
// translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ttt.h"

namespace ttt {

constexpr unsigned kStatusNonFinite = 1u;
constexpr unsigned kStatusTimeout = 2u;    // a bounded wait between workgroups expired
constexpr size_t kStatusBytes = 256;  // status word region at the start of a workspace
constexpr int kMaxChunk = 16;
constexpr int kThreads = 256;         // threads per workgroup of the portable kernels

// Everything a kernel needs about one call; plain values and device pointers.
struct ScanParams {
  int kind, B, H, T, d, hid, chunk, io, gelu, flags;
  float eps, eta_scale;
  const void* Q;
  const void* K;
  const void* V;
  const float* eta;
  const float* gamma;
  const float* beta;
  const float* w0_1;
  const float* w0_2;
  void* Z;
  float* wt_1;
  float* wt_2;
  float* loss;
  float* saved;    // [B*H, T/chunk, nW] chunk-start weights, or null
  float* wbuf;     // [B*H, nW] fp32 working weights (portable kernel); [B*H, 2 nW] with momentum
  unsigned* status;
  // momentum / forget-gate variant (portable kernel only; null mom = the plain scan)
  const float* mom;    // [B*H, T] momentum decay per token
  const float* alpha;  // [B*H, T] forget gate per token
  const float* s0_1;   // [B*H, ..] momentum carried in, or null (zero)
  const float* s0_2;
  float* st_1;         // [B*H, ..] momentum out, or null
  float* st_2;
};

struct BwdParams {
  int kind, B, H, T, d, hid, chunk, io, gelu, flags;
  float eps, eta_scale;
  const void* Q;
  const void* K;
  const void* V;
  const float* eta;
  const float* gamma;
  const float* beta;
  const float* saved;
  const void* dZ;
  const float* dwt_1;   // nullable
  const float* dwt_2;
  void* dQ;
  void* dK;
  void* dV;
  float* deta;
  float* dw0_1;
  float* dw0_2;
  float* dgamma;        // nullable
  float* dbeta;         // nullable
  float* work;          // per-head scratch: dW accumulators and chunk intermediates
  float* dgb;           // [B*H, 2, d] per-head dgamma/dbeta partials
  unsigned* status;
};

struct DecodeParams {
  int kind, B, H, d, hid, chunk, io, gelu, flags, pos;
  float eps, eta_scale;
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* gamma;
  const float* beta;
  float* ws_1;
  float* ws_2;
  float* acc_1;
  float* acc_2;
  void* z;
  unsigned* status;
};

__host__ __device__ inline size_t n_weights(int kind, int d, int hid) {
  return kind == TTT_MLP ? static_cast<size_t>(2) * d * hid : static_cast<size_t>(d) * d;
}

// Launchers (return hipSuccess or the launch error).
hipError_t launch_fwd_generic(const ScanParams& p, hipStream_t s);
size_t fwd_generic_lds_bytes(int kind, int d, int hid, int chunk, bool momentum = false);
bool fwd_mfma_supported(const ScanParams& p);
hipError_t launch_fwd_mfma(const ScanParams& p, hipStream_t s);
// Two-workgroup (producer/consumer) variant of the tuned forward: its workspace region
// (after the status word), its grid size, whether the current device can co-schedule that
// grid, and its launcher (wbuf points at the region).
constexpr int kPairMaxHeads = 128;
// Largest mini-batch of the paired kernel (a multiple of 16 tokens); every other kernel takes
// mini-batches of at most kMaxChunk tokens.
constexpr int kMaxPairChunk = 1024;
bool fwd_pair_supported(const ScanParams& p);
size_t fwd_pair_workspace_bytes(int nheads);
int fwd_pair_blocks(int nheads);
bool fwd_pair_fits(int nheads);
hipError_t launch_fwd_mfma_pair(const ScanParams& p, hipStream_t s);
// The large-chunk SwiGLU layer (ttt_lact_fwd), MLP-like d = 64, hidden = 256, bf16 I/O.
struct LactLaunch {
  int B, H, T, chunk, flags;
  float eta_scale;
  const void* Q;
  const void* K;
  const void* V;
  const float* eta;
  const float* w0_1;
  const float* w0_2;
  const float* w0_3;
  void* Z;
  float* wt_1;  // nullable (then wt_2, wt_3 unused)
  float* wt_2;
  float* wt_3;
  unsigned* status;
  float* work;  // lact_workspace_bytes(B * H), 16-byte aligned
};
bool lact_supported(int d, int hid, int io, int chunk);
size_t lact_workspace_bytes(int nheads);
hipError_t launch_lact_fwd(const LactLaunch& L, hipStream_t s);

// The key-side output rule (TTT_OUTPUT_KEY) on the same head shape, 16-token mini-batches:
// the paired kernel's producer alone, one workgroup per head, no workspace.
bool fwd_key_supported(const ScanParams& p);
hipError_t launch_fwd_mfma_key(const ScanParams& p, hipStream_t s);
// Forward for the d = 128, hidden = 512 head: each head split by hidden units over four
// workgroups that exchange [chunk x d] partial sums through the workspace; up to the heads one
// launch holds, four more workgroups per head take the query side (producer/consumer form).
bool fwd_split_supported(const ScanParams& p);
size_t fwd_split_workspace_bytes(int nheads);
bool fwd_split_fits(int nheads);
hipError_t launch_fwd_mfma_split(const ScanParams& p, hipStream_t s);
// Momentum / forget-gate forward for the d = 64, hidden = 256 bf16 head: each head split by
// hidden units over two workgroups that hold the memory and the momentum in registers and
// exchange [chunk x d] partial sums through the workspace.
bool fwd_mom_supported(const ScanParams& p);
size_t fwd_mom_workspace_bytes(int nheads);
bool fwd_mom_fits();
hipError_t launch_fwd_mfma_mom(const ScanParams& p, hipStream_t s);
// Per-head backward workspace (floats): the carried dW, then kBwdArrays [chunk x hidden]
// intermediates (MLP only).
constexpr int kBwdArrays = 12;
__host__ __device__ inline size_t bwd_work_floats_per_head(int kind, int d, int hid, int chunk) {
  const size_t nW = kind == TTT_MLP ? static_cast<size_t>(2) * d * hid : static_cast<size_t>(d) * d;
  return nW + (kind == TTT_MLP ? static_cast<size_t>(kBwdArrays) * chunk * hid : 0);
}
hipError_t launch_bwd_generic(const BwdParams& p, hipStream_t s);
// Tuned backward (d = 64, hidden = 256, chunk 16, bf16 I/O); writes the same per-head dW
// and dgamma/dbeta partials as the portable kernel, for the same finalize kernel.
bool bwd_mfma_supported(const BwdParams& p);
hipError_t launch_bwd_mfma(const BwdParams& p, hipStream_t s);
// The same backward with two workgroups per head: the bytes of its exchange region (in the
// workspace after the per-head dW and dgamma / dbeta regions), whether the device can hold
// one group of eight heads' workgroups at once, and its launcher (xbuf: the region).
size_t bwd_split_workspace_bytes(int heads);
bool bwd_split_fits();
hipError_t launch_bwd_mfma_split(const BwdParams& p, float* xbuf, hipStream_t s);
size_t bwd_generic_lds_bytes(int kind, int d, int hid, int chunk);
hipError_t launch_bwd_finalize(const BwdParams& p, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
// Tuned decode step (MLP, d = 64, hidden = 256): one 1024-thread workgroup per head that
// streams W_start and acc through registers once.
bool decode_stream_supported(const DecodeParams& p);
hipError_t launch_decode_stream(const DecodeParams& p, hipStream_t s);
// Decode with four workgroups per head (MLP d = 64, hidden = 256); xbuf is its exchange area
// in the workspace (after the status word), decode_split_workspace_bytes(B * H) bytes that are
// zero before the first call and that every call leaves zero.
constexpr int kDecodeSplitMaxHeads = 128;
bool decode_split_supported(const DecodeParams& p);
size_t decode_split_workspace_bytes(int heads);
hipError_t launch_decode_split(const DecodeParams& p, void* xbuf, hipStream_t s);
hipError_t launch_reset_status(unsigned* status, hipStream_t s);
// dst[0] = src[0] on the stream (the status word of a workspace the caller cannot address)
hipError_t launch_copy_status(const unsigned* src, unsigned* dst, hipStream_t s);

}  // namespace ttt
