// C-ABI host layer of libttt.so: argument validation (host only), workspace sizing
// and kernel dispatch. Nothing here allocates device memory; every check runs before
// anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "ttt_internal.h"

using namespace ttt;

namespace {

constexpr size_t kMaxLds = 160 * 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Mini-batches above kMaxChunk tokens run on the paired d = 64 kernel only (forward scan and
// decode): MLP, d = 64, hidden = 256, bf16 I/O, a multiple of 16 up to kMaxPairChunk tokens,
// at most kPairMaxHeads (batch, head) pairs, and none of the flags that select another kernel.
// With TTT_OUTPUT_KEY the forward runs the key-output kernel instead (one workgroup per head,
// no head limit) and decode is not available.
bool large_chunk_ok(const ttt_config* c) {
  const bool key = (c->flags & TTT_OUTPUT_KEY) != 0;
  return c->kind == TTT_MLP && c->d == 64 && c->hidden == 256 && c->io_dtype == TTT_BF16 &&
         c->chunk % 16 == 0 && c->chunk <= kMaxPairChunk &&
         !(c->flags & TTT_FORCE_GENERIC) &&
         (key || (!(c->flags & TTT_ONE_WG_PER_HEAD) && static_cast<long long>(c->B) * c->H <= kPairMaxHeads));
}

ttt_status check_common(const ttt_config* c, bool need_T) {
  if (!c) return TTT_ERR_NULL;
  if (c->kind != TTT_LINEAR && c->kind != TTT_MLP) return TTT_ERR_UNSUPPORTED;
  if (c->io_dtype != TTT_F32 && c->io_dtype != TTT_BF16) return TTT_ERR_DTYPE;
  if (c->gelu != TTT_GELU_ERF && c->gelu != TTT_GELU_TANH) return TTT_ERR_UNSUPPORTED;
  if (c->flags & ~(TTT_W0_PER_SEQ | TTT_FORCE_GENERIC | TTT_ONE_WG_PER_HEAD | TTT_OUTPUT_KEY |
                   TTT_FORCE_DEVICE_SCOPE | TTT_DECODE_SPLIT))
    return TTT_ERR_ARG;
  if (c->B < 1 || c->H < 1 || c->d < 1 || c->chunk < 1) return TTT_ERR_SHAPE;
  if (need_T && c->T < 1) return TTT_ERR_SHAPE;
  if (c->d < 16 || c->d > 128 || c->d % 16 != 0) return TTT_ERR_UNSUPPORTED;
  if (c->kind == TTT_MLP && c->hidden != 4 * c->d) return TTT_ERR_UNSUPPORTED;
  if (c->chunk > kMaxChunk && !large_chunk_ok(c)) return TTT_ERR_UNSUPPORTED;
  if (need_T && c->T % c->chunk != 0) return TTT_ERR_SHAPE;
  if (!std::isfinite(c->ln_eps) || c->ln_eps < 0.f) return TTT_ERR_ARG;
  if (!std::isfinite(c->eta_scale)) return TTT_ERR_ARG;
  // sizes must fit the 32-bit grid and 64-bit offsets comfortably
  const double elems = static_cast<double>(c->B) * c->H * (need_T ? c->T : 1) * c->d;
  if (static_cast<double>(c->B) * c->H > 2147483647.0 || elems > 9.0e15) return TTT_ERR_SHAPE;
  const int hid = c->kind == TTT_MLP ? c->hidden : c->d;
  if (c->chunk <= kMaxChunk && fwd_generic_lds_bytes(c->kind, c->d, hid, c->chunk) > kMaxLds)
    return TTT_ERR_UNSUPPORTED;
  return TTT_OK;
}

int hidden_of(const ttt_config* c) { return c->kind == TTT_MLP ? c->hidden : c->d; }

// Configuration check of the large-chunk SwiGLU layer (ttt_lact_fwd), host only.
ttt_status check_lact(const ttt_config* c) {
  if (!c) return TTT_ERR_NULL;
  if (c->kind != TTT_SWIGLU) return TTT_ERR_UNSUPPORTED;
  if (c->io_dtype != TTT_F32 && c->io_dtype != TTT_BF16) return TTT_ERR_DTYPE;
  if (c->flags & ~(TTT_W0_PER_SEQ | TTT_LACT_READ_BEFORE)) return TTT_ERR_ARG;
  if (c->B < 1 || c->H < 1 || c->T < 1 || c->d < 1 || c->hidden < 1 || c->chunk < 1) return TTT_ERR_SHAPE;
  if (c->T % c->chunk != 0) return TTT_ERR_SHAPE;
  if (!std::isfinite(c->eta_scale)) return TTT_ERR_ARG;
  // one launch holds a block per (head rounded up to 8, up to 1024 tokens of a chunk)
  if (static_cast<double>(c->B) * c->H > (1 << 24)) return TTT_ERR_SHAPE;
  if (!lact_supported(c->d, c->hidden, c->io_dtype, c->chunk)) return TTT_ERR_UNSUPPORTED;
  return TTT_OK;
}

size_t weights_per_head(const ttt_config* c) { return n_weights(c->kind, c->d, hidden_of(c)); }

ScanParams scan_params(const ttt_config* c) {
  ScanParams p{};
  p.kind = c->kind;
  p.B = c->B;
  p.H = c->H;
  p.T = c->T;
  p.d = c->d;
  p.hid = hidden_of(c);
  p.chunk = c->chunk;
  p.io = c->io_dtype;
  p.gelu = c->gelu;
  p.flags = c->flags;
  p.eps = c->ln_eps;
  p.eta_scale = c->eta_scale;
  return p;
}

// The tuned kernels implement the default output rule; TTT_OUTPUT_KEY has its own tuned
// forward (use_key) and otherwise runs on the portable kernels.
bool tuned_allowed(const ttt_config* c) { return !(c->flags & (TTT_FORCE_GENERIC | TTT_OUTPUT_KEY)); }

// Forward with the key-side output rule, MLP d = 64 bf16, chunk a multiple of 16 up to
// kMaxPairChunk: the paired kernel's producer alone, one workgroup per head (any number of heads).
bool use_key(const ttt_config* c) {
  if (c->flags & TTT_FORCE_GENERIC) return false;
  ScanParams p = scan_params(c);
  return fwd_key_supported(p);
}

bool use_mfma(const ttt_config* c) {
  if (!tuned_allowed(c)) return false;
  ScanParams p = scan_params(c);
  return fwd_mfma_supported(p);
}

bool use_pair(const ttt_config* c) {
  if (!tuned_allowed(c) || (c->flags & TTT_ONE_WG_PER_HEAD)) return false;
  ScanParams p = scan_params(c);
  return fwd_pair_supported(p) && static_cast<long long>(c->B) * c->H <= kPairMaxHeads;
}

bool use_split(const ttt_config* c) {
  if (!tuned_allowed(c)) return false;
  ScanParams p = scan_params(c);
  return fwd_split_supported(p);
}

size_t fwd_ws_bytes(const ttt_config* c) {
  if (use_key(c)) return kStatusBytes;
  if (use_pair(c)) return kStatusBytes + fwd_pair_workspace_bytes(c->B * c->H);
  if (use_mfma(c)) return kStatusBytes;
  const size_t generic = static_cast<size_t>(c->B) * c->H * weights_per_head(c) * sizeof(float);
  // the split kernel falls back to the portable one when its grid does not fit the device
  if (use_split(c)) return kStatusBytes + std::max(generic, fwd_split_workspace_bytes(c->B * c->H));
  return kStatusBytes + generic;
}

bool use_bwd_mfma(const ttt_config* c) {
  if (!tuned_allowed(c)) return false;
  BwdParams p{};
  p.kind = c->kind;
  p.d = c->d;
  p.hid = hidden_of(c);
  p.chunk = c->chunk;
  p.io = c->io_dtype;
  return bwd_mfma_supported(p);
}

bool use_decode_stream(const ttt_config* c) {
  if (!tuned_allowed(c)) return false;
  DecodeParams p{};
  p.kind = c->kind;
  p.d = c->d;
  p.hid = hidden_of(c);
  return decode_stream_supported(p);
}

// Four workgroups per head for the decode of the tuned shape, on request.
bool use_decode_split(const ttt_config* c) {
  return use_decode_stream(c) && (c->flags & TTT_DECODE_SPLIT) &&
         static_cast<long>(c->B) * c->H <= kDecodeSplitMaxHeads;
}

size_t decode_ws_bytes(const ttt_config* c) {
  return kStatusBytes + (use_decode_split(c) ? decode_split_workspace_bytes(c->B * c->H) : 0);
}

// The tuned backward over two workgroups per head, unless TTT_ONE_WG_PER_HEAD asks for one
// (host only; at launch the one-workgroup kernel runs instead if the device cannot hold a group
// of eight heads' workgroups at once).
bool use_bwd_split(const ttt_config* c) {
  return use_bwd_mfma(c) && !(c->flags & TTT_ONE_WG_PER_HEAD);
}

// Workspace of the backward: status word, per-head dW (and the portable kernel's chunk
// intermediates), per-head dgamma / dbeta partials, then the split kernel's exchange region.
size_t bwd_ws_base_bytes(const ttt_config* c) {
  const size_t heads = static_cast<size_t>(c->B) * c->H;
  return kStatusBytes +
         heads * bwd_work_floats_per_head(c->kind, c->d, hidden_of(c), c->chunk) * sizeof(float) +
         heads * 2 * c->d * sizeof(float);
}

size_t bwd_ws_bytes(const ttt_config* c) {
  const size_t base = bwd_ws_base_bytes(c);
  if (!use_bwd_split(c)) return base;
  return (base + 255) / 256 * 256 + bwd_split_workspace_bytes(c->B * c->H);
}

ttt_status map_hip(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_ERR_HIP; }

// TTT_DEBUG (an environment variable, set to anything but "" or "0"): every entry point that
// enqueues work waits for it and returns the device-side outcome as its own status:
// TTT_ERR_HIP if the stream reports an error, else TTT_ERR_TIMEOUT or TTT_ERR_NONFINITE from
// the status word, else TTT_OK. Read at every call, so it can be switched while running.
bool debug_mode() {
  const char* e = std::getenv("TTT_DEBUG");
  return e && *e && std::strcmp(e, "0") != 0;
}
ttt_status debug_finish(ttt_status st, const void* status_word, hipStream_t s) {
  if (st != TTT_OK || !debug_mode()) return st;
  if (hipStreamSynchronize(s) != hipSuccess) return TTT_ERR_HIP;
  unsigned word = 0;
  if (hipMemcpy(&word, status_word, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return TTT_ERR_HIP;
  if (word & kStatusTimeout) return TTT_ERR_TIMEOUT;
  return (word & kStatusNonFinite) ? TTT_ERR_NONFINITE : TTT_OK;
}

// Workspace of ttt_scan_fwd_static: a file-scope device array, one per GPU, held until the
// process ends. In host code its name is only a stand-in; the device address of each GPU's
// copy comes from hipGetSymbolAddress, taken once per device (with that device current) on
// the first call there, and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

void* static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int32_t ttt_abi_version(void) { return TTT_ABI_VERSION; }

const char* ttt_status_str(ttt_status s) {
  switch (s) {
    case TTT_OK: return "ok";
    case TTT_ERR_NULL: return "null pointer";
    case TTT_ERR_SHAPE: return "bad shape";
    case TTT_ERR_DTYPE: return "bad dtype";
    case TTT_ERR_UNSUPPORTED: return "unsupported configuration";
    case TTT_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TTT_ERR_WORKSPACE: return "workspace missing or too small";
    case TTT_ERR_HIP: return "HIP runtime error";
    case TTT_ERR_NONFINITE: return "non-finite value seen by a kernel";
    case TTT_ERR_ARG: return "bad argument";
    case TTT_ERR_TIMEOUT: return "a bounded wait between cooperating workgroups expired";
  }
  return "unknown status";
}

ttt_status ttt_validate(const ttt_config* cfg) {
  return (cfg && cfg->kind == TTT_SWIGLU) ? check_lact(cfg) : check_common(cfg, true);
}

ttt_status ttt_lact_fwd(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                        const float* eta, const ttt_swiglu_weights* W0, void* Z,
                        const ttt_swiglu_weights* W_T, void* workspace, size_t ws_bytes,
                        void* stream) {
  ttt_status st = check_lact(cfg);
  if (st != TTT_OK) return st;
  if (!Q || !K || !V || !eta || !W0 || !W0->w1 || !W0->w2 || !W0->w3 || !Z) return TTT_ERR_NULL;
  if (W_T && (!W_T->w1 || !W_T->w2 || !W_T->w3)) return TTT_ERR_NULL;
  const void* ptrs[] = {Q, K, V, eta, W0->w1, W0->w2, W0->w3, Z};
  for (const void* p : ptrs)
    if (!aligned16(p)) return TTT_ERR_ALIGN;
  if (W_T && (!aligned16(W_T->w1) || !aligned16(W_T->w2) || !aligned16(W_T->w3))) return TTT_ERR_ALIGN;
  if (!workspace) return TTT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TTT_ERR_ALIGN;
  if (ws_bytes < kStatusBytes + lact_workspace_bytes(cfg->B * cfg->H)) return TTT_ERR_WORKSPACE;
  LactLaunch L{};
  L.B = cfg->B;
  L.H = cfg->H;
  L.T = cfg->T;
  L.chunk = cfg->chunk;
  L.flags = cfg->flags;
  L.eta_scale = cfg->eta_scale;
  L.Q = Q;
  L.K = K;
  L.V = V;
  L.eta = eta;
  L.w0_1 = W0->w1;
  L.w0_2 = W0->w2;
  L.w0_3 = W0->w3;
  L.Z = Z;
  L.wt_1 = W_T ? W_T->w1 : nullptr;
  L.wt_2 = W_T ? W_T->w2 : nullptr;
  L.wt_3 = W_T ? W_T->w3 : nullptr;
  L.status = static_cast<unsigned*>(workspace);
  L.work = reinterpret_cast<float*>(static_cast<char*>(workspace) + kStatusBytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return debug_finish(map_hip(launch_lact_fwd(L, s)), workspace, s);
}

bool use_mom(const ttt_config* c) {
  if (!tuned_allowed(c)) return false;
  ScanParams p = scan_params(c);
  return fwd_mom_supported(p);
}

size_t fwd_momentum_ws_bytes(const ttt_config* c) {
  const size_t generic = static_cast<size_t>(c->B) * c->H * 2 * weights_per_head(c) * sizeof(float);
  // the tuned kernel falls back to the portable one when its grid does not fit the device
  return kStatusBytes + (use_mom(c) ? std::max(generic, fwd_mom_workspace_bytes(c->B * c->H)) : generic);
}

ttt_status ttt_workspace_size(const ttt_config* cfg, int32_t op, size_t* bytes) {
  if (!bytes) return TTT_ERR_NULL;
  if (op == TTT_OP_LACT) {
    const ttt_status sl = check_lact(cfg);
    if (sl != TTT_OK) return sl;
    *bytes = kStatusBytes + lact_workspace_bytes(cfg->B * cfg->H);
    return TTT_OK;
  }
  const bool need_T = op != TTT_OP_DECODE;
  ttt_status st = check_common(cfg, need_T);
  if (st != TTT_OK) return st;
  switch (op) {
    case TTT_OP_FWD: *bytes = fwd_ws_bytes(cfg); return TTT_OK;
    case TTT_OP_BWD:
      if (cfg->chunk > kMaxChunk) return TTT_ERR_UNSUPPORTED;  // no backward for these
      *bytes = bwd_ws_bytes(cfg);
      return TTT_OK;
    case TTT_OP_DECODE: *bytes = decode_ws_bytes(cfg); return TTT_OK;
    case TTT_OP_FWD_MOMENTUM:
      if (fwd_generic_lds_bytes(cfg->kind, cfg->d, hidden_of(cfg), cfg->chunk, true) > kMaxLds)
        return TTT_ERR_UNSUPPORTED;
      *bytes = fwd_momentum_ws_bytes(cfg);
      return TTT_OK;
    default: return TTT_ERR_ARG;
  }
}

ttt_status ttt_saved_size(const ttt_config* cfg, size_t* bytes) {
  if (!bytes) return TTT_ERR_NULL;
  ttt_status st = check_common(cfg, true);
  if (st != TTT_OK) return st;
  *bytes = static_cast<size_t>(cfg->B) * cfg->H * (cfg->T / cfg->chunk) * weights_per_head(cfg) *
           sizeof(float);
  return TTT_OK;
}

const char* ttt_fwd_kernel_name(const ttt_config* cfg) {
  if (check_common(cfg, true) != TTT_OK) return "";
  if (use_key(cfg)) return "ttt_fwd_mfma_key_d64";
  if (use_pair(cfg)) return "ttt_fwd_mfma_pair_d64";
  if (use_split(cfg)) return "ttt_fwd_mfma_split_d128";
  return use_mfma(cfg) ? "ttt_fwd_mfma_d64" : "ttt_fwd_generic";
}

const char* ttt_fwd_momentum_kernel_name(const ttt_config* cfg) {
  if (check_common(cfg, true) != TTT_OK || (cfg->flags & TTT_OUTPUT_KEY)) return "";
  if (fwd_generic_lds_bytes(cfg->kind, cfg->d, hidden_of(cfg), cfg->chunk, true) > kMaxLds) return "";
  return use_mom(cfg) ? "ttt_fwd_mfma_mom_d64" : "ttt_fwd_generic";
}

const char* ttt_bwd_kernel_name(const ttt_config* cfg) {
  if (check_common(cfg, true) != TTT_OK || cfg->chunk > kMaxChunk) return "";
  if (use_bwd_split(cfg)) return "ttt_bwd_mfma_split_d64";
  return use_bwd_mfma(cfg) ? "ttt_bwd_mfma_d64" : "ttt_bwd_generic";
}

const char* ttt_decode_kernel_name(const ttt_config* cfg) {
  if (check_common(cfg, false) != TTT_OK) return "";
  if (cfg->chunk > kMaxChunk && !use_decode_stream(cfg)) return "";  // not available
  if (use_decode_split(cfg)) return "ttt_decode_split_d64";
  return use_decode_stream(cfg) ? "ttt_decode_stream_d64" : "ttt_decode_generic";
}

// Checks of ttt_scan_fwd's pointers (everything but the workspace), host only.
static ttt_status fwd_check_args(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                                 const float* eta, const float* ln_gamma, const float* ln_beta,
                                 const ttt_weights* W0, const void* Z, const ttt_weights* W_T,
                                 const float* loss, const void* saved) {
  ttt_status st = check_common(cfg, true);
  if (st != TTT_OK) return st;
  const bool mlp = cfg->kind == TTT_MLP;
  if (!Q || !K || !V || !eta || !ln_gamma || !ln_beta || !W0 || !W0->w1 || !Z) return TTT_ERR_NULL;
  if (mlp && !W0->w2) return TTT_ERR_NULL;
  if (W_T && (!W_T->w1 || (mlp && !W_T->w2))) return TTT_ERR_NULL;
  const void* ptrs[] = {Q, K, V, eta, ln_gamma, ln_beta, W0->w1, Z};
  for (const void* p : ptrs)
    if (!aligned16(p)) return TTT_ERR_ALIGN;
  if (mlp && !aligned16(W0->w2)) return TTT_ERR_ALIGN;
  if (W_T && (!aligned16(W_T->w1) || (mlp && !aligned16(W_T->w2)))) return TTT_ERR_ALIGN;
  if ((loss && !aligned16(loss)) || (saved && !aligned16(saved))) return TTT_ERR_ALIGN;
  return TTT_OK;
}

// Enqueues the forward on `workspace` (already checked to be large enough).
static ttt_status fwd_launch(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                             const float* eta, const float* ln_gamma, const float* ln_beta,
                             const ttt_weights* W0, void* Z, const ttt_weights* W_T, float* loss,
                             void* saved, void* workspace, hipStream_t s) {
  const bool mlp = cfg->kind == TTT_MLP;
  ScanParams p = scan_params(cfg);
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.eta = eta;
  p.gamma = ln_gamma;
  p.beta = ln_beta;
  p.w0_1 = W0->w1;
  p.w0_2 = mlp ? W0->w2 : nullptr;
  p.Z = Z;
  p.wt_1 = W_T ? W_T->w1 : nullptr;
  p.wt_2 = (W_T && mlp) ? W_T->w2 : nullptr;
  p.loss = loss;
  p.saved = static_cast<float*>(saved);
  p.status = static_cast<unsigned*>(workspace);
  p.wbuf = reinterpret_cast<float*>(static_cast<char*>(workspace) + kStatusBytes);
  if (use_key(cfg)) return map_hip(launch_fwd_mfma_key(p, s));
  if (use_pair(cfg) && fwd_pair_fits(cfg->B * cfg->H)) return map_hip(launch_fwd_mfma_pair(p, s));
  if (cfg->chunk > kMaxChunk) return TTT_ERR_UNSUPPORTED;  // only the paired kernel takes these
  if (use_split(cfg) && fwd_split_fits(cfg->B * cfg->H)) return map_hip(launch_fwd_mfma_split(p, s));
  return map_hip(use_mfma(cfg) ? launch_fwd_mfma(p, s) : launch_fwd_generic(p, s));
}

ttt_status ttt_scan_fwd(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                        const float* eta, const float* ln_gamma, const float* ln_beta,
                        const ttt_weights* W0, void* Z, const ttt_weights* W_T, float* loss,
                        void* saved, void* workspace, size_t ws_bytes, void* stream) {
  ttt_status st = fwd_check_args(cfg, Q, K, V, eta, ln_gamma, ln_beta, W0, Z, W_T, loss, saved);
  if (st != TTT_OK) return st;
  if (!workspace) return TTT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TTT_ERR_ALIGN;
  if (ws_bytes < fwd_ws_bytes(cfg)) return TTT_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return debug_finish(fwd_launch(cfg, Q, K, V, eta, ln_gamma, ln_beta, W0, Z, W_T, loss, saved, workspace, s),
                      workspace, s);
}

ttt_status ttt_scan_fwd_static(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                               const float* eta, const float* ln_gamma, const float* ln_beta,
                               const ttt_weights* W0, void* Z, const ttt_weights* W_T, float* loss,
                               void* saved, unsigned* status_out, void* stream) {
  ttt_status st = fwd_check_args(cfg, Q, K, V, eta, ln_gamma, ln_beta, W0, Z, W_T, loss, saved);
  if (st != TTT_OK) return st;
  if (status_out && (reinterpret_cast<uintptr_t>(status_out) & 3u) != 0) return TTT_ERR_ALIGN;
  if (fwd_ws_bytes(cfg) > kStaticScratchBytes) return TTT_ERR_WORKSPACE;
  unsigned* ws = static_cast<unsigned*>(static_scratch());
  if (!ws) return TTT_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the array keeps the previous call's contents: the status word starts at zero here, and
  // every kernel that uses the rest of the region clears or initialises what it reads
  if (launch_reset_status(ws, s) != hipSuccess) return TTT_ERR_HIP;
  st = fwd_launch(cfg, Q, K, V, eta, ln_gamma, ln_beta, W0, Z, W_T, loss, saved, ws, s);
  if (st == TTT_OK && status_out) st = map_hip(launch_copy_status(ws, status_out, s));
  return debug_finish(st, ws, s);
}

ttt_status ttt_scan_fwd_momentum(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                                 const float* theta, const float* mom, const float* alpha,
                                 const float* ln_gamma, const float* ln_beta, const ttt_weights* W0,
                                 const ttt_weights* S0, void* Z, const ttt_weights* W_T,
                                 const ttt_weights* S_T, float* loss, void* workspace,
                                 size_t ws_bytes, void* stream) {
  ttt_status st = check_common(cfg, true);
  if (st != TTT_OK) return st;
  if (cfg->flags & TTT_OUTPUT_KEY) return TTT_ERR_UNSUPPORTED;
  if (fwd_generic_lds_bytes(cfg->kind, cfg->d, hidden_of(cfg), cfg->chunk, true) > kMaxLds)
    return TTT_ERR_UNSUPPORTED;
  const bool mlp = cfg->kind == TTT_MLP;
  if (!Q || !K || !V || !theta || !mom || !alpha || !ln_gamma || !ln_beta || !W0 || !W0->w1 || !Z)
    return TTT_ERR_NULL;
  if (mlp && !W0->w2) return TTT_ERR_NULL;
  for (const ttt_weights* w : {S0, W_T, S_T})
    if (w && (!w->w1 || (mlp && !w->w2))) return TTT_ERR_NULL;
  const void* ptrs[] = {Q, K, V, theta, mom, alpha, ln_gamma, ln_beta, W0->w1, Z};
  for (const void* p : ptrs)
    if (!aligned16(p)) return TTT_ERR_ALIGN;
  if (mlp && !aligned16(W0->w2)) return TTT_ERR_ALIGN;
  for (const ttt_weights* w : {S0, W_T, S_T})
    if (w && (!aligned16(w->w1) || (mlp && !aligned16(w->w2)))) return TTT_ERR_ALIGN;
  if (loss && !aligned16(loss)) return TTT_ERR_ALIGN;
  if (!workspace) return TTT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TTT_ERR_ALIGN;
  if (ws_bytes < fwd_momentum_ws_bytes(cfg)) return TTT_ERR_WORKSPACE;

  ScanParams p = scan_params(cfg);
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.eta = theta;
  p.gamma = ln_gamma;
  p.beta = ln_beta;
  p.w0_1 = W0->w1;
  p.w0_2 = mlp ? W0->w2 : nullptr;
  p.Z = Z;
  p.wt_1 = W_T ? W_T->w1 : nullptr;
  p.wt_2 = (W_T && mlp) ? W_T->w2 : nullptr;
  p.loss = loss;
  p.saved = nullptr;
  p.status = static_cast<unsigned*>(workspace);
  p.wbuf = reinterpret_cast<float*>(static_cast<char*>(workspace) + kStatusBytes);
  p.mom = mom;
  p.alpha = alpha;
  p.s0_1 = S0 ? S0->w1 : nullptr;
  p.s0_2 = (S0 && mlp) ? S0->w2 : nullptr;
  p.st_1 = S_T ? S_T->w1 : nullptr;
  p.st_2 = (S_T && mlp) ? S_T->w2 : nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_mom(cfg) && fwd_mom_fits()) return debug_finish(map_hip(launch_fwd_mfma_mom(p, s)), workspace, s);
  return debug_finish(map_hip(launch_fwd_generic(p, s)), workspace, s);
}

ttt_status ttt_scan_bwd(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                        const float* eta, const float* ln_gamma, const float* ln_beta,
                        const void* saved, const void* dZ, const ttt_weights* dW_T, void* dQ,
                        void* dK, void* dV, float* deta, const ttt_weights* dW0, float* dgamma,
                        float* dbeta, void* workspace, size_t ws_bytes, void* stream) {
  ttt_status st = check_common(cfg, true);
  if (st != TTT_OK) return st;
  if (cfg->chunk > kMaxChunk) return TTT_ERR_UNSUPPORTED;  // no backward for these
  const bool mlp = cfg->kind == TTT_MLP;
  if (!Q || !K || !V || !eta || !ln_gamma || !ln_beta || !saved || !dZ || !dQ || !dK || !dV ||
      !deta || !dW0 || !dW0->w1)
    return TTT_ERR_NULL;
  if (mlp && !dW0->w2) return TTT_ERR_NULL;
  if (dW_T && (!dW_T->w1 || (mlp && !dW_T->w2))) return TTT_ERR_NULL;
  const void* ptrs[] = {Q, K, V, eta, ln_gamma, ln_beta, saved, dZ, dQ, dK, dV, deta, dW0->w1};
  for (const void* p : ptrs)
    if (!aligned16(p)) return TTT_ERR_ALIGN;
  if (mlp && !aligned16(dW0->w2)) return TTT_ERR_ALIGN;
  if (dW_T && (!aligned16(dW_T->w1) || (mlp && !aligned16(dW_T->w2)))) return TTT_ERR_ALIGN;
  if ((dgamma && !aligned16(dgamma)) || (dbeta && !aligned16(dbeta))) return TTT_ERR_ALIGN;
  if (!workspace) return TTT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TTT_ERR_ALIGN;
  if (ws_bytes < bwd_ws_bytes(cfg)) return TTT_ERR_WORKSPACE;
  const bool tuned = use_bwd_mfma(cfg);
  if (!tuned && bwd_generic_lds_bytes(cfg->kind, cfg->d, hidden_of(cfg), cfg->chunk) > kMaxLds)
    return TTT_ERR_UNSUPPORTED;

  BwdParams p{};
  p.kind = cfg->kind;
  p.B = cfg->B;
  p.H = cfg->H;
  p.T = cfg->T;
  p.d = cfg->d;
  p.hid = hidden_of(cfg);
  p.chunk = cfg->chunk;
  p.io = cfg->io_dtype;
  p.gelu = cfg->gelu;
  p.flags = cfg->flags;
  p.eps = cfg->ln_eps;
  p.eta_scale = cfg->eta_scale;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.eta = eta;
  p.gamma = ln_gamma;
  p.beta = ln_beta;
  p.saved = static_cast<const float*>(saved);
  p.dZ = dZ;
  p.dwt_1 = dW_T ? dW_T->w1 : nullptr;
  p.dwt_2 = (dW_T && mlp) ? dW_T->w2 : nullptr;
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.deta = deta;
  p.dw0_1 = dW0->w1;
  p.dw0_2 = mlp ? dW0->w2 : nullptr;
  p.dgamma = dgamma;
  p.dbeta = dbeta;
  p.status = static_cast<unsigned*>(workspace);
  const size_t heads = static_cast<size_t>(cfg->B) * cfg->H;
  p.work = reinterpret_cast<float*>(static_cast<char*>(workspace) + kStatusBytes);
  p.dgb = p.work + heads * bwd_work_floats_per_head(cfg->kind, cfg->d, p.hid, cfg->chunk);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (use_bwd_split(cfg) && bwd_split_fits()) {
    float* xbuf = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           (bwd_ws_base_bytes(cfg) + 255) / 256 * 256);
    e = launch_bwd_mfma_split(p, xbuf, s);
  } else {
    e = tuned ? launch_bwd_mfma(p, s) : launch_bwd_generic(p, s);
  }
  if (e != hipSuccess) return TTT_ERR_HIP;
  return debug_finish(map_hip(launch_bwd_finalize(p, s)), workspace, s);
}

ttt_status ttt_decode_step(const ttt_config* cfg, const void* q, const void* k, const void* v,
                           const float* eta, const float* ln_gamma, const float* ln_beta,
                           const ttt_weights* W_start, const ttt_weights* acc,
                           int32_t pos_in_chunk, void* z, void* workspace, size_t ws_bytes,
                           void* stream) {
  ttt_status st = check_common(cfg, false);
  if (st != TTT_OK) return st;
  if (cfg->chunk > kMaxChunk && !use_decode_stream(cfg)) return TTT_ERR_UNSUPPORTED;
  const bool mlp = cfg->kind == TTT_MLP;
  if (!q || !k || !v || !eta || !ln_gamma || !ln_beta || !W_start || !acc || !z ||
      !W_start->w1 || !acc->w1)
    return TTT_ERR_NULL;
  if (mlp && (!W_start->w2 || !acc->w2)) return TTT_ERR_NULL;
  if (pos_in_chunk < 0 || pos_in_chunk >= cfg->chunk) return TTT_ERR_ARG;
  const void* ptrs[] = {q, k, v, eta, ln_gamma, ln_beta, W_start->w1, acc->w1, z};
  for (const void* p : ptrs)
    if (!aligned16(p)) return TTT_ERR_ALIGN;
  if (mlp && (!aligned16(W_start->w2) || !aligned16(acc->w2))) return TTT_ERR_ALIGN;
  if (!workspace) return TTT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TTT_ERR_ALIGN;
  if (ws_bytes < decode_ws_bytes(cfg)) return TTT_ERR_WORKSPACE;
  DecodeParams p{};
  p.kind = cfg->kind;
  p.B = cfg->B;
  p.H = cfg->H;
  p.d = cfg->d;
  p.hid = hidden_of(cfg);
  p.chunk = cfg->chunk;
  p.io = cfg->io_dtype;
  p.gelu = cfg->gelu;
  p.flags = cfg->flags;
  p.pos = pos_in_chunk;
  p.eps = cfg->ln_eps;
  p.eta_scale = cfg->eta_scale;
  p.q = q;
  p.k = k;
  p.v = v;
  p.eta = eta;
  p.gamma = ln_gamma;
  p.beta = ln_beta;
  p.ws_1 = W_start->w1;
  p.ws_2 = mlp ? W_start->w2 : nullptr;
  p.acc_1 = acc->w1;
  p.acc_2 = mlp ? acc->w2 : nullptr;
  p.z = z;
  p.status = static_cast<unsigned*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_decode_split(cfg))
    return debug_finish(map_hip(launch_decode_split(p, static_cast<char*>(workspace) + kStatusBytes, s)), workspace, s);
  return debug_finish(map_hip(use_decode_stream(cfg) ? launch_decode_stream(p, s) : launch_decode(p, s)), workspace, s);
}

ttt_status ttt_read_status(const void* workspace, void* stream) {
  if (!workspace) return TTT_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return TTT_ERR_HIP;
  unsigned word = 0;
  if (hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
    return TTT_ERR_HIP;
  if (word & kStatusTimeout) return TTT_ERR_TIMEOUT;
  return (word & kStatusNonFinite) ? TTT_ERR_NONFINITE : TTT_OK;
}

ttt_status ttt_reset_status(void* workspace, void* stream) {
  if (!workspace) return TTT_ERR_NULL;
  return map_hip(launch_reset_status(static_cast<unsigned*>(workspace),
                                     static_cast<hipStream_t>(stream)));
}

}  // extern "C"
