/*
 * ttt.h -- C ABI of libttt.so, the MI355X (gfx950) TTT inner-loop scan.
 *
 * The operation (per independent (batch, head) pair) is the mini-batch test-time
 * training scan of a TTT-Linear or TTT-MLP fast-weight layer, as defined on the page
 * "Test-Time Training(TTT)과 LLM 메모리" (juhoplayground), section "TTT layer"
 * (update Eq. 2, loss Eq. 4, output Eq. 5, TTT-Linear / TTT-MLP, mini-batch b = 16,
 * dual form, learnable W0 and eta), with the stabilising form f(x) = x + LN(f_res(x))
 * from section "재현성과 공개 구현" of the same page, and the mini-batch rule of
 * "LLM : 빠른 논문 리뷰 : End-to-End Test-Time Training for Long Context"
 * (aiflower), section 2.3, Eq. 5 (all gradients of a mini-batch taken at the weights
 * the mini-batch starts from; weights carried into the next mini-batch):
 *
 *   g(x;W) = GELU(x W1) W2   (MLP: W1 [d, hidden], W2 [hidden, d], hidden = 4d)
 *   g(x;W) = x W             (Linear: W [d, d])
 *   f(x;W) = x + LN(g(x;W)),  LN(z) = gamma * (z - mean) / sqrt(var + eps) + beta
 *   l_t(W) = || f(K_t;W) - V_t ||^2
 *   in chunk i, for token t:  W_t = W_start - eta_scale * sum_{s in chunk, s <= t} eta_s grad l_s(W_start)
 *                             z_t = f(Q_t; W_t);   W carried = W at the chunk's last token.
 *
 * Row-vector convention. All arithmetic on the weights is fp32 on the device.
 *
 * Conventions shared by every entry point:
 *  - Pointers to tensors are DEVICE pointers; all tensors are dense and row-major
 *    (last axis fastest). Q, K, V, Z (and dQ, dK, dV, dZ) are [B, H, T, d] in the
 *    I/O dtype (fp32 or bf16); eta is [B, H, T] fp32; gamma, beta are [H, d] fp32;
 *    fast weights are fp32: W0 is [H, ...] shared over B, or [B, H, ...] with
 *    TTT_W0_PER_SEQ; W_T is always [B, H, ...].
 *  - Ownership: the caller allocates and frees every buffer (tensors and
 *    workspace). The library never allocates device memory and keeps no pointer
 *    after a call returns.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = default stream).
 *    Every call only enqueues work on it and returns; nothing synchronises the
 *    stream except ttt_read_status, and the debug mode below.
 *  - Errors: every argument, shape, dtype, alignment (16 bytes) and workspace check
 *    runs on the host before anything is enqueued, so a non-OK return means nothing
 *    ran. A failed launch returns TTT_ERR_HIP. A non-finite loss or output detected
 *    inside a kernel is OR-ed into a status word in the workspace (sticky until
 *    ttt_reset_status); ttt_read_status reports it as TTT_ERR_NONFINITE. The forward
 *    kernels whose workgroups wait for each other (the paired d = 64 kernel, two
 *    workgroups per head; the split d = 128 kernel, four) bound every wait; an expired
 *    wait sets TTT_ERR_TIMEOUT in the same word (the outputs of that call are then
 *    undefined).
 *  - Debug mode: with the environment variable TTT_DEBUG set (to anything but "" or
 *    "0"; read at every call), each entry point that enqueues work then synchronises
 *    its stream and returns the device-side outcome itself: TTT_ERR_HIP if the stream
 *    reports an error, else TTT_ERR_TIMEOUT or TTT_ERR_NONFINITE from the status word
 *    (which stays set as usual), else TTT_OK.
 *  - No C++ exception crosses this interface. Calls that share a workspace must be
 *    ordered on one stream.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 1

typedef enum {
  TTT_OK = 0,
  TTT_ERR_NULL = 1,        /* a required pointer is NULL                            */
  TTT_ERR_SHAPE = 2,       /* non-positive size, T not a multiple of chunk, ...     */
  TTT_ERR_DTYPE = 3,       /* unknown io_dtype                                      */
  TTT_ERR_UNSUPPORTED = 4, /* a combination no kernel is built for                  */
  TTT_ERR_ALIGN = 5,       /* a tensor pointer is not 16-byte aligned               */
  TTT_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than ttt_workspace_size     */
  TTT_ERR_HIP = 7,         /* a HIP runtime call failed                             */
  TTT_ERR_NONFINITE = 8,   /* a kernel saw a NaN/Inf loss or output                 */
  TTT_ERR_ARG = 9,         /* any other bad argument (unknown op, pos_in_chunk ...) */
  TTT_ERR_TIMEOUT = 10     /* a bounded wait between cooperating workgroups expired */
} ttt_status;

/* TTT_SWIGLU: the large-chunk SwiGLU layer of ttt_lact_fwd (no other entry point takes it) */
enum { TTT_LINEAR = 0, TTT_MLP = 1, TTT_SWIGLU = 2 };
enum { TTT_F32 = 0, TTT_BF16 = 1 };
enum { TTT_GELU_ERF = 0, TTT_GELU_TANH = 1 };
/* ttt_config.flags */
enum {
  TTT_W0_PER_SEQ = 1 << 0,    /* W0 (and dW0) are [B, H, ...] instead of [H, ...]         */
  TTT_FORCE_GENERIC = 1 << 1, /* use the portable fp32 kernel even where a tuned one exists */
  TTT_ONE_WG_PER_HEAD = 1 << 2, /* tuned forward: one workgroup per (batch, head) instead of a
                                   producer/consumer pair of workgroups                      */
  TTT_OUTPUT_KEY = 1 << 3, /* output rule of Eq. 9 in the E2E paper review, section 2.4.2:
                             z_t = f(K_t; W) with W the weights the token's gradient is taken at
                             (the chunk start; W_{t-1} when chunk = 1), i.e. the key-side
                             prediction reused as the output. Q does not enter it (dQ = 0). The
                             forward of MLP d = 64, hidden 256, bf16 (chunk 16, or a multiple of
                             16 up to 1024) runs it on a tuned kernel (the paired kernel's
                             producer alone, one workgroup per head); backward and decode (chunk
                             up to 16) and every other shape run it on the portable kernels. */
  TTT_FORCE_DEVICE_SCOPE = 1 << 4 /* tuned kernels with several workgroups per head (forward,
                                     momentum forward, decode): they hand partial results
                                     to each other with device-scope atomics and fences even
                                     when they share an XCD (slower). This is the path taken when
                                     they do not; the flag lets a test run it. */,
  TTT_DECODE_SPLIT = 1 << 5, /* decode, MLP d = 64: four workgroups per (batch, head), split by
                               hidden units, instead of one (at most 128 heads). Measured slower
                               than one workgroup per head at every head count tried (12-120);
                               kept as the alternative the library can run and test. */
  TTT_LACT_READ_BEFORE = 1 << 6 /* ttt_lact_fwd only: a chunk's tokens are read out with the
                                   weights the chunk started from instead of the updated ones */
};
/* op codes for ttt_workspace_size */
enum { TTT_OP_FWD = 0, TTT_OP_BWD = 1, TTT_OP_DECODE = 2, TTT_OP_FWD_MOMENTUM = 3, TTT_OP_LACT = 4 };

typedef struct {
  int32_t kind;      /* TTT_LINEAR or TTT_MLP                                         */
  int32_t B, H, T;   /* batch, heads, tokens (T ignored by ttt_decode_step)           */
  int32_t d;         /* head dimension: 16 <= d <= 128, multiple of 16                */
  int32_t hidden;    /* MLP hidden width, must be 4*d; ignored for TTT_LINEAR         */
  int32_t chunk;     /* mini-batch size b, 1 <= b <= 16; T % b == 0 for scans          */
  int32_t io_dtype;  /* TTT_F32 or TTT_BF16 for Q, K, V, Z, dQ, dK, dV, dZ             */
  int32_t gelu;      /* TTT_GELU_ERF (exact) or TTT_GELU_TANH                          */
  int32_t flags;     /* TTT_W0_PER_SEQ | TTT_FORCE_GENERIC | TTT_ONE_WG_PER_HEAD |
                        TTT_OUTPUT_KEY | TTT_FORCE_DEVICE_SCOPE | TTT_DECODE_SPLIT    */
  float ln_eps;      /* LayerNorm epsilon inside the square root (e.g. 1e-6)           */
  float eta_scale;   /* multiplies every eta_t (1 = plain sum; 1/b = averaged sum)     */
} ttt_config;

/* Fast weights, fp32 device pointers. MLP: w1 [.., d, hidden], w2 [.., hidden, d].
 * Linear: w1 [.., d, d], w2 unused (may be NULL). */
typedef struct {
  float* w1;
  float* w2;
} ttt_weights;

/* SwiGLU fast weights of ttt_lact_fwd, fp32 device pointers: w1, w3 [.., d, hidden],
 * w2 [.., hidden, d]. */
typedef struct {
  float* w1;
  float* w2;
  float* w3;
} ttt_swiglu_weights;

/* Host-only check of a configuration (no HIP call). */
ttt_status ttt_validate(const ttt_config* cfg);

/* Bytes of workspace the op needs (TTT_OP_FWD / TTT_OP_BWD / TTT_OP_DECODE /
 * TTT_OP_FWD_MOMENTUM / TTT_OP_LACT; the last one with a TTT_SWIGLU config).
 * Host only. The first 256 bytes of every workspace hold the status word; the
 * caller zero-fills a new workspace once (or calls ttt_reset_status). */
ttt_status ttt_workspace_size(const ttt_config* cfg, int32_t op, size_t* bytes);

/* Bytes of the `saved` buffer ttt_scan_fwd fills for ttt_scan_bwd: the fp32 fast
 * weights at the start of every chunk, [B, H, T/chunk, weights]. Host only. */
ttt_status ttt_saved_size(const ttt_config* cfg, size_t* bytes);

/* Forward scan over T tokens for every (batch, head).
 *  Q, K, V [B,H,T,d] io dtype; eta [B,H,T]; ln_gamma, ln_beta [H,d]; W0 as above.
 *  Z [B,H,T,d] io dtype (written).
 *  W_T   (nullable): final weights, [B,H,...] (written).
 *  loss  (nullable): [B,H,T] fp32, l_t at the chunk-start weights (written).
 *  saved (nullable): ttt_saved_size bytes, needed by ttt_scan_bwd (written).
 *  Definition: the page "Test-Time Training(TTT)과 LLM 메모리", section "TTT layer",
 *  Eq. 2/4/5 with mini-batches as in the E2E paper review, section 2.3, Eq. 5. */
ttt_status ttt_scan_fwd(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                        const float* eta, const float* ln_gamma, const float* ln_beta,
                        const ttt_weights* W0, void* Z, const ttt_weights* W_T, float* loss,
                        void* saved, void* workspace, size_t ws_bytes, void* stream);

/* Allocation-free variant of ttt_scan_fwd, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, kernels and results are those of ttt_scan_fwd, except that the workspace is a
 * device array inside the library: 16 MiB on each GPU the library runs on, held until the
 * process ends. A configuration whose ttt_workspace_size(TTT_OP_FWD) exceeds 16 MiB returns
 * TTT_ERR_WORKSPACE before anything is enqueued (the paired d = 64 kernel needs 108 KiB per
 * (batch, head), so all of its up to 128 heads fit; the portable kernel needs the fp32
 * weights of every head).
 *  status_out (nullable, 4-byte aligned device pointer): receives the call's status word on
 *  the stream after the scan: 0, or bit 0 = a kernel saw a NaN/Inf, bit 1 = a bounded wait
 *  between cooperating workgroups expired (the meanings ttt_read_status reports).
 * Every call on one GPU shares that GPU's array and the array keeps the last call's
 * contents (each call clears what it needs cleared): calls that overlap on one GPU (other
 * streams, other threads) race, so the caller orders them. No call allocates or frees
 * device memory. */
ttt_status ttt_scan_fwd_static(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                               const float* eta, const float* ln_gamma, const float* ln_beta,
                               const ttt_weights* W0, void* Z, const ttt_weights* W_T, float* loss,
                               void* saved, unsigned* status_out, void* stream);

/* Forward scan with momentum and a forget gate: the page "Test-Time Training(TTT)과 LLM
 * 메모리", section "Titans와 Miras", Eq. 14 (S_t = mom_t S_{t-1} - theta_t grad l(M_{t-1}; x_t))
 * and Eq. 13 (M_t = (1 - alpha_t) M_{t-1} + S_t), with the loss, f and output of
 * ttt_scan_fwd and its mini-batch rule (inside a chunk every gradient is taken at the
 * memory the chunk started from; chunk = 1 is the per-token rule as written).
 *  theta [B,H,T] fp32: step size per token (times cfg->eta_scale); mom [B,H,T] fp32:
 *  momentum decay; alpha [B,H,T] fp32: forget gate (0 keeps, 1 resets). Any real values
 *  are accepted; the pages give (0, 1) for alpha.
 *  W0: initial memory, shaped as for ttt_scan_fwd. S0 (nullable = zero): momentum carried
 *  in, always per sequence [B,H,...]. W_T, S_T (nullable): final memory and momentum,
 *  [B,H,...] (written). Z, loss: as for ttt_scan_fwd.
 *  Kernels: for MLP, d = 64, hidden = 256, chunk 16, bf16 I/O a tuned bf16 MFMA kernel that
 *  splits each head over two workgroups (the memory and the momentum in registers, bounded
 *  waits between the two as in the split d = 128 forward, TTT_ERR_TIMEOUT on expiry);
 *  every other supported shape (and TTT_FORCE_GENERIC) runs the portable fp32 kernel.
 *  TTT_OUTPUT_KEY is rejected (TTT_ERR_UNSUPPORTED); there is no saved state and no
 *  backward for this variant. Workspace: ttt_workspace_size(.., TTT_OP_FWD_MOMENTUM, ..)
 *  bytes. Errors as for ttt_scan_fwd. */
ttt_status ttt_scan_fwd_momentum(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                                 const float* theta, const float* mom, const float* alpha,
                                 const float* ln_gamma, const float* ln_beta, const ttt_weights* W0,
                                 const ttt_weights* S0, void* Z, const ttt_weights* W_T,
                                 const ttt_weights* S_T, float* loss, void* workspace,
                                 size_t ws_bytes, void* stream);

/* Outer-loop backward through the scan (gradients of gradients, the outer loop of
 * the E2E paper review, section 2.2): given dZ [B,H,T,d] (io dtype) and optionally
 * dW_T ([B,H,...] fp32, nullable = zero), writes dQ, dK, dV [B,H,T,d] (io dtype),
 * deta [B,H,T] fp32 and dW0 (fp32, shaped like W0; summed over B unless
 * TTT_W0_PER_SEQ). dgamma, dbeta ([H,d] fp32, summed over B) are nullable.
 * `saved` must come from ttt_scan_fwd on the same inputs and config. */
ttt_status ttt_scan_bwd(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                        const float* eta, const float* ln_gamma, const float* ln_beta,
                        const void* saved, const void* dZ, const ttt_weights* dW_T, void* dQ,
                        void* dK, void* dV, float* deta, const ttt_weights* dW0, float* dgamma,
                        float* dbeta, void* workspace, size_t ws_bytes, void* stream);

/* One decode token per (batch, head) (the E2E paper review, section 2.3.2: a
 * gradient step is committed only when the decoded tokens fill a mini-batch).
 *  q, k, v [B,H,d] io dtype; eta [B,H] fp32; ln_gamma, ln_beta [H,d].
 *  W_start [B,H,...] fp32 in/out: weights at the start of the current chunk.
 *  acc     [B,H,...] fp32 in/out: eta_scale * sum of eta_s grad l_s(W_start) over the
 *          chunk's tokens so far (caller zero-fills it at a chunk start).
 *  pos_in_chunk: 0..chunk-1, tracked by the caller. At pos_in_chunk == chunk-1 the
 *          step commits: W_start -= acc and acc = 0.
 *  z [B,H,d] io dtype (written) = f(q; W_start - acc), acc including this token.
 *  A scan of T tokens followed by decode steps equals a scan of the longer sequence.
 *  workspace: ttt_workspace_size(.., TTT_OP_DECODE, ..) bytes, zero-filled before its first
 *          use. For the four-workgroup kernel (TTT_DECODE_SPLIT) it holds, after the status
 *          word, an exchange area per head that every call leaves zero; after TTT_ERR_TIMEOUT
 *          zero-fill it again. Calls that overlap on one workspace race. */
ttt_status ttt_decode_step(const ttt_config* cfg, const void* q, const void* k, const void* v,
                           const float* eta, const float* ln_gamma, const float* ln_beta,
                           const ttt_weights* W_start, const ttt_weights* acc,
                           int32_t pos_in_chunk, void* z, void* workspace, size_t ws_bytes,
                           void* stream);

/* The large-chunk SwiGLU TTT layer ("Test-Time Training(TTT)과 LLM 메모리", section "LaCT"):
 *   f_W(x) = (SiLU(x W1) * (x W3)) W2                          (Eq. 6, row vectors)
 *   chunk of b tokens: g = eta_scale * sum_t eta_t grad_W (-f_W(K_t) . V_t) at the chunk-start
 *                      W (Eq. 7 and 4);  W <- L2-Normalize(W - g)  (Eq. 8)
 *   z_t = f_W(Q_t)  (Eq. 2) with the weights after the chunk's update (TTT_LACT_READ_BEFORE:
 *                      with the chunk-start weights).
 * L2-Normalize scales every output unit's weight vector to unit norm: each column of W1 and
 * W3 (over d) and each column of W2 (over hidden); W0 itself is used as given.
 *  cfg: kind TTT_SWIGLU, d = 64, hidden = 256, io TTT_BF16, chunk a multiple of 64 that
 *       divides T; flags from TTT_W0_PER_SEQ | TTT_LACT_READ_BEFORE; ln_eps and gelu ignored
 *       (anything else: TTT_ERR_UNSUPPORTED or TTT_ERR_ARG).
 *  Q, K, V, Z [B,H,T,d] bf16; eta [B,H,T] fp32; W0 [H,..] or [B,H,..] (TTT_W0_PER_SEQ);
 *  W_T (nullable) [B,H,..], the weights after the last chunk.
 *  workspace: ttt_workspace_size(.., TTT_OP_LACT, ..) bytes (status word, then two weight
 *  buffers and the W2 column sums of every head, about 385 KiB per (batch, head)).
 *  Runs one launch per chunk plus one of the kernel
 *  "ttt_lact_fwd_d64" (bf16 MFMA products, fp32 weights and sums); the W_T copy-out joins the
 *  last launch (with TTT_LACT_READ_BEFORE it takes one more). Errors as for ttt_scan_fwd;
 *  a non-finite weight norm sets TTT_ERR_NONFINITE in the status word. */
ttt_status ttt_lact_fwd(const ttt_config* cfg, const void* Q, const void* K, const void* V,
                        const float* eta, const ttt_swiglu_weights* W0, void* Z,
                        const ttt_swiglu_weights* W_T, void* workspace, size_t ws_bytes,
                        void* stream);

/* Synchronises `stream`, then reads the workspace status word: TTT_OK,
 * TTT_ERR_TIMEOUT if a forward launch of cooperating workgroups (the paired d = 64 or the
 * split d = 128 kernel) since the last reset had a wait expire,
 * else TTT_ERR_NONFINITE if any kernel since the last reset saw a NaN/Inf. */
ttt_status ttt_read_status(const void* workspace, void* stream);

/* Enqueues a zero-fill of the workspace status word on `stream`. */
ttt_status ttt_reset_status(void* workspace, void* stream);

/* Name of the kernel variant ttt_scan_fwd would launch for cfg ("" if invalid). Host
 * only: "ttt_fwd_mfma_pair_d64" is chosen for the tuned shape when B*H <= 128 and
 * TTT_ONE_WG_PER_HEAD is not set; if the device then cannot hold all 2*ceil(B*H/8)*8
 * workgroups at once, ttt_scan_fwd launches "ttt_fwd_mfma_d64" instead. With TTT_OUTPUT_KEY the
 * tuned shape (chunk a multiple of 16 up to 1024) takes "ttt_fwd_mfma_key_d64" (one workgroup
 * per head, any head count, workspace: the status word only). For MLP d = 128,
 * hidden = 512, chunk 16, bf16 I/O the name is "ttt_fwd_mfma_split_d128" (four workgroups per
 * head that wait for each other); ttt_scan_fwd launches it once per group of heads whose
 * workgroups the device holds at once (64 heads on a 256-CU device), and launches
 * "ttt_fwd_generic" instead only if not even eight heads fit. */
const char* ttt_fwd_kernel_name(const ttt_config* cfg);

/* Name of the kernel variant ttt_scan_fwd_momentum would launch for cfg ("" if invalid):
 * "ttt_fwd_mfma_mom_d64" for the tuned shape (the portable kernel runs instead if the device
 * cannot hold a group of eight heads' workgroups at once), else "ttt_fwd_generic". Host only. */
const char* ttt_fwd_momentum_kernel_name(const ttt_config* cfg);

/* Name of the kernel variant ttt_scan_bwd would launch for cfg ("" if invalid). Host only. */
const char* ttt_bwd_kernel_name(const ttt_config* cfg);

/* Name of the kernel variant ttt_decode_step would launch for cfg ("" if invalid). Host
 * only: for MLP d = 64, hidden = 256 "ttt_decode_stream_d64" (one workgroup per head), or
 * "ttt_decode_split_d64" (four workgroups per head) with TTT_DECODE_SPLIT when B*H <= 128;
 * "ttt_decode_generic" for every other shape or with TTT_FORCE_GENERIC. */
const char* ttt_decode_kernel_name(const ttt_config* cfg);

const char* ttt_status_str(ttt_status s);
int32_t ttt_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H_ */
