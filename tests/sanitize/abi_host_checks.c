/* Host-side checks of libttt's C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitize.py). Every call here is rejected by host validation before anything is
 * enqueued, so no GPU is needed: fake, aligned device addresses stand in for tensors. Exits 0
 * when every return code is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/ttt.h"

static int failures = 0;
#define EXPECT(call, code)                                                            \
  do {                                                                                \
    int got_ = (int)(call);                                                           \
    if (got_ != (code)) {                                                             \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
              got_, (code));                                                          \
      ++failures;                                                                     \
    }                                                                                 \
  } while (0)

static ttt_config mlp_d64(void) {
  ttt_config c;
  memset(&c, 0, sizeof c);
  c.kind = TTT_MLP; c.B = 8; c.H = 12; c.T = 8192; c.d = 64; c.hidden = 256; c.chunk = 16;
  c.io_dtype = TTT_BF16; c.gelu = TTT_GELU_ERF; c.flags = 0; c.ln_eps = 1e-6f; c.eta_scale = 1.0f;
  return c;
}

#define P(x) ((void*)(uintptr_t)(x))

int main(void) {
  ttt_config c = mlp_d64();
  size_t n = 0;
  EXPECT(ttt_abi_version(), TTT_ABI_VERSION);
  EXPECT(ttt_validate(NULL), TTT_ERR_NULL);
  EXPECT(ttt_validate(&c), TTT_OK);
  for (int s = 0; s <= 11; ++s)
    if (ttt_status_str((ttt_status)s) == NULL) ++failures;
  EXPECT(ttt_workspace_size(&c, TTT_OP_FWD, NULL), TTT_ERR_NULL);
  EXPECT(ttt_workspace_size(&c, TTT_OP_FWD, &n), TTT_OK);
  EXPECT(ttt_workspace_size(&c, 99, &n), TTT_ERR_ARG);
  EXPECT(ttt_saved_size(&c, &n), TTT_OK);
  if (n != (size_t)8 * 12 * 512 * 2 * 64 * 256 * 4) ++failures;
  /* shapes and enums */
  ttt_config b = c; b.T = 8200; EXPECT(ttt_validate(&b), TTT_ERR_SHAPE);
  b = c; b.B = 0; EXPECT(ttt_validate(&b), TTT_ERR_SHAPE);
  b = c; b.B = 1 << 20; b.H = 1 << 20; EXPECT(ttt_validate(&b), TTT_ERR_SHAPE);  /* B*H overflows int */
  b = c; b.d = 40; b.hidden = 160; EXPECT(ttt_validate(&b), TTT_ERR_UNSUPPORTED);
  b = c; b.chunk = 24; EXPECT(ttt_validate(&b), TTT_ERR_UNSUPPORTED);
  b = c; b.chunk = 1024; EXPECT(ttt_validate(&b), TTT_OK);
  b = c; b.chunk = 2048; EXPECT(ttt_validate(&b), TTT_ERR_UNSUPPORTED);
  b = c; b.io_dtype = 7; EXPECT(ttt_validate(&b), TTT_ERR_DTYPE);
  b = c; b.flags = 1 << 30; EXPECT(ttt_validate(&b), TTT_ERR_ARG);
  b = c; b.ln_eps = -1.0f; EXPECT(ttt_validate(&b), TTT_ERR_ARG);
  /* kernel names (host only) */
  if (strcmp(ttt_fwd_kernel_name(&c), "ttt_fwd_mfma_pair_d64") != 0) ++failures;
  b = c; b.T = 7; if (strcmp(ttt_fwd_kernel_name(&b), "") != 0) ++failures;
  if (strcmp(ttt_bwd_kernel_name(&c), "ttt_bwd_mfma_split_d64") != 0) ++failures;
  b = c; b.flags = TTT_ONE_WG_PER_HEAD;
  if (strcmp(ttt_bwd_kernel_name(&b), "ttt_bwd_mfma_d64") != 0) ++failures;
  if (strcmp(ttt_decode_kernel_name(&c), "ttt_decode_stream_d64") != 0) ++failures;
  b = c; b.flags = TTT_DECODE_SPLIT;
  if (strcmp(ttt_decode_kernel_name(&b), "ttt_decode_split_d64") != 0) ++failures;
  /* forward: null, alignment, workspace */
  ttt_weights w = {(float*)P(0x10000), (float*)P(0x20000)};
  ttt_weights w_bad = {(float*)P(0x10000), NULL};
  EXPECT(ttt_scan_fwd(&c, NULL, P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), &w, P(0x80000),
                      NULL, NULL, NULL, P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_NULL);
  EXPECT(ttt_scan_fwd(&c, P(0x1000), P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), &w_bad,
                      P(0x80000), NULL, NULL, NULL, P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_NULL);
  EXPECT(ttt_scan_fwd(&c, P(0x1008), P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), &w,
                      P(0x80000), NULL, NULL, NULL, P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_ALIGN);
  EXPECT(ttt_scan_fwd(&c, P(0x1000), P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), &w,
                      P(0x80000), NULL, NULL, NULL, P(0x90000), 16, NULL), TTT_ERR_WORKSPACE);
  EXPECT(ttt_scan_fwd(&c, P(0x1000), P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), &w,
                      P(0x80000), NULL, NULL, NULL, NULL, (size_t)1 << 40, NULL), TTT_ERR_WORKSPACE);
  /* allocation-free forward: the size limit and the status word's alignment */
  ttt_config big = c; big.kind = TTT_MLP; big.B = 1; big.H = 32; big.T = 64; big.d = 128; big.hidden = 512;
  EXPECT(ttt_scan_fwd_static(&big, P(0x1000), P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), &w,
                             P(0x80000), NULL, NULL, NULL, NULL, NULL), TTT_ERR_WORKSPACE);
  EXPECT(ttt_scan_fwd_static(&c, P(0x1000), P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), &w,
                             P(0x80000), NULL, NULL, NULL, (unsigned*)P(0x90002), NULL), TTT_ERR_ALIGN);
  /* backward: missing saved buffer; larger mini-batches have no backward */
  EXPECT(ttt_scan_bwd(&c, P(0x1000), P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), NULL,
                      P(0x40000), NULL, P(0x50000), P(0x60000), P(0x70000), (float*)P(0x71000), &w,
                      NULL, NULL, P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_NULL);
  b = c; b.chunk = 256;
  EXPECT(ttt_scan_bwd(&b, P(0x1000), P(0x1000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), P(0x6000),
                      P(0x40000), NULL, P(0x50000), P(0x60000), P(0x70000), (float*)P(0x71000), &w,
                      NULL, NULL, P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_UNSUPPORTED);
  /* decode: position out of range */
  EXPECT(ttt_decode_step(&c, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), (float*)P(0x5000),
                         (float*)P(0x6000), &w, &w, 16, P(0x70000), P(0x90000), 256, NULL), TTT_ERR_ARG);
  /* decode: a workspace without room for the four-workgroup kernel's exchange area */
  b = c; b.flags = TTT_DECODE_SPLIT;
  EXPECT(ttt_decode_step(&b, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), (float*)P(0x5000),
                         (float*)P(0x6000), &w, &w, 3, P(0x70000), P(0x90000), 256, NULL), TTT_ERR_WORKSPACE);
  /* momentum: unsupported flag */
  b = c; b.flags = TTT_OUTPUT_KEY;
  EXPECT(ttt_scan_fwd_momentum(&b, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), (float*)P(0x5000),
                               (float*)P(0x6000), (float*)P(0x7000), (float*)P(0x8000), &w, NULL, P(0x70000),
                               NULL, NULL, NULL, P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_UNSUPPORTED);
  /* the large-chunk SwiGLU layer: its own kind, checks and workspace op */
  {
    ttt_config l = c;
    l.kind = TTT_SWIGLU; l.chunk = 2048;
    EXPECT(ttt_validate(&l), TTT_OK);
    EXPECT(ttt_workspace_size(&l, TTT_OP_LACT, &n), TTT_OK);
    if (n != 256 + (size_t)96 * (2 * 3 * 64 * 256 + 2 * 2 * 64) * 4) ++failures;
    EXPECT(ttt_workspace_size(&l, TTT_OP_FWD, &n), TTT_ERR_UNSUPPORTED);
    EXPECT(ttt_workspace_size(&c, TTT_OP_LACT, &n), TTT_ERR_UNSUPPORTED);
    ttt_swiglu_weights w3 = {(float*)P(0x10000), (float*)P(0x20000), (float*)P(0x30000)};
    ttt_swiglu_weights w3n = {(float*)P(0x10000), NULL, (float*)P(0x30000)};
    /* every call below is rejected before anything is enqueued */
    EXPECT(ttt_lact_fwd(&l, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), &w3n, P(0x5000), NULL,
                        P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_NULL);
    EXPECT(ttt_lact_fwd(&l, P(0x1008), P(0x2000), P(0x3000), (float*)P(0x4000), &w3, P(0x5000), NULL,
                        P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_ALIGN);
    EXPECT(ttt_lact_fwd(&l, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), &w3, P(0x5000), NULL,
                        P(0x90000), 4096, NULL), TTT_ERR_WORKSPACE);
    EXPECT(ttt_lact_fwd(&l, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), &w3, P(0x5000), NULL,
                        NULL, (size_t)1 << 40, NULL), TTT_ERR_WORKSPACE);
    EXPECT(ttt_lact_fwd(&c, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), &w3, P(0x5000), NULL,
                        P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_UNSUPPORTED);
    ttt_config lb = l; lb.flags = TTT_FORCE_GENERIC;
    EXPECT(ttt_lact_fwd(&lb, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), &w3, P(0x5000), NULL,
                        P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_ARG);
    lb = l; lb.chunk = 96;
    EXPECT(ttt_validate(&lb), TTT_ERR_SHAPE);
    lb = l; lb.chunk = 48; lb.T = 96;
    EXPECT(ttt_validate(&lb), TTT_ERR_UNSUPPORTED);
    EXPECT(ttt_lact_fwd(NULL, P(0x1000), P(0x2000), P(0x3000), (float*)P(0x4000), &w3, P(0x5000), NULL,
                        P(0x90000), (size_t)1 << 40, NULL), TTT_ERR_NULL);
  }
  EXPECT(ttt_read_status(NULL, NULL), TTT_ERR_NULL);
  EXPECT(ttt_reset_status(NULL, NULL), TTT_ERR_NULL);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("all host ABI checks passed\n");
  return 0;
}
