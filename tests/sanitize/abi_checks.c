/* Host-side checks of the C ABI under AddressSanitizer / UndefinedBehaviorSanitizer: every entry
 * point with arguments that must be rejected before any device work, the size queries over a
 * range of shapes, and the status strings.  No GPU is needed (nothing here reaches a device
 * call); built by tests/test_sanitizers.py with the library's host code instrumented. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sage_attn.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      failures++;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  void* A = (void*)(uintptr_t)256; /* 16-byte aligned stand-in address, never dereferenced */
  void* M = (void*)(uintptr_t)258; /* misaligned */
  /* dense forward: nulls, misalignment, sizes, head dims, causal modes, variant bits */
  EXPECT(sage_attn_fwd(NULL, A, A, A, 1, 1, 64, 64, 64, 0, 0.0f, 0, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_fwd(M, A, A, A, 1, 1, 64, 64, 64, 0, 0.0f, 0, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_fwd(A, A, A, A, 0, 1, 64, 64, 64, 0, 0.0f, 0, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_fwd(A, A, A, A, 1, 1, 64, 64, 96, 0, 0.0f, 0, NULL) == SAGE_ERR_UNSUPPORTED);
  EXPECT(sage_attn_fwd(A, A, A, A, 1, 1, 65, 64, 64, 2, 0.0f, 0, NULL) == SAGE_ERR_UNSUPPORTED);
  EXPECT(sage_attn_fwd(A, A, A, A, 1, 1, 64, 64, 64, 3, 0.0f, 0, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_fwd(A, A, A, A, 1, 1, 64, 64, 64, 0, 0.0f, 0x8u, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_fwd(A, A, A, A, 1, 1, 64, 64, 64, 0, 0.0f, SAGE_PATH_MXFP4 | SAGE_QK_FP8, NULL) ==
         SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_fwd(A, A, A, A, 70000, 1, 64, 64, 64, 0, 0.0f, 0, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_fwd(A, A, A, A, 1, 32, 1 << 30, 64, 128, 0, 0.0f, 0, NULL) == SAGE_ERR_INVALID_ARG);
  /* workspace sizes grow with the problem and vanish on bad arguments */
  size_t prev = 0;
  for (int n = 1; n <= 65536; n *= 4) {
    for (unsigned var = 0; var <= SAGE_PATH_MXFP4; var++) {
      size_t w = sage_attn_workspace_bytes(2, 3, n, n + 7, var ? 128 : 64, n & 1, var);
      EXPECT(w > 0);
      if (!var) {
        EXPECT(w >= prev);
        prev = w;
      }
    }
  }
  EXPECT(sage_attn_workspace_bytes(1, 1, 64, 64, 80, 0, 0) == 0);
  /* extended entry points */
  sage_attn_shape sh = {1, 8, 2, 300, 700, 128, 1, 0.0f, SAGE_SMOOTH_V};
  size_t ws = sage_attn_workspace_bytes_ex(&sh);
  EXPECT(ws > 0);
  EXPECT(sage_attn_fwd_ex(&sh, A, A, A, A, A, ws - 1, NULL) == SAGE_ERR_NO_MEMORY);
  EXPECT(sage_attn_fwd_ex(&sh, A, A, A, A, (char*)A + 16, ws, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_fwd_ex(NULL, A, A, A, A, NULL, 0, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_workspace_bytes_ex(NULL) == 0);
  sage_attn_shape bad = sh;
  bad.Hkv = 3;
  EXPECT(sage_attn_workspace_bytes_ex(&bad) == 0);
  EXPECT(sage_attn_quantize_ex(&bad, A, A, A, NULL, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_quantize_ex(&sh, A, A, A, NULL, NULL) == SAGE_ERR_INVALID_ARG);
  /* variable-length batches */
  sage_attn_varlen_shape vl = {3, 4, 2, 64, 500, 700, 300, 400, (const int*)A, (const int*)((char*)A + 64), 1, 0.0f, 0};
  EXPECT(sage_attn_varlen_workspace_bytes(&vl) > 0);
  sage_attn_varlen_shape vb = vl;
  vb.cu_seqlens_q = (const int*)((char*)A + 2);
  EXPECT(sage_attn_varlen_workspace_bytes(&vb) == 0);
  EXPECT(sage_attn_varlen_fwd(&vb, A, A, A, A, NULL, 0, NULL) == SAGE_ERR_INVALID_ARG);
  vb = vl;
  vb.batch = 0;
  EXPECT(sage_attn_varlen_fwd(&vb, A, A, A, A, NULL, 0, NULL) == SAGE_ERR_INVALID_ARG);
  EXPECT(sage_attn_varlen_fwd(NULL, A, A, A, A, NULL, 0, NULL) == SAGE_ERR_INVALID_ARG);
  /* SageBwd */
  sage_attn_shape tr = {1, 4, 4, 256, 256, 128, 1, 0.0f, 0};
  EXPECT(sage_attn_train_workspace_bytes(&tr) > 0);
  sage_attn_shape tg = tr;
  tg.Hkv = 2;
  EXPECT(sage_attn_train_fwd(&tg, A, A, A, A, (float*)A, NULL, 0, NULL) == SAGE_ERR_UNSUPPORTED);
  sage_attn_shape tv = tr;
  tv.variant = SAGE_PATH_MXFP4;
  EXPECT(sage_attn_train_workspace_bytes(&tv) == 0);
  EXPECT(sage_attn_train_bwd(&tr, A, A, A, A, NULL, (const float*)A, (float*)A, (float*)A, (float*)A, NULL, 0,
                             NULL) == SAGE_ERR_INVALID_ARG);
  /* the no-allocation entry point rejects problems beyond its scratch before any device work */
  sage_attn_shape big = {1, 32, 32, 32768, 32768, 128, 1, 0.0f, 0};
  EXPECT(sage_attn_fwd_noalloc(&big, A, A, A, A, NULL) == SAGE_ERR_NO_MEMORY);
  EXPECT(sage_attn_fwd_noalloc(NULL, A, A, A, A, NULL) == SAGE_ERR_INVALID_ARG);
  /* diagnostics */
  for (int s = -6; s <= 1; s++) EXPECT(sage_attn_status_string(s) != NULL && strlen(sage_attn_status_string(s)) > 0);
  EXPECT(sage_attn_version() >= 100);
  sage_attn_set_profile_events(NULL, NULL);
  if (failures) return 1;
  printf("abi checks ok\n");
  return 0;
}
