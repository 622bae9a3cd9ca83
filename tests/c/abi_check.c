/* Plain C99 client of the C ABI: includes the public header in a C
 * translation unit, links against the shared library and exercises the
 * host-side entry points (version, status strings, configuration queries and
 * argument checks), none of which needs a GPU.  Exit status 0 on success. */
#include <stdio.h>
#include <string.h>

#include "rmsnorm_rows.h"

static int failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  EXPECT(rn_abi_version() == RN_ABI_VERSION);
  EXPECT(strncmp(rn_status_string(RN_OK), "RN_OK", 5) == 0);

  rn_launch_config cfg;
  uint32_t flags = RN_MAKE_FLAGS(RN_DTYPE_BF16, RN_DTYPE_F32, RN_DTYPE_BF16, RN_DTYPE_BF16, 0);
  EXPECT(rmsnorm_query_config(16384, 8192, flags, 1, 256, &cfg) == RN_OK);
  EXPECT(cfg.kernel == RN_KERNEL_ROWS && cfg.grid == 16384);
  EXPECT((int64_t)64 * cfg.waves_per_row * cfg.vecs_per_lane * cfg.vec >= 8192);

  EXPECT(qknorm_query_config(4096, 32, 0, 128, 0, 256, &cfg) == RN_OK);
  EXPECT(cfg.kernel == RN_KERNEL_HEADS);

  uint32_t act = (RN_DTYPE_BF16 << RN_FLAGS_X_SHIFT) | (RN_DTYPE_FP4_E2M1 << RN_FLAGS_OUT_SHIFT) |
                 (RN_SCALE_NV16 << RN_FLAGS_SCALE_SHIFT);
  EXPECT(silu_mul_query_config(8192, 14336, act, 256, &cfg) == RN_OK);
  EXPECT(silu_mul_query_config(8192, 14336 + 8, act, 256, &cfg) == RN_ERR_UNSUPPORTED);

  /* argument checks run before any HIP call: fake (never dereferenced) pointers */
  const void* p = (const void*)(uintptr_t)0x10000;
  void* q = (void*)(uintptr_t)0x20000;
  EXPECT(rmsnorm_fwd(p, p, p, q, NULL, NULL, 4, 1024, 1e-6f, flags, NULL) == RN_ERR_INVALID_ARG);
  EXPECT(strlen(rn_last_error()) > 0);
  EXPECT(rmsnorm_fwd(p, p, p, q, q, NULL, 4, 1001, 1e-6f, flags, NULL) == RN_ERR_UNSUPPORTED);
  EXPECT(rmsnorm_fwd(NULL, NULL, NULL, NULL, NULL, NULL, 0, 1024, 1e-6f, flags, NULL) == RN_OK);
  EXPECT(rn_launch_copy(p, q, 1000, NULL) == RN_ERR_INVALID_ARG);
  /* the call-record form: the same checks */
  rn_rmsnorm_call call;
  memset(&call, 0, sizeof call);
  call.x = p; call.residual = p; call.weight = p; call.out = q; call.rows = 4; call.hidden = 1024;
  call.eps = 1e-6f; call.flags = flags;
  EXPECT(rmsnorm_fwd_call(&call) == RN_ERR_INVALID_ARG); /* residual_out missing */
  call.residual_out = q; call.hidden = 1001;
  EXPECT(rmsnorm_fwd_call(&call) == RN_ERR_UNSUPPORTED);
  EXPECT(rmsnorm_fwd_call(NULL) == RN_ERR_INVALID_ARG);
  call.rows = 0; call.hidden = 1024;
  EXPECT(rmsnorm_fwd_call(&call) == RN_OK);

  /* partial inputs: a host array of device pointers */
  const void* parts[3] = {p, p, (const void*)(uintptr_t)0x30008};
  EXPECT(rmsnorm_partials_query_config(2048, 8192, 8, flags, 1, 256, &cfg) == RN_OK);
  EXPECT(cfg.vecs_per_lane <= 2 && (int64_t)64 * cfg.waves_per_row * cfg.vecs_per_lane * cfg.vec >= 8192);
  EXPECT(rmsnorm_fwd_partials(parts, 3, p, p, q, (void*)(uintptr_t)0x40000, NULL, NULL, NULL, 4, 1024, 1e-6f,
                              flags, NULL) == RN_ERR_MISALIGNED);
  EXPECT(rmsnorm_fwd_partials(parts, 9, p, p, q, q, NULL, NULL, NULL, 4, 1024, 1e-6f, flags, NULL) ==
         RN_ERR_INVALID_ARG);
  EXPECT(rmsnorm_fwd_partials(NULL, 2, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 1024, 1e-6f, flags, NULL) ==
         RN_OK);

  if (failures == 0) printf("c abi check: ok\n");
  return failures == 0 ? 0 : 1;
}
