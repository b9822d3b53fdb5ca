/* A plain C11 client of the library's C ABI.  It includes both public headers, binds
 * every declared entry point to a function pointer of the declared type (so the
 * prototypes are valid C and every symbol resolves at link time), and makes only the
 * calls that return before any HIP call: the workspace queries, the status strings and
 * argument checks.  Prints "ok" and exits 0 when every check holds; otherwise names the
 * failed check and exits 1.  Built and run by tests/test_abi_c.py on the CPU. */
#include <stdio.h>
#include <string.h>

#include "distill.h"

static int failures = 0;

#define CHECK(cond)                                            \
  do {                                                         \
    if (!(cond)) {                                             \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                              \
    }                                                          \
  } while (0)

int main(void) {
  /* every entry point, through a pointer of its declared type */
  size_t (*q_ws)(int64_t, int64_t, int) = rn_bwd_workspace_bytes;
  int (*rms_f)(const void*, int64_t, const void*, void*, int64_t, float*, int64_t, int64_t,
               float, float, rn_dtype, rn_dtype, hipStream_t) = rmsnorm_fwd;
  int (*rms_b)(const void*, int64_t, const void*, int64_t, const void*, void*, int64_t, float*,
               void*, size_t, int64_t, int64_t, float, float, rn_dtype, rn_dtype,
               hipStream_t) = rmsnorm_bwd;
  int (*rms_na)(const void*, int64_t, const void*, int64_t, const void*, void*, int64_t, float*,
                int64_t, int64_t, float, float, rn_dtype, rn_dtype, hipStream_t) =
      rmsnorm_bwd_noalloc;
  int (*ln_f)(const void*, int64_t, const void*, const void*, void*, int64_t, float*, float*,
              int64_t, int64_t, float, rn_dtype, rn_dtype, hipStream_t) = layernorm_fwd;
  int (*ln_b)(const void*, int64_t, const void*, int64_t, const void*, void*, int64_t, float*,
              float*, void*, size_t, int64_t, int64_t, float, rn_dtype, rn_dtype,
              hipStream_t) = layernorm_bwd;
  int (*fa_f)(const void*, int64_t, const void*, int64_t, const void*, void*, int64_t, void*,
              int64_t, float*, int64_t, int64_t, float, float, rn_dtype, rn_dtype,
              hipStream_t) = fused_add_rmsnorm_fwd;
  int (*fa_b)(const void*, int64_t, const void*, int64_t, const void*, int64_t, const void*,
              void*, int64_t, float*, void*, size_t, int64_t, int64_t, float, float, rn_dtype,
              rn_dtype, hipStream_t) = fused_add_rmsnorm_bwd;
  const char* (*st)(int) = rn_status_str;
  size_t (*d_ws)(int64_t, int64_t, int64_t, int64_t, int64_t, int, int, int) =
      fused_linear_jsd_workspace_bytes;
  int (*d_f)(const void*, int64_t, const void*, const void*, const void*, int64_t,
             const void*, const void*, int64_t, int64_t, int64_t, int64_t, float, float,
             int64_t, float*, void*, int64_t, float*, float*, void*, size_t, hipStream_t) =
      fused_linear_jsd;

  /* host-only calls */
  CHECK(strcmp(st(RN_OK), "ok") == 0);
  for (int s = RN_ERR_SCRATCH; s <= RN_OK; ++s) CHECK(st(s) != NULL && st(s)[0] != '\0');
  CHECK(q_ws(8192, 8192, 0) == 0);
  CHECK(q_ws(8192, 8192, 1) > 0 && q_ws(8192, 8192, 2) == 2 * q_ws(8192, 8192, 1));
  CHECK(q_ws(-1, 64, 1) == 0 && q_ws(4, 0, 1) == 0);
  CHECK(d_ws(4096, 4096, 4096, 128256, 1024, 1, 1, 1) >
        d_ws(4096, 4096, 4096, 128256, 1024, 1, 0, 0));

  /* argument checks that return before any HIP call: the addresses are distinct,
   * aligned and never dereferenced */
  const void* p = (const void*)(uintptr_t)4096;
  void* o = (void*)(uintptr_t)8192;
  float* r = (float*)(uintptr_t)12288;
  void* wsp = (void*)(uintptr_t)(1u << 20);
  CHECK(rms_f(p, 64, p, o, 64, NULL, 0, 64, 1e-6f, 0.0f, RN_BF16, RN_BF16, NULL) == RN_OK);
  CHECK(rms_f(NULL, 64, p, o, 64, NULL, 4, 64, 1e-6f, 0.0f, RN_BF16, RN_BF16, NULL) ==
        RN_ERR_NULL);
  CHECK(rms_f(p, 64, p, o, 64, NULL, -1, 64, 1e-6f, 0.0f, RN_BF16, RN_BF16, NULL) ==
        RN_ERR_SHAPE);
  CHECK(rms_f(p, 64, p, o, 64, NULL, 4, 64, 1e-6f, 0.0f, (rn_dtype)7, RN_BF16, NULL) ==
        RN_ERR_DTYPE);
  CHECK(rms_f(p, 63, p, o, 64, NULL, 4, 64, 1e-6f, 0.0f, RN_BF16, RN_BF16, NULL) ==
        RN_ERR_STRIDE);
  CHECK(rms_b(p, 64, p, 64, p, o, 64, r, NULL, 0, 4, 64, 1e-6f, 0.0f, RN_BF16, RN_BF16,
              NULL) == RN_ERR_WORKSPACE);
  CHECK(rms_na(p, 16384, p, 16384, p, o, 16384, r, 4096, 16384, 1e-6f, 0.0f, RN_BF16,
               RN_BF16, NULL) == RN_ERR_SCRATCH);
  CHECK(ln_f(p, 64, NULL, NULL, o, 64, NULL, NULL, 4, 64, 1e-5f, RN_F32, RN_F32, NULL) ==
        RN_ERR_NULL);
  CHECK(ln_b(p, 64, p, 64, p, o, 64, r, r, wsp, 1u << 20, 4, 64, 1e-5f, RN_F32, RN_F32,
             NULL) == RN_ERR_ALIAS);
  CHECK(fa_f(p, 64, p, 64, p, o, 64, o, 64, NULL, 4, 64, 1e-6f, 1.0f, RN_BF16, RN_BF16,
             NULL) == RN_ERR_ALIAS);
  CHECK(fa_b(p, 64, NULL, 0, NULL, 64, p, o, 64, NULL, NULL, 0, 4, 64, 1e-6f, 1.0f, RN_BF16,
             RN_BF16, NULL) == RN_ERR_NULL);
  const size_t need = d_ws(16, 64, 64, 100, 8, 0, 0, 0);
  CHECK(need > 0);
  CHECK(d_f(NULL, 64, p, NULL, p, 64, p, NULL, 16, 64, 64, 100, 0.5f, 1.0f, 8, r, NULL, 0,
            NULL, NULL, wsp, need, NULL) == RN_ERR_NULL);
  CHECK(d_f(p, 64, p, NULL, p, 64, p, NULL, 16, 60, 64, 100, 0.5f, 1.0f, 8, r, NULL, 0, NULL,
            NULL, wsp, need, NULL) == RN_ERR_SHAPE);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
