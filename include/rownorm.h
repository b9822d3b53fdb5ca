/*
 * rownorm.h — C ABI of the row-wise normalisation library for AMD MI355X (gfx950).
 *
 * Operations (forward and backward): RMSNorm, LayerNorm and FusedAddRMSNorm over the
 * rows of an [M, N] matrix.  Sources, cited by page title and section:
 *   [frozen] "perf(norm): skip dW/dB calculation when parameters are frozen (#1067)"
 *            — Motivation, Key Changes: backward kernels whose weight/bias gradient
 *            work is pruned at compile time when the parameter is frozen; unused
 *            gradient pointers are passed as null.
 *   [gemma]  "fix(cutedsl): fuse Gemma RMSNorm weight offset in FP32"
 *            — Summary: the weight and the Gemma offset are passed separately and
 *            added in (at least) FP32 inside the forward and backward kernels;
 *            Testing Done: mixed FP32 weights, strided inputs, in-place backward,
 *            residual-output gradients, hidden sizes up to 18432.
 *
 * Definitions (the pages name the operations but print no formulas; these are the
 * textbook / torch.nn.functional conventions):
 *   RMSNorm    y = x * rstd * (w + offset),  rstd = 1 / sqrt(mean_j x_j^2 + eps)
 *   LayerNorm  y = (x - mean) * rstd * w + b, rstd = 1 / sqrt(var + eps), var biased
 *   FusedAdd   residual_out = round(x + residual); y = RMSNorm(residual_out)
 *   Backward   g = dy * weight_eff, xhat = normalised row
 *     RMSNorm    dx = rstd * (g - xhat * mean_j(g * xhat))
 *     LayerNorm  dx = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat))
 *     FusedAdd   dx = dres_out + RMSNorm backward at residual_out; dx is the gradient
 *                of both x and residual
 *     dw = sum over rows of dy * xhat, db = sum over rows of dy (fp32 outputs)
 *
 * Conventions for every entry point:
 *   - Matrices are row-major [M, N]; ld* is the row stride in ELEMENTS (ld >= N, the
 *     last dimension is contiguous).  M >= 0, 1 <= N <= RN_MAX_N.
 *   - x, residual, y, residual_out, dy, dres_out and dx share the I/O type `xt`;
 *     w and b share the weight type `wt`, which is `xt` or RN_F32 (mixed precision).
 *     rstd, mean, dw and db are float32.
 *   - All pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronises: every call only enqueues kernels on `stream`
 *     (NULL = the null stream) and returns.  Calls are therefore capturable in a
 *     hipGraph.
 *   - Arithmetic: row statistics and every output that can cancel (LayerNorm y, all
 *     dx) are formed in fp64 and rounded once to the output type (through fp32, so a
 *     16-bit output is at most 1 unit in the last place from the correctly rounded
 *     value).  RMSNorm y is formed in fp32 from (float)w + offset.
 *   - Errors: arguments are checked before any HIP call; on error nothing is enqueued
 *     and an rn_status < 0 is returned.  RN_ERR_HIP reports that the HIP runtime refused
 *     one of this call's launches (the status of that launch itself, not an error left
 *     behind by earlier HIP work).  The library keeps no mutable process-wide state.
 *   - Backward workspace (parameter gradients only): caller-owned device memory of at
 *     least rn_bwd_workspace_bytes() bytes, 16-byte aligned, any contents; it holds the
 *     per-workgroup partial rows of dw / db between the two kernels of one call.  One
 *     workspace must not be used by two calls that can run at the same time (different
 *     streams without ordering).
 *   - Aliasing: an output may alias an input of the same shape and stride (y == x,
 *     residual_out == residual, dx == dy or dx == dres_out): such calls run kernels
 *     in which each element is read before it is written by the same thread (never
 *     the split-row kernels, whose workgroups read the whole row).  Any other overlap
 *     is undefined.
 *   - Few long rows (aligned rows of at least two spans of 256 16-byte accesses, at
 *     most 128 rows) are spread over several workgroups each; the results meet the
 *     same accuracy contract, and dx does not depend on which parameter gradients are
 *     requested.
 */
#ifndef ROWNORM_H
#define ROWNORM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rn_dtype {
  RN_F32 = 0,
  RN_F16 = 1,
  RN_BF16 = 2,
  /* Not types.  They make every 32-bit int a value of the enumeration, so that an
   * unchecked value from a C or foreign-function caller is well defined in the library
   * and reaches its check (RN_ERR_DTYPE). */
  RN_DTYPE_RANGE_LO_ = -2147483647 - 1,
  RN_DTYPE_RANGE_HI_ = 2147483647
} rn_dtype;

typedef enum rn_status {
  RN_OK = 0,
  RN_ERR_NULL = -1,       /* a required pointer is NULL (with M > 0)              */
  RN_ERR_SHAPE = -2,      /* M < 0, N < 1 or N > RN_MAX_N                          */
  RN_ERR_DTYPE = -3,      /* unknown type, or a weight type other than xt / F32   */
  RN_ERR_STRIDE = -4,     /* a row stride below N                                  */
  RN_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than rn_bwd_workspace_bytes */
  RN_ERR_HIP = -6,        /* a kernel launch failed                                */
  RN_ERR_ALIAS = -7,      /* two outputs share storage                             */
  RN_ERR_INTERNAL = -8,   /* no compiled kernel instance for the planned launch    */
  RN_ERR_SCRATCH = -9     /* rmsnorm_bwd_noalloc: the shape needs more partial-row */
                          /* space than its fixed scratch holds                    */
} rn_status;

#define RN_MAX_N 24576

/* Bytes of workspace a backward call needs for `n_param_grads` (0, 1 or 2) fp32
 * parameter gradients at this shape ([frozen], Motivation: per-program partial rows of
 * dw / db written by the first kernel, then summed over the rows by a second kernel, in
 * a fixed order).  0 when n_param_grads == 0 (frozen parameters need no workspace and
 * get no second kernel).  Returns 0 for invalid shapes.  When the call has a single
 * partial row (very small M: one workgroup covering every row, or one row spread over
 * workgroups) and dw / db are 16-byte aligned, the gradients are written directly and
 * the workspace is left untouched; it must still be passed. */
size_t rn_bwd_workspace_bytes(int64_t M, int64_t N, int n_param_grads);

/* RMSNorm forward.  [gemma] Summary: offset added to the weight in fp32 in-kernel.
 *   x [M, ldx] in, w [N] in, y [M, ldy] out, rstd [M] out (fp32, may be NULL when no
 *   backward follows).  eps >= 0. */
int rmsnorm_fwd(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                float* rstd, int64_t M, int64_t N, float eps, float offset,
                rn_dtype xt, rn_dtype wt, hipStream_t stream);

/* RMSNorm backward.  [frozen] Key Changes (RMSNorm dW pruned when frozen);
 * [gemma] Summary (offset applied in the backward too).
 *   dy [M, lddy] in, x [M, ldx] in (the forward's input), w [N] in,
 *   dx [M, lddx] out (may equal dy), dw [N] fp32 out or NULL (frozen weight: no
 *   workspace, no partials, no second kernel), ws / ws_bytes: workspace of at least
 *   rn_bwd_workspace_bytes(M, N, dw != NULL) bytes (may be NULL / 0 when dw is NULL).
 *   Statistics: this entry point takes eps where a plain rendering of the method would
 *   take the forward's saved rstd.  It recomputes the row's statistics from x in fp64
 *   while it reads x anyway (no extra HBM traffic): a saved fp32 rstd carries a 2^-24
 *   relative error that the cancellation in g - xhat * mean(g * xhat) turns into
 *   whole-unit errors of small 16-bit dx values.  The forward's rstd output is
 *   therefore informational (it may be NULL). */
int rmsnorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w,
                void* dx, int64_t lddx, float* dw, void* ws, size_t ws_bytes,
                int64_t M, int64_t N, float eps, float offset,
                rn_dtype xt, rn_dtype wt, hipStream_t stream);

/* RMSNorm backward that allocates nothing and takes no workspace, for callers that
 * cannot allocate (code under hipGraph capture without a memory pool, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and contract as
 * rmsnorm_bwd without ws / ws_bytes: the partial rows of dw live in a device array
 * inside the library, one per GPU (8 MiB, held until the process ends; its address is
 * looked up once per device).  Limit: rn_bwd_workspace_bytes(M, N, 1) <= 8 MiB, i.e.
 * every shape with N <= 8192, and wider rows while min(M, 256) partial rows fit; a
 * larger call returns RN_ERR_SCRATCH before anything is enqueued.  dw == NULL (frozen)
 * has no limit.  Calls on one GPU share the array: calls that may overlap in time
 * (different streams without ordering) race and must not be made. */
int rmsnorm_bwd_noalloc(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                        const void* w, void* dx, int64_t lddx, float* dw, int64_t M,
                        int64_t N, float eps, float offset, rn_dtype xt, rn_dtype wt,
                        hipStream_t stream);

/* LayerNorm forward.  [frozen] Key Changes (LayerNorm with weight and bias).
 *   x in, w [N] in, b [N] in or NULL (no bias), y out, mean / rstd [M] fp32 out or
 *   NULL.  eps >= 0. */
int layernorm_fwd(const void* x, int64_t ldx, const void* w, const void* b, void* y,
                  int64_t ldy, float* mean, float* rstd, int64_t M, int64_t N, float eps,
                  rn_dtype xt, rn_dtype wt, hipStream_t stream);

/* LayerNorm backward.  [frozen] Key Changes: dW and dB are pruned independently.
 *   dw, db: fp32 [N] out, each may be NULL.  Workspace of at least
 *   rn_bwd_workspace_bytes(M, N, (dw != NULL) + (db != NULL)) bytes.
 *   Statistics: takes eps instead of the forward's saved mean / rstd and recomputes
 *   them from x in fp64, for the reason given at rmsnorm_bwd; the forward's mean and
 *   rstd outputs are informational (they may be NULL). */
int layernorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w,
                  void* dx, int64_t lddx, float* dw, float* db, void* ws, size_t ws_bytes,
                  int64_t M, int64_t N, float eps, rn_dtype xt, rn_dtype wt,
                  hipStream_t stream);

/* FusedAddRMSNorm forward.  [gemma] Summary (Gemma offset on this op),
 * PyTorch accuracy comparison (the rounded sum is what is saved).
 *   x, residual in; residual_out = round(x + residual) out (may equal residual);
 *   y out; rstd [M] fp32 out or NULL. */
int fused_add_rmsnorm_fwd(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                          const void* w, void* y, int64_t ldy, void* residual_out,
                          int64_t ldro, float* rstd, int64_t M, int64_t N, float eps,
                          float offset, rn_dtype xt, rn_dtype wt, hipStream_t stream);

/* FusedAddRMSNorm backward.  [gemma] PyTorch accuracy comparison (residual-output
 * gradient; the backward works from the rounded saved residual).
 *   dy in; dres_out in or NULL (no gradient reaches residual_out); residual_out in
 *   (the forward's output); dx out = gradient of x and of residual (may equal dy or
 *   dres_out); dw fp32 out or NULL; workspace as for rmsnorm_bwd.
 *   Statistics: takes eps instead of the forward's saved rstd and recomputes it from
 *   residual_out in fp64, for the reason given at rmsnorm_bwd. */
int fused_add_rmsnorm_bwd(const void* dy, int64_t lddy, const void* dres_out, int64_t lddr,
                          const void* residual_out, int64_t ldro, const void* w, void* dx,
                          int64_t lddx, float* dw, void* ws, size_t ws_bytes, int64_t M,
                          int64_t N, float eps, float offset, rn_dtype xt, rn_dtype wt,
                          hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* rn_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* ROWNORM_H */
