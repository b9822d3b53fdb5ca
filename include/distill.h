/*
 * distill.h — C ABI of the fused linear + Jensen-Shannon distillation loss on MI355X
 * (gfx950), the second operation of librownorm.so.
 *
 * Source, cited by page title and section:
 *   [distill] "perf(distillation): skip dW/dB calculation when parameters are frozen"
 *     — Summary: a fused linear distillation loss runs the student and teacher heads
 *       over chunks of tokens and a divergence between their distributions; when the
 *       student head's weight (bias) does not require a gradient, no gradient buffer is
 *       allocated and no per-chunk weight-gradient product runs, and when nothing
 *       requires a gradient only the forward runs.  Details: bf16, B*T = 4096 tokens,
 *       H = 4096, V = 128256 or 151936, chunks of 1024 tokens; loss and input gradients
 *       are unchanged by the skipping.
 *
 * Definition (the page prints no formula; the textbook weighted Jensen-Shannon
 * divergence): per token, z_s = x_s W_s^T (+ b_s), z_t = x_t W_t^T (+ b_t),
 * S = softmax(z_s / tau), T = softmax(z_t / tau), M = beta T + (1 - beta) S,
 * J = beta KL(T || M) + (1 - beta) KL(S || M); loss = mean of J over the tokens.  The
 * teacher is a fixed target: gradients are for the student's input, weight and bias.
 *
 * Arithmetic: the products on the MFMA units in bf16 with fp32 accumulation; the
 * per-token softmax, divergence and logit gradient in fp32 with fp64 row sums, e^x and
 * ln x per vocabulary entry through the hardware's base-2 exponential and logarithm
 * (relative error about 1e-6 at the magnitudes that carry weight); the logit gradient is
 * rounded to bf16 before the two gradient products (dx, dW), whose accumulation is fp32;
 * dx is stored in bf16, dW and db in fp32, the loss in fp32.  Every reduction has a
 * fixed order: results are bitwise reproducible, and the loss and dx do not depend on
 * which parameter gradients are requested.  With beta = 0 or 1 the mixture is S or T
 * itself: the loss and every gradient are then exactly zero.
 *
 * Schedule: per chunk, the two logits products, the per-token statistics, the logit
 * gradient and the dx product; dW is one product over all tokens after the last chunk
 * (the bf16 transposed logit gradient of every token is kept for it), so the chunking
 * bounds the fp32 logits, 2 x chunk x V x 4 bytes, not the dW input.
 *
 * Conventions: all pointers are DEVICE pointers owned by the caller; the call only
 * enqueues kernels on `stream` (no allocation, no synchronisation).  Matrices are
 * row-major; ld* are row strides in elements.  x_s [BT, H] (ld ldxs), W_s [V, H]
 * (contiguous), b_s [V] or NULL, x_t [BT, Ht] (ld ldxt), W_t [V, Ht], b_t [V] or NULL,
 * all bf16.  H, Ht, ldxs and ldxt must be multiples of 8 and every bf16 base pointer
 * 16-byte aligned.  Errors are the rn_status codes of rownorm.h, returned before any
 * HIP call (RN_ERR_HIP: a launch was refused).
 */
#ifndef DISTILL_H
#define DISTILL_H

#include "rownorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes of fused_linear_jsd for these sizes and requested gradients
 * (want_* = 0 / 1): two fp32 logit blocks of chunk x V, per-token statistics, the bf16
 * transposed logit gradient (V x chunk for dx alone, V x BT with dw), for dx split
 * partial sums, for dw the transposed student input (H x BT), for db column sums per 64
 * tokens of a chunk.  A frozen head (want_dw = 0) needs none of the dW buffers
 * ([distill], Summary).  0 for invalid sizes (with want_dw, BT rounded up to 8 must not
 * exceed 2^22). */
size_t fused_linear_jsd_workspace_bytes(int64_t BT, int64_t H, int64_t Ht, int64_t V,
                                        int64_t chunk, int want_dx, int want_dw, int want_db);

/* Loss and student gradients.  loss: fp32 [1] out.  dxs: bf16 [BT, H] out (ld lddx) or
 * NULL; dws: fp32 [V, H] out or NULL (frozen weight: no dW product, no dW buffers);
 * dbs: fp32 [V] out or NULL (needs b_s).  All three NULL: forward only.  beta in [0, 1],
 * temperature > 0, 1 <= chunk (tokens per chunk; the products are sized by it; taken
 * as min(chunk, BT, 2^22) rounded up to a multiple of 8, which changes no result but the
 * summation order of dbs).
 * ws / ws_bytes: workspace of at least fused_linear_jsd_workspace_bytes(...) bytes,
 * 256-byte aligned, any contents. */
int fused_linear_jsd(const void* xs, int64_t ldxs, const void* ws_weight, const void* bs,
                     const void* xt, int64_t ldxt, const void* wt, const void* bt, int64_t BT,
                     int64_t H, int64_t Ht, int64_t V, float beta, float temperature,
                     int64_t chunk, float* loss, void* dxs, int64_t lddx, float* dws, float* dbs,
                     void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DISTILL_H */
