// dl_kernels.h — the non-GEMM kernels of the fused linear JSD distillation loss:
// the per-token loss and logit gradient over the vocabulary, transposes into the
// K-contiguous layout the GEMM takes, and fixed-order reductions.
//
// Source: [distill] "perf(distillation): skip dW/dB calculation when parameters are
// frozen", Summary (the loss differentiates the student head on every chunk unless it
// is frozen) and Details (B*T = 4096 tokens, H = 4096, V = 128256 / 151936, chunks of
// 1024 tokens, bf16).  Loss (the textbook weighted Jensen-Shannon divergence, the page
// prints no formula): S = softmax(z_s / tau), T = softmax(z_t / tau),
// M = beta T + (1 - beta) S, J = beta KL(T || M) + (1 - beta) KL(S || M), mean over tokens;
// dJ/dz_s,v = S_v (g_v - sum_u S_u g_u) / tau with g_v = (1 - beta) log(S_v / M_v).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dl_gemm.h"

namespace dl {

constexpr int JT = 1024;  // threads per token row

// Sum over the workgroup (fixed tree order); every thread gets the result.
__device__ __forceinline__ double block_sum(double v, double* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int h = blockDim.x / 2; h >= 1; h /= 2) {
    if (t < h) sh[t] += sh[t + h];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}
// Combined (max, sum of exp(x - max)) pairs over the workgroup, in a fixed tree order.
__device__ __forceinline__ void block_lse(float& m, double& s, float* shm, double* shs) {
  const int t = threadIdx.x;
  shm[t] = m;
  shs[t] = s;
  __syncthreads();
  for (int h = blockDim.x / 2; h >= 1; h /= 2) {
    if (t < h) {
      const float m1 = shm[t], m2 = shm[t + h];
      const float mm = fmaxf(m1, m2);
      const double s1 = m1 == -INFINITY ? 0.0 : shs[t] * static_cast<double>(expf(m1 - mm));
      const double s2 = m2 == -INFINITY ? 0.0 : shs[t + h] * static_cast<double>(expf(m2 - mm));
      shm[t] = mm;
      shs[t] = s1 + s2;
    }
    __syncthreads();
  }
  m = shm[0];
  s = shs[0];
  __syncthreads();
}

struct JsdArgs {
  float* zs; const float* zt; int64_t ldz;  // [rows][ldz] fp32 logits; zs becomes fp32 dz
  uint16_t* gb; int64_t ldg;                // bf16 dz [rows][ldg], or null
  double* jtok;                             // per-token J [rows]
  int rows, V, vpad;                        // vpad: gb row length written (zeros past V)
  float beta, inv_tau;
  float grad_scale;                         // 1 / (tau * tokens): dL/dz = grad_scale * S (g - A)
  int want_grad;                            // 0: loss only
  int write_f32;                            // fp32 dz into zs (for dW / db)
};

// log(a e^x + b e^y) for a, b >= 0, stable for any x, y (a or b may be 0)
__device__ __forceinline__ float log_mix(float la, float x, float lb, float y) {
  const float p = la + x, q = lb + y;
  const float mx = fmaxf(p, q);
  if (mx == -INFINITY) return -INFINITY;
  return mx + log1pf(expf(-fabsf(p - q)));
}

// One workgroup per token row: three passes over the row's V logits (which the caches
// mostly hold after the first): log-sum-exp of both rows (online max and sum), the
// divergence and sum_u S_u g_u, then the gradient.
__global__ __launch_bounds__(JT) void jsd_rows_kernel(JsdArgs a) {
  __shared__ float shm[JT];
  __shared__ double shs[JT];
  const int row = blockIdx.x;
  if (row >= a.rows) return;
  const int t = threadIdx.x;
  float* zs = a.zs + static_cast<int64_t>(row) * a.ldz;
  const float* zt = a.zt + static_cast<int64_t>(row) * a.ldz;
  const int V = a.V;
  const float it = a.inv_tau;

  float ms = -INFINITY, mt = -INFINITY;
  double ss = 0.0, st = 0.0;
  for (int v = t; v < V; v += JT) {
    const float xs = zs[v] * it, xt = zt[v] * it;
    if (xs > ms) { ss = ss * static_cast<double>(expf(ms - xs)) + 1.0; ms = xs; }
    else ss += static_cast<double>(expf(xs - ms));
    if (xt > mt) { st = st * static_cast<double>(expf(mt - xt)) + 1.0; mt = xt; }
    else st += static_cast<double>(expf(xt - mt));
  }
  block_lse(ms, ss, shm, shs);
  block_lse(mt, st, shm, shs);
  const float lse_s = ms + static_cast<float>(log(ss));
  const float lse_t = mt + static_cast<float>(log(st));
  const float b = a.beta;
  const float lb = logf(b), l1b = logf(1.0f - b);

  double jsum = 0.0, gsum = 0.0;
  for (int v = t; v < V; v += JT) {
    const float ls = zs[v] * it - lse_s, lt = zt[v] * it - lse_t;
    const float lm = log_mix(lb, lt, l1b, ls);
    const float s = expf(ls), tt = expf(lt);
    const float g = (1.0f - b) * (ls - lm);
    jsum += static_cast<double>(b * tt * (lt - lm) + (1.0f - b) * s * (ls - lm));
    gsum += static_cast<double>(s * g);
  }
  jsum = block_sum(jsum, shs);
  if (t == 0) a.jtok[row] = jsum;
  if (!a.want_grad) return;
  const float A = static_cast<float>(block_sum(gsum, shs));
  uint16_t* gb = a.gb != nullptr ? a.gb + static_cast<int64_t>(row) * a.ldg : nullptr;
  for (int v = t; v < V; v += JT) {
    const float ls = zs[v] * it - lse_s, lt = zt[v] * it - lse_t;
    const float lm = log_mix(lb, lt, l1b, ls);
    const float s = expf(ls);
    const float g = (1.0f - b) * (ls - lm);
    const float dz = a.grad_scale * s * (g - A);
    if (gb != nullptr) gb[v] = f_to_bf16(dz);
    if (a.write_f32) zs[v] = dz;
  }
  if (gb != nullptr)
    for (int v = V + t; v < a.vpad; v += JT) gb[v] = 0;  // K padding of the dx product
}

// out[c][r] = bf16(in[r][c]) for an R x C block, in 64 x 64 tiles through LDS; output
// columns r in [R, Rpad) are written as zeros (K padding of a following product).
template <typename TIN>
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const TIN* in, int64_t ldi, int R,
                                                             int Cc, uint16_t* out, int64_t ldo,
                                                             int Rpad) {
  __shared__ uint16_t tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    uint16_t v = 0;
    if (r < R && c < Cc) {
      if constexpr (sizeof(TIN) == 2) v = static_cast<uint16_t>(in[static_cast<int64_t>(r) * ldi + c]);
      else v = f_to_bf16(static_cast<float>(in[static_cast<int64_t>(r) * ldi + c]));
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < Cc && r < Rpad) out[static_cast<int64_t>(c) * ldo + r] = r < R ? tile[tx][i] : 0;
  }
}

// out[m][n] = bf16(sum over z = 0..S-1, in that order, of part[z][m][n])
__global__ __launch_bounds__(256) void split_sum_bf16_kernel(const float* part, int64_t stride,
                                                             int S, int M, int N, int64_t ldp,
                                                             uint16_t* out, int64_t ldo) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * N) return;
  const int m = static_cast<int>(i / N), n = static_cast<int>(i % N);
  const int64_t o = static_cast<int64_t>(m) * ldp + n;
  float s = part[o];
  for (int z = 1; z < S; ++z) s += part[z * stride + o];
  out[static_cast<int64_t>(m) * ldo + n] = f_to_bf16(s);
}

// db[v] (+)= sum over rows r = 0..R-1, in that order, of dz[r][v]
__global__ __launch_bounds__(256) void colsum_rows_kernel(const float* dz, int64_t ldz, int R,
                                                          int V, float* db, int accumulate) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  float s = 0.0f;
  for (int r = 0; r < R; ++r) s += dz[static_cast<int64_t>(r) * ldz + v];
  db[v] = accumulate ? db[v] + s : s;
}

// loss = (sum over tokens, fixed tree order, of J) / tokens
__global__ __launch_bounds__(1024) void loss_sum_kernel(const double* jtok, int64_t n, float* loss) {
  __shared__ double sh[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) s += jtok[i];
  s = block_sum(s, sh);
  if (threadIdx.x == 0) *loss = n > 0 ? static_cast<float>(s / static_cast<double>(n)) : 0.0f;
}

// zero fill (fp32), for outputs of an empty batch
__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace dl
