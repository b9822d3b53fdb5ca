// rn_kernels.h — forward, backward (stage 1) and column-sum (stage 2) kernels.
//
// Sources (web pages, by title and section):
//   [frozen] "perf(norm): skip dW/dB calculation when parameters are frozen (#1067)",
//            Motivation / Key Changes: the backward accumulates dW (and dB) per
//            program across its tokens, writes per-program partial rows, and a second
//            reduction sums them; all of it is pruned at compile time when frozen.
//   [gemma]  "fix(cutedsl): fuse Gemma RMSNorm weight offset in FP32", Summary: the
//            offset is added to the weight inside the forward and backward kernels,
//            not pre-added in the 16-bit weight type.
//
// Arithmetic policy.  Row sums are accumulated in fp64 (full rate on CDNA4 vector
// ALUs, and this path is bound by HBM, not by the ALUs).  Every output whose value
// can cancel (LayerNorm y against the bias; every dx) is formed in fp64 from exact
// fp64 copies of the inputs and rounded once to the output type through fp32.  The
// backward recomputes the row statistics from x instead of reading a saved fp32
// rstd: a rounded rstd would carry a 2^-24 relative error that the cancellation in
// g - xhat * mean(g * xhat) turns into whole-ulp errors of small dx values.
#pragma once
#include "rn_device.h"

namespace rn {

struct FwdArgs {
  const void* x; int64_t ldx;
  const void* res; int64_t ldr;     // fused add: residual
  const void* w; const void* b;     // b may be null (LayerNorm without bias)
  void* y; int64_t ldy;
  void* ro; int64_t ldro;           // fused add: residual_out
  float* rstd; float* mean;         // may be null
  int64_t M; int N; int team; int rows_per_wg;
  float eps, offset;
};

struct BwdArgs {
  const void* dy; int64_t lddy;
  const void* x; int64_t ldx;       // x (RMS, LN) or residual_out (fused add)
  const void* dres; int64_t lddr;   // fused add: gradient reaching residual_out, may be null
  const void* w;
  void* dx; int64_t lddx;
  float* ws; int64_t ldws; int P;   // partial rows: [P][ldws] for dw, then [P][ldws] for db
  int64_t M; int N; int team; int rows_per_wg;
  float eps, offset;
};

// ------------------------------------------------------------------------------------
// Forward.  One team per row; the workgroup holds R = blockDim / team teams and walks
// rows_per_wg consecutive rows, R at a time.
// ------------------------------------------------------------------------------------
// Largest workgroup a kernel with V elements per thread is compiled for: 16 waves
// (128 VGPRs per lane) up to V = 16, 12 waves (168 VGPRs) above.
constexpr int max_wg(int V) { return V <= 16 ? 1024 : 768; }

template <int OP, int DX, int DW, int V, bool VEC>
__global__ __launch_bounds__(max_wg(V)) void fwd_kernel(FwdArgs p) {
  constexpr int EVE = 16 / Ty<DX>::B;
  using FX = Frag<DX, V, EVE, VEC>;
  using FW = Frag<DW, V, EVE, VEC>;
  __shared__ double red[2][16][4];
  int parity = 0;
  const int T = p.team;
  const int tid = threadIdx.x;
  const int r = tid / T;
  const int t = tid - r * T;
  const int R = blockDim.x / T;
  const int wpr = T >> 6;
  const int wave0 = (r * T) >> 6;
  const int N = p.N;
  const double inv_n = 1.0 / N;

  // Weight (and bias) columns owned by this thread, loaded once per workgroup.
  float wv[V];
  float bv[V];
  {
    FW wf;
    wf.load(p.w, t, T, N, true);
#pragma unroll
    for (int i = 0; i < V; ++i) wv[i] = wf.get(i);
    if constexpr (OP == OP_LN) {
      if (p.b != nullptr) {
        wf.load(p.b, t, T, N, true);
#pragma unroll
        for (int i = 0; i < V; ++i) bv[i] = wf.get(i);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) bv[i] = 0.0f;
      }
    } else {
      // [gemma] Summary: offset added to the weight in fp32, inside the kernel.
#pragma unroll
      for (int i = 0; i < V; ++i) wv[i] = wv[i] + p.offset;
    }
  }

  const int64_t row_begin = static_cast<int64_t>(blockIdx.x) * p.rows_per_wg;
  const int64_t row_end = min(row_begin + p.rows_per_wg, p.M);
  const int iters = (p.rows_per_wg + R - 1) / R;

  for (int it = 0; it < iters; ++it) {
    const int64_t row = row_begin + static_cast<int64_t>(it) * R + r;
    const bool valid = row < row_end;
    FX xf;
    xf.load(static_cast<const typename Ty<DX>::S*>(p.x) + row * p.ldx, t, T, N, valid);

    if constexpr (OP == OP_FADD) {
      FX rf;
      rf.load(static_cast<const typename Ty<DX>::S*>(p.res) + row * p.ldr, t, T, N, valid);
      float s[V];
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] = xf.get(i) + rf.get(i);
      xf.pack(s);  // residual_out = round(x + residual); the norm works on this value
      xf.store_raw(static_cast<typename Ty<DX>::S*>(p.ro) + row * p.ldro, t, T, N, valid);
    }

    float o[V];
    if constexpr (OP == OP_RMS || OP == OP_FADD) {
      double acc[1] = {0.0};
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double v = static_cast<double>(xf.get(i));
        acc[0] = fma(v, v, acc[0]);
      }
      team_sum<1>(acc, wpr, wave0, red, parity);
      const double rstd = 1.0 / sqrt(acc[0] * inv_n + static_cast<double>(p.eps));
      const float rs = static_cast<float>(rstd);
#pragma unroll
      for (int i = 0; i < V; ++i) o[i] = (xf.get(i) * rs) * wv[i];
      if (valid && t == 0 && p.rstd != nullptr) p.rstd[row] = rs;
    } else {  // LayerNorm: one pass of shifted sums (shift = the row's first element)
      const typename Ty<DX>::S* xrow = static_cast<const typename Ty<DX>::S*>(p.x) + row * p.ldx;
      const double K = valid ? static_cast<double>(bits_to_f<DX>(xrow[0])) : 0.0;
      double d[V];
      double acc[2] = {0.0, 0.0};
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const bool in = FX::inb(i / FX::VE, t, T, N);
        d[i] = in ? static_cast<double>(xf.get(i)) - K : 0.0;
        acc[0] += d[i];
        acc[1] = fma(d[i], d[i], acc[1]);
      }
      team_sum<2>(acc, wpr, wave0, red, parity);
      const double delta = acc[0] * inv_n;
      const double var = fmax(acc[1] * inv_n - delta * delta, 0.0);
      const double rstd = 1.0 / sqrt(var + static_cast<double>(p.eps));
#pragma unroll
      for (int i = 0; i < V; ++i)
        o[i] = static_cast<float>(fma((d[i] - delta) * rstd, static_cast<double>(wv[i]),
                                      static_cast<double>(bv[i])));
      if (valid && t == 0) {
        if (p.rstd != nullptr) p.rstd[row] = static_cast<float>(rstd);
        if (p.mean != nullptr) p.mean[row] = static_cast<float>(K + delta);
      }
    }
    FX yf;
    yf.pack(o);
    yf.store_raw(static_cast<typename Ty<DX>::S*>(p.y) + row * p.ldy, t, T, N, valid);
  }
}

// ------------------------------------------------------------------------------------
// Backward, stage 1: dx for every row, plus (CDW / CDB) per-thread fp32 accumulators of
// dw / db over the workgroup's rows, combined across the workgroup's teams in LDS and
// written as one partial row per workgroup.  With CDW = CDB = false none of that code
// exists in the kernel ([frozen], Key Changes).
// ------------------------------------------------------------------------------------
// Add the R teams' per-thread accumulators in LDS, in team order, and let team 0
// write the workgroup's partial row.  LDS layout [team-1][element][thread] keeps the
// 64 lanes of a wave on 64 consecutive words (no bank conflicts).
template <int V, bool VEC, int EVE, int DX>
__device__ __forceinline__ void combine_store(float (&acc)[V], float* dst, float* part, int r, int R,
                                              int t, int T, int N) {
  using FX = Frag<DX, V, EVE, VEC>;
  if (R > 1) {
    if (r > 0) {
#pragma unroll
      for (int i = 0; i < V; ++i) part[((r - 1) * V + i) * T + t] = acc[i];
    }
    __syncthreads();
    if (r == 0) {
      for (int q = 1; q < R; ++q) {
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += part[((q - 1) * V + i) * T + t];
      }
    }
  }
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int c = FX::col(i, t, T);
      if (c < N) dst[c] = acc[i];
    }
  }
}

template <int OP, int DX, int DW, int V, bool VEC, bool CDW, bool CDB>
__global__ __launch_bounds__(max_wg(V)) void bwd_kernel(BwdArgs p) {
  constexpr int EVE = 16 / Ty<DX>::B;
  using FX = Frag<DX, V, EVE, VEC>;
  using FW = Frag<DW, V, EVE, VEC>;
  static_assert(!(CDB && OP != OP_LN), "only LayerNorm has a bias");
  __shared__ double red[2][16][4];
  extern __shared__ float part[];
  int parity = 0;
  const int T = p.team;
  const int tid = threadIdx.x;
  const int r = tid / T;
  const int t = tid - r * T;
  const int R = blockDim.x / T;
  const int wpr = T >> 6;
  const int wave0 = (r * T) >> 6;
  const int N = p.N;
  const double inv_n = 1.0 / N;
  const double off = (OP == OP_LN) ? 0.0 : static_cast<double>(p.offset);

  float wv[V];
  {
    FW wf;
    wf.load(p.w, t, T, N, true);
#pragma unroll
    for (int i = 0; i < V; ++i) wv[i] = wf.get(i);
  }
  float dwacc[CDW ? V : 1];
  float dbacc[CDB ? V : 1];
#pragma unroll
  for (int i = 0; i < (CDW ? V : 1); ++i) dwacc[i] = 0.0f;
#pragma unroll
  for (int i = 0; i < (CDB ? V : 1); ++i) dbacc[i] = 0.0f;

  const int64_t row_begin = static_cast<int64_t>(blockIdx.x) * p.rows_per_wg;
  const int64_t row_end = min(row_begin + p.rows_per_wg, p.M);
  const int iters = (p.rows_per_wg + R - 1) / R;

  for (int it = 0; it < iters; ++it) {
    const int64_t row = row_begin + static_cast<int64_t>(it) * R + r;
    const bool valid = row < row_end;
    FX gf, xf;
    gf.load(static_cast<const typename Ty<DX>::S*>(p.dy) + row * p.lddy, t, T, N, valid);
    xf.load(static_cast<const typename Ty<DX>::S*>(p.x) + row * p.ldx, t, T, N, valid);
    float o[V];

    if constexpr (OP == OP_RMS || OP == OP_FADD) {
      FX df;
      if constexpr (OP == OP_FADD) {
        if (p.dres != nullptr)
          df.load(static_cast<const typename Ty<DX>::S*>(p.dres) + row * p.lddr, t, T, N, valid);
        else
          df.zero();
      }
      double acc[2] = {0.0, 0.0};  // sum x^2, sum g*x with g = dy * (w + offset)
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double xd = static_cast<double>(xf.get(i));
        const double gd = static_cast<double>(gf.get(i)) * (static_cast<double>(wv[i]) + off);
        acc[0] = fma(xd, xd, acc[0]);
        acc[1] = fma(gd, xd, acc[1]);
      }
      team_sum<2>(acc, wpr, wave0, red, parity);
      xf.opaque();
      gf.opaque();
      const double rstd = 1.0 / sqrt(acc[0] * inv_n + static_cast<double>(p.eps));
      // dx = rstd * (g - xhat * mean(g * xhat)) = rstd * (g - x * k), k = rstd^2 * mean(g * x)
      const double k = rstd * rstd * (acc[1] * inv_n);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double xd = static_cast<double>(xf.get(i));
        const double gd = static_cast<double>(gf.get(i)) * (static_cast<double>(wv[i]) + off);
        double dxd = fma(-xd, k, gd) * rstd;
        if constexpr (OP == OP_FADD) dxd += static_cast<double>(df.get(i));
        o[i] = static_cast<float>(dxd);
      }
      if constexpr (CDW) {
        if (valid) {
          const float rs = static_cast<float>(rstd);
#pragma unroll
          for (int i = 0; i < V; ++i) dwacc[i] = fmaf(gf.get(i), xf.get(i) * rs, dwacc[i]);
        }
      }
    } else {  // LayerNorm
      const typename Ty<DX>::S* xrow = static_cast<const typename Ty<DX>::S*>(p.x) + row * p.ldx;
      const double K = valid ? static_cast<double>(bits_to_f<DX>(xrow[0])) : 0.0;
      double acc[4] = {0.0, 0.0, 0.0, 0.0};  // sum d, sum d^2, sum g, sum g*d; d = x - K
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const bool in = FX::inb(i / FX::VE, t, T, N);
        const double d = in ? static_cast<double>(xf.get(i)) - K : 0.0;
        const double g = static_cast<double>(gf.get(i)) * static_cast<double>(wv[i]);
        acc[0] += d;
        acc[1] = fma(d, d, acc[1]);
        acc[2] += g;
        acc[3] = fma(g, d, acc[3]);
      }
      team_sum<4>(acc, wpr, wave0, red, parity);
      xf.opaque();
      gf.opaque();
      const double delta = acc[0] * inv_n;                 // mean - K
      const double var = fmax(acc[1] * inv_n - delta * delta, 0.0);
      const double rstd = 1.0 / sqrt(var + static_cast<double>(p.eps));
      const double mg = acc[2] * inv_n;                    // mean(g)
      const double mgd = acc[3] * inv_n - delta * mg;      // mean(g * (x - mean))
      const double c2 = mgd * rstd * rstd;             // xhat * mean(g*xhat) = (x-mean) * c2
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const bool in = FX::inb(i / FX::VE, t, T, N);
        const double e = (in ? static_cast<double>(xf.get(i)) - K : 0.0) - delta;
        const double g = static_cast<double>(gf.get(i)) * static_cast<double>(wv[i]);
        o[i] = static_cast<float>(fma(-e, c2, g - mg) * rstd);
      }
      if constexpr (CDW || CDB) {
        if (valid) {
#pragma unroll
          for (int i = 0; i < V; ++i) {
            if constexpr (CDW) {
              const bool in = FX::inb(i / FX::VE, t, T, N);
              const double e = (in ? static_cast<double>(xf.get(i)) - K : 0.0) - delta;
              dwacc[i] = fmaf(gf.get(i), static_cast<float>(e * rstd), dwacc[i]);
            }
            if constexpr (CDB) dbacc[i] += gf.get(i);
          }
        }
      }
    }
    FX of;
    of.pack(o);
    of.store_raw(static_cast<typename Ty<DX>::S*>(p.dx) + row * p.lddx, t, T, N, valid);
  }

  if constexpr (CDW) {
    combine_store<V, VEC, EVE, DX>(dwacc, p.ws + static_cast<int64_t>(blockIdx.x) * p.ldws, part,
                                  r, R, t, T, N);
  }
  if constexpr (CDB) {
    if constexpr (CDW) __syncthreads();  // LDS is reused after the dw pass
    combine_store<V, VEC, EVE, DX>(
        dbacc, p.ws + (static_cast<int64_t>(CDW ? p.P : 0) + blockIdx.x) * p.ldws, part, r, R, t, T, N);
  }
}

}  // namespace rn
