// rn_kernels.h — forward and backward (stage 1) kernels.
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
// ALUs).  Every output whose value can cancel (LayerNorm y against the bias; every
// dx) is formed in fp64 from exact fp64 copies of the inputs and rounded once to the
// output type through fp32.  The backward recomputes the row statistics from x
// instead of reading a saved fp32 rstd: a rounded rstd would carry a 2^-24 relative
// error that the cancellation in g - xhat * mean(g * xhat) turns into whole-ulp
// errors of small dx values.  RMSNorm y (no cancellation) is formed in fp32.
//
// Work layout.  A team of T threads owns one row at a time (rn_device.h): T = 64 * W
// (whole waves), or T = TS = 8, 16 or 32 lanes for rows of at most 256 elements
// (several rows per wave).  A workgroup holds R teams and makes rows_per_wg / R
// passes.  Pass `it` of workgroup `b` takes rows (it * grid + b) * R .. + R - 1
// (grid-stride): the rows in flight across the chip at any moment form one contiguous
// window of the tensor, instead of one slice per workgroup scattered over all of it
// (measured faster at large M).  When a thread's share of the row tensors is small
// enough (fwd_prefetch, bwd_prefetch), the next row's tensors are loaded into a second
// register set before the current row is reduced (two rows in flight per team; three
// in the fused add's trainable backward, bwd_prefetch2).
// Columns past N inside the team's span are loaded as zeros; LayerNorm's shifted sums
// are corrected for them once per row.
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
  int spans_per_wg;                 // split rows (rn_split.h): spans each workgroup writes
};

struct BwdArgs {
  const void* dy; int64_t lddy;
  const void* x; int64_t ldx;       // x (RMS, LN) or residual_out (fused add)
  const void* dres; int64_t lddr;   // fused add: gradient reaching residual_out, may be null
  const void* w;
  void* dx; int64_t lddx;
  float* pw; float* pb; int64_t ldws;  // partial rows of dw and db: [P][ldws] each (when one
                                       // workgroup covers every row: dw and db themselves)
  int64_t M; int N; int team; int rows_per_wg;
  float eps, offset;
  int spans_per_wg;                 // split rows (rn_split.h): spans each workgroup writes
};

// Cache policy of the row tensors' loads and stores: non-temporal (cache-policy operand 2
// of the buffer instructions).  Each row element is read or written once per kernel, and
// streams that allocate in L2 and the memory-side cache only evict what is reused (the
// weight, the partial rows the column sum reads next).  Graph-replayed fwd + bwd steps,
// trainable / frozen, us, against the default policy: RMSNorm 8192 x 8192 bf16 130.1 /
// 121.0 -> 119.4-120.2 / 108.9-109.5, LayerNorm 2048 x 4096 bf16 33.2 / 25.3 -> 28.2-28.6
// / 20.9-21.2, FusedAdd 2048 x 8192 bf16 62.5 / 54.4 -> 56.3-56.7 / 48.9-49.3.  The fused
// add's forward keeps default loads (non-temporal they cost it about 1 us); non-temporal
// stores in the backward alone made the RMSNorm step slower (134.7 us).
constexpr int kNonTemporal = 2;
constexpr int fwd_load_pol(int op) { return op == OP_FADD ? 0 : kNonTemporal; }
constexpr int kFwdStorePol = kNonTemporal;
constexpr int kBwdLoadPol = kNonTemporal;
constexpr int kBwdStorePol = kNonTemporal;

// Register-budget policy (build-time tunable for launch-shape studies).
#ifndef RN_FWD_PF_BYTES
#define RN_FWD_PF_BYTES 64   // forward: prefetch the next row up to this many bytes per lane
#endif
#ifndef RN_BWD_PF_BYTES
#define RN_BWD_PF_BYTES 64   // backward with parameter gradients: as the forward
#endif
#ifndef RN_FROZEN_PF_BYTES
#define RN_FROZEN_PF_BYTES 0   // backward without: none (its many short-lived workgroups
#endif                         // hide the latency better)
#ifndef RN_FWD_BIG_WG_BYTES
#define RN_FWD_BIG_WG_BYTES 32   // forward: 1024-thread workgroups up to this many bytes per lane
#endif
#ifndef RN_BWD_BIG_WG_BYTES
#define RN_BWD_BIG_WG_BYTES 0    // backward: always 512 (its fp64 passes need the VGPRs)
#endif

// Bytes one thread holds of one row of one tensor.
constexpr int lane_bytes(int V, int B) { return V * B; }
// Two rows in flight per team when a thread's share is small enough.
constexpr bool fwd_prefetch(int V, int B) { return lane_bytes(V, B) <= RN_FWD_PF_BYTES; }
// `nin` row tensors are read per row (2, or 3 for the fused add's backward): the limit
// is for two, so a third tensor lowers it in proportion.
constexpr bool bwd_prefetch(int V, int B, bool grads, int nin) {
  return lane_bytes(V, B) * nin <= 2 * (grads ? RN_BWD_PF_BYTES : RN_FROZEN_PF_BYTES);
}
// The fused add's backward with parameter gradients keeps two rows in flight ahead of
// the one it reduces (three register sets).  Its three row tensors, read by at most one
// workgroup per CU, leave too few bytes in flight with one row ahead (graph-replayed
// fwd + bwd steps, bf16: 2048 x 8192 60.7 -> 58.4 us, 8192 x 4096 103.5 -> 101.1 us;
// fp16 with an fp32 weight 4096 x 4096 58.4 -> 56.8 us).  The two-tensor kernels gained
// nothing from it and some lost (LayerNorm fp32 4096 x 8192 137.6 -> 140.3 us, narrow
// rows 3-4 % slower); at V = 32, and with element accesses, the third set spills.
constexpr bool bwd_prefetch2(int op, int V, bool vec, bool prefetch, bool grads) {
  return prefetch && grads && vec && op == OP_FADD && V <= 16;
}
// Wider shares of 16-bit rows that still take one row ahead in a trainable backward
// with all accumulators in LDS: the fused add at V = 32, and RMSNorm / LayerNorm at V = 48
// with a 16-bit weight (WB = 2).  Their instances keep the second register set within
// 256 VGPRs without spilling; with an fp32 weight they spill and ran 45-60 % slower.
// Graph-replayed fwd + bwd steps, trainable, us: RMSNorm 4096 x 18432 bf16 171.6 ->
// 158.5, fp16 2048 x 20480 101.5 -> 93.3, fused add 2048 x 12288 bf16 90.6 -> 86.7,
// 2048 x 16384 bf16 Gemma 120.7 -> 115.9.
constexpr bool bwd_prefetch_wide(int op, int V, int B, int WB, bool vec, int acc, bool grads) {
  return grads && vec && (acc == 1 || acc == 2) && B == 2 &&
         ((op == OP_FADD && V == 32) || (op != OP_FADD && V == 48 && WB == 2));
}
// Largest workgroup a kernel is compiled for (sets its VGPR budget): 16 waves
// (128 VGPRs per lane) for small per-lane shares, 8 waves (256 VGPRs) above.
constexpr int fwd_max_wg(int V, int B) {
  return lane_bytes(V, B) <= RN_FWD_BIG_WG_BYTES ? 1024 : 512;
}
constexpr int bwd_max_wg(int V, int B) {
  return lane_bytes(V, B) <= RN_BWD_BIG_WG_BYTES ? 1024 : 512;
}
// LDS accumulator stride of the ACC = 2 instances (V = 48, one team of <= 384 threads).
constexpr int kAccS48 = 384;

// The row's first element (0 for a zero-byte resource).
template <int DX> __device__ __forceinline__ double first_elem(rsrc_t rs) {
  uint32_t b;
  if constexpr (Ty<DX>::B == 2) b = __builtin_amdgcn_raw_buffer_load_b16(rs, 0, 0, 0);
  else b = __builtin_amdgcn_raw_buffer_load_b32(rs, 0, 0, 0);
  return static_cast<double>(bits_to_f<DX>(b));
}

// Where one row of one tensor lives for this lane.  Whole-wave teams (TS = 0): a buffer
// resource over exactly that row (rows are uniform per wave).  Teams narrower than a
// wave (TS = 8, 16 or 32 lanes: several rows per wave): one resource over the
// workgroup's block of rows for the pass, plus this lane's row offset; columns past N
// are masked per access.  Either way rows past M read zeros and their stores vanish.
struct RowAt {
  rsrc_t rs;
  uint32_t base;
};

template <typename SX, int TS>
__device__ __forceinline__ RowAt row_at(const void* base, int64_t ld, int64_t row, int64_t row0,
                                        int R, int r, int N, int64_t M) {
  constexpr uint32_t B = sizeof(SX);
  if constexpr (TS == 0) {
    return {make_rsrc(static_cast<const SX*>(base) + row * ld,
                      row < M ? static_cast<uint32_t>(N) * B : 0u), 0u};
  } else {
    // the block holds rows row0 .. row0 + R - 1; only the first nv exist
    const int64_t nv = min(max(M - row0, int64_t(0)), static_cast<int64_t>(R));
    const uint32_t bytes = nv > 0 ? static_cast<uint32_t>(((nv - 1) * ld + N) * B) : 0u;
    return {make_rsrc(static_cast<const SX*>(base) + row0 * ld, bytes),
            static_cast<uint32_t>(r * ld * B)};
  }
}

template <int TS, int POL = 0, typename F>
__device__ __forceinline__ void frag_load(F& f, const RowAt& a, int t, int T, int N) {
  if constexpr (TS == 0) f.template load<POL>(a.rs, t, T);
  else f.template load_at<POL>(a.rs, a.base, t, T, N);
}
template <int TS, int POL = 0, typename F>
__device__ __forceinline__ void frag_store(const F& f, const RowAt& a, int t, int T, int N) {
  if constexpr (TS == 0) f.template store_raw<POL>(a.rs, t, T);
  else f.template store_at<POL>(a.rs, a.base, t, T, N);
}
// The row's first element (0 past the end).
template <int DX, int TS> __device__ __forceinline__ double first_at(const RowAt& a) {
  if constexpr (TS == 0) {
    return first_elem<DX>(a.rs);
  } else {
    uint32_t b;
    if constexpr (Ty<DX>::B == 2) b = __builtin_amdgcn_raw_buffer_load_b16(a.rs, a.base, 0, 0);
    else b = __builtin_amdgcn_raw_buffer_load_b32(a.rs, a.base, 0, 0);
    return static_cast<double>(bits_to_f<DX>(b));
  }
}
// Row sums over the team: DPP inside a lane group, or across waves through LDS.
template <int TS, int NV>
__device__ __forceinline__ void row_sum(double (&v)[NV], int wpr, int wave0, double (*red)[16][4],
                                        int& parity) {
  if constexpr (TS == 0) team_sum<NV>(v, wpr, wave0, red, parity);
  else group_sum<TS, NV>(v);
}

// ------------------------------------------------------------------------------------
// Forward.
// ------------------------------------------------------------------------------------
template <int OP, int DX, int DW, int V, bool VEC, int TS = 0>
__global__ __launch_bounds__(fwd_max_wg(V, Ty<DX>::B)) void fwd_kernel(FwdArgs p) {
  constexpr int EVE = 16 / Ty<DX>::B;
  constexpr bool PF = fwd_prefetch(V, Ty<DX>::B);
  using FX = Frag<DX, V, EVE, VEC>;
  using FW = Frag<DW, V, EVE, VEC>;
  using SX = typename Ty<DX>::S;
  __shared__ double red[2][16][4];
  int parity = 0;
  const int T = TS > 0 ? TS : p.team;
  const int tid = threadIdx.x;
  const int r = tid / T;
  const int t = tid - r * T;
  const int R = blockDim.x / T;
  const int wpr = T >> 6;
  const int wave0 = (r * T) >> 6;
  const int N = p.N;
  const double inv_n = 1.0 / N;
  const double pad = static_cast<double>(T * V - N);  // zero-filled slots of the span

  const uint32_t par_bytes = static_cast<uint32_t>(N) * Ty<DW>::B;

  // Parameters of this thread's columns, loaded once per workgroup.  LayerNorm keeps w
  // and b as loaded (16-bit words are unpacked on use: half the VGPRs of fp32 copies,
  // which lets the bf16 instance run four waves per SIMD); the RMS forms hold
  // w + offset in fp32.
  float wv[OP == OP_LN ? 1 : V];
  FW wf, bf;
  wf.load(make_rsrc(p.w, par_bytes), t, T);
  if constexpr (OP == OP_LN) {
    if (p.b != nullptr)
      bf.load(make_rsrc(p.b, par_bytes), t, T);
    else
      bf.zero();
  } else {
    // [gemma] Summary: offset added to the weight in fp32, inside the kernel.
#pragma unroll
    for (int i = 0; i < V; ++i) wv[i] = wf.get(i) + p.offset;
  }

  const int64_t row_end = p.M;
  const int iters = (p.rows_per_wg + R - 1) / R;

  struct In {
    FX x;
    FX res;
    double k;
  };
  // whole-wave teams: the row is uniform per wave; narrower teams: one row per lane group
  auto row0_of = [&](int it) {
    return uniform((static_cast<int64_t>(it) * gridDim.x + blockIdx.x) * R);
  };
  auto row_of = [&](int it) {
    const int64_t row = (static_cast<int64_t>(it) * gridDim.x + blockIdx.x) * R + r;
    if constexpr (TS == 0) return uniform(row);
    else return row;
  };
  auto at = [&](const void* base, int64_t ld, int it) {
    return row_at<SX, TS>(base, ld, row_of(it), row0_of(it), R, r, N, row_end);
  };
  auto load = [&](In& in, int it) {
    const RowAt ax = at(p.x, p.ldx, it);
    frag_load<TS, fwd_load_pol(OP)>(in.x, ax, t, T, N);
    if constexpr (OP == OP_FADD) frag_load<TS, fwd_load_pol(OP)>(in.res, at(p.res, p.ldr, it), t, T, N);
    if constexpr (OP == OP_LN) in.k = first_at<DX, TS>(ax);
  };

  auto process = [&](In& in, int it) {
    const int64_t row = row_of(it);
    const bool valid = row < row_end;
    if constexpr (OP == OP_LN) {
      wf.opaque();
      bf.opaque();
    } else {
      opaque<V>(wv);
    }
    FX& xf = in.x;
    if constexpr (OP == OP_FADD) {
      float s[V];
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] = xf.get(i) + in.res.get(i);
      xf.pack(s);  // residual_out = round(x + residual); the norm works on this value
      frag_store<TS, kFwdStorePol>(xf, at(p.ro, p.ldro, it), t, T, N);
    }
    float o[V];
    if constexpr (OP == OP_RMS || OP == OP_FADD) {
      double acc[1] = {0.0};
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double v = static_cast<double>(xf.get(i));
        acc[0] = fma(v, v, acc[0]);
      }
      row_sum<TS, 1>(acc, wpr, wave0, red, parity);
      xf.opaque();
      const double rstd = rsqrt_d(acc[0] * inv_n + static_cast<double>(p.eps));
      const float rs = static_cast<float>(rstd);
#pragma unroll
      for (int i = 0; i < V; ++i) o[i] = (xf.get(i) * rs) * wv[i];
      if (valid && t == 0 && p.rstd != nullptr) p.rstd[row] = rs;
    } else {  // LayerNorm: shifted sums d = x - K with K the row's first element
      const double K = in.k;
      double acc[2] = {0.0, 0.0};
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double d = static_cast<double>(xf.get(i)) - K;
        acc[0] += d;
        acc[1] = fma(d, d, acc[1]);
      }
      row_sum<TS, 2>(acc, wpr, wave0, red, parity);
      xf.opaque();
      acc[0] = fma(pad, K, acc[0]);          // the zero-filled slots added -K each
      acc[1] = fma(-pad * K, K, acc[1]);     // ... and K^2 each to the squares
      const double delta = acc[0] * inv_n;
      const double var = fmax(acc[1] * inv_n - delta * delta, 0.0);
      const double rstd = rsqrt_d(var + static_cast<double>(p.eps));
      const double mean = K + delta;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double e = static_cast<double>(xf.get(i)) - mean;
        o[i] = static_cast<float>(
            fma(e * rstd, static_cast<double>(wf.get(i)), static_cast<double>(bf.get(i))));
      }
      if (valid && t == 0) {
        if (p.rstd != nullptr) p.rstd[row] = static_cast<float>(rstd);
        if (p.mean != nullptr) p.mean[row] = static_cast<float>(mean);
      }
    }
    FX yf;
    yf.pack(o);
    frag_store<TS, kFwdStorePol>(yf, at(p.y, p.ldy, it), t, T, N);
  };

  if constexpr (PF) {
    // The next row's loads are issued unconditionally (past the share they read
    // zeros): a load issued on one path only makes the wait before the current row's
    // data a full vmcnt(0), which also waits for the previous row's stores.
    In a, b;
    load(a, 0);
    for (int it = 0; it < iters; it += 2) {
      load(b, it + 1);
      process(a, it);
      if (it + 1 >= iters) break;
      load(a, it + 2);
      process(b, it + 1);
    }
  } else {
    In a;
    for (int it = 0; it < iters; ++it) {
      load(a, it);
      process(a, it);
    }
  }
}

// Parameter-gradient accumulators of one thread: V fp32 partial sums over the rows a
// team has processed, for the thread's V columns.  Two homes:
//   ACC = 0: registers (V VGPRs per gradient).
//   ACC = 1: the workgroup's LDS, a [V/4][S][4] block per gradient (S = the kernel's
//            largest workgroup): group j (elements 4j .. 4j+3) of workgroup thread tid
//            is the float4 at j * S + tid.  Each group is one 16-byte read-modify-write;
//            a wave's 64 lanes cover 1 KiB of consecutive words (no bank conflict),
//            and j * S * 16 is an immediate offset from one base register, so the
//            compiler sees that the groups do not overlap and can overlap their reads.
//            Only this thread touches its float4s: deterministic sums.
//   ACC = 2: as ACC = 1 with S = kAccS48 (V = 48 with teams of at most 384 threads):
//            both LayerNorm gradients' blocks then fit (144 KiB) where two blocks of
//            stride 512 (192 KiB) would not.
//   ACC = 3: both LayerNorm gradients at V = 48 with wider teams: dW in LDS as for
//            ACC = 1, dB in registers.
// Both add with one rounding: acc = fma(a, b, acc).
template <int V, int ACC, int S> struct Acc {
  static_assert(V % 4 == 0, "accumulators are kept in groups of four");
  float reg[ACC == 0 ? V : 1];
  float4* lds;  // ACC = 1: this thread's group 0

  // ACC = 1 needs no zeroing: the first pass stores instead of adding (`first`).
  __device__ __forceinline__ void init(float* block, int tid) {
    if constexpr (ACC == 0) {
#pragma unroll
      for (int i = 0; i < V; ++i) reg[i] = 0.0f;
    } else {
      lds = reinterpret_cast<float4*>(block) + tid;
    }
  }
  // acc[4j + k] += a[k] * b[k]; on the workgroup's first pass (uniform) the LDS copy is
  // written as fma(a, b, 0), the same value an add to a zeroed accumulator gives, which
  // saves the zeroing pass and one read.
  __device__ __forceinline__ void add4(int j, const float (&a)[4], const float (&b)[4],
                                       bool first) {
    if constexpr (ACC == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) reg[4 * j + k] = fmaf(a[k], b[k], reg[4 * j + k]);
    } else if (first) {
      lds[j * S] = make_float4(fmaf(a[0], b[0], 0.0f), fmaf(a[1], b[1], 0.0f),
                               fmaf(a[2], b[2], 0.0f), fmaf(a[3], b[3], 0.0f));
    } else {
      float4 v = lds[j * S];
      v.x = fmaf(a[0], b[0], v.x);
      v.y = fmaf(a[1], b[1], v.y);
      v.z = fmaf(a[2], b[2], v.z);
      v.w = fmaf(a[3], b[3], v.w);
      lds[j * S] = v;
    }
  }
  __device__ __forceinline__ float get(int i) const { return reg[i]; }  // ACC = 0
};

// Register accumulators (ACC = 0): the R teams' sums are added in team order through
// `part` and team 0 writes the workgroup's partial row `dst` (16-byte aligned; columns
// past N are not written).
template <int V, bool VEC, int EVE, int DX, int S>
__device__ __forceinline__ void combine_regs(const Acc<V, 0, S>& acc, float* dst, float* part, int r,
                                             int R, int t, int T, int N) {
  using FX = Frag<DX, V, EVE, VEC>;
  float tot[V];
#pragma unroll
  for (int i = 0; i < V; ++i) tot[i] = acc.get(i);
  if (R > 1) {
    if (r > 0) {
#pragma unroll
      for (int i = 0; i < V; ++i) part[((r - 1) * V + i) * T + t] = tot[i];
    }
    __syncthreads();
    if (r == 0) {
      for (int q = 1; q < R; ++q) {
#pragma unroll
        for (int i = 0; i < V; ++i) tot[i] += part[((q - 1) * V + i) * T + t];
      }
    }
  }
  if (r == 0) {
    if constexpr (VEC) {
      static_assert(FX::VE % 4 == 0, "16-byte accesses hold 4 or 8 elements");
      // elements 4 j .. 4 j + 3 are four adjacent columns of one access (VE = 4 or 8),
      // wholly inside or outside the row (N is a multiple of VE): one 16-byte store
      // each instead of four 4-byte stores whose lanes lie 32 bytes apart
#pragma unroll
      for (int j = 0; j < V / 4; ++j) {
        const int c0 = FX::col(4 * j, t, T);
        if (c0 < N)
          *reinterpret_cast<float4*>(dst + c0) =
              make_float4(tot[4 * j], tot[4 * j + 1], tot[4 * j + 2], tot[4 * j + 3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int c = FX::col(i, t, T);
        if (c < N) dst[c] = tot[i];
      }
    }
  }
}

// LDS accumulators (ACC = 1): the R teams' float4 of each group j and thread slot t are
// added in team order, in chunks of kCombineChunk teams when R is larger (sub-wave
// teams): first every chunk is summed in order into its first team's slot, then the
// chunk sums are added in order.  Either way a fixed order, independent of timing.
// Every thread of the workgroup takes part; each output float4 is written as one
// 16-byte store of four columns of the partial row `dst`.  The dW and dB blocks are
// combined in the same pass (LayerNorm 2048 x 4096 bf16 stage 1: 18.8 -> 18.4 us against
// one pass each).  The caller has synchronised the workgroup after the last
// accumulation.
constexpr int kCombineChunk = 8;

template <int V, bool VEC, int EVE, int DX, int S, int NB>
__device__ __forceinline__ void combine_lds(float* block, float* const (&dst)[NB], int R, int T,
                                            int N) {
  // NB gradients' blocks lie back to back ([NB][V/4][S] float4); both are combined in the
  // same pass, each in its own fixed team order
  using FX = Frag<DX, V, EVE, VEC>;
  constexpr int G = V / 4;
  constexpr int C = kCombineChunk;
  float4* b4 = reinterpret_cast<float4*>(block);
  const int nth = blockDim.x;
  const int tid = threadIdx.x;
  int step = 1;
  if (R > C) {
    const int nch = (R + C - 1) / C;
    for (int k = tid; k < G * T * nch; k += nth) {
      const int t = k % T;          // consecutive lanes: consecutive float4, no conflict
      const int cj = k / T;
      const int ch = cj % nch;
      const int j = cj / nch;
      const int nq = min(C, R - ch * C);
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        float4* src = b4 + (g * G + j) * S + ch * C * T + t;
        float4 a = src[0];
        for (int q = 1; q < nq; ++q) {
          const float4 b = src[q * T];
          a.x += b.x;
          a.y += b.y;
          a.z += b.z;
          a.w += b.w;
        }
        src[0] = a;
      }
    }
    __syncthreads();
    step = C;
  }
  for (int k = tid; k < G * T; k += nth) {
    const int t = k % T;
    const int j = k / T;
    float4 a[NB];
#pragma unroll
    for (int g = 0; g < NB; ++g) a[g] = b4[(g * G + j) * S + t];
    for (int q = step; q < R; q += step) {
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        const float4 b = b4[(g * G + j) * S + q * T + t];
        a[g].x += b.x;
        a[g].y += b.y;
        a[g].z += b.z;
        a[g].w += b.w;
      }
    }
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      if constexpr (VEC) {
        // a group lies inside one access of VE >= 4 contiguous columns, and N is a
        // multiple of VE: the group is wholly inside the row or wholly outside
        const int c0 = FX::col(4 * j, t, T);
        if (c0 < N) *reinterpret_cast<float4*>(dst[g] + c0) = a[g];
      } else {
        const float v[4] = {a[g].x, a[g].y, a[g].z, a[g].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = FX::col(4 * j + q, t, T);
          if (c < N) dst[g][c] = v[q];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Backward, stage 1: dx for every row, plus (CDW / CDB) per-thread fp32 accumulators of
// dw / db over the workgroup's rows, combined across the workgroup's teams and written
// as one partial row per workgroup.  With CDW = CDB = false none of that code exists in
// the kernel ([frozen], Key Changes).  dx does not depend on CDW, CDB or ACC.
// XG: the weight is a 16-bit type and no offset is added, so g = dy * w is exact as an
// fp32 product (at most 11 + 11 significant bits; exact unless it underflows fp32).
// ------------------------------------------------------------------------------------
template <int OP, int DX, int DW, int V, bool VEC, bool CDW, bool CDB, bool XG, int ACC,
          int TS = 0>
__global__ __launch_bounds__(bwd_max_wg(V, Ty<DX>::B)) void bwd_kernel(BwdArgs p) {
  constexpr int EVE = 16 / Ty<DX>::B;
  constexpr int NG = (CDW ? 1 : 0) + (CDB ? 1 : 0);
  constexpr bool PF = (TS == 0 && bwd_prefetch_wide(OP, V, Ty<DX>::B, Ty<DW>::B, VEC, ACC, NG > 0)) ||
                      bwd_prefetch(V, Ty<DX>::B, NG > 0, OP == OP_FADD ? 3 : 2);
  constexpr bool PF2 = bwd_prefetch2(OP, V, VEC, PF, NG > 0);
  using FX = Frag<DX, V, EVE, VEC>;
  using FW = Frag<DW, V, EVE, VEC>;
  using SX = typename Ty<DX>::S;
  static_assert(!(CDB && OP != OP_LN), "only LayerNorm has a bias");
  static_assert(!(XG && Ty<DW>::B != 2), "exact fp32 products need a 16-bit weight");
  static_assert(NG > 0 || ACC == 0, "accumulators only exist with parameter gradients");
  static_assert(ACC != 2 || (V == 48 && TS == 0), "the 384-stride blocks are for V = 48");
  static_assert(ACC != 3 || (CDW && CDB && TS == 0), "split homes are for dW and dB");
  __shared__ double red[2][16][4];
  // dynamic LDS (accumulator blocks, team combine, reducer tree), accessed as 16-byte
  // groups: declared as float4 so that it starts 16-byte aligned after the static slots
  extern __shared__ float4 part_lds[];
  float* const part = reinterpret_cast<float*>(part_lds);
  int parity = 0;
  const int T = TS > 0 ? TS : p.team;
  const int tid = threadIdx.x;
  const int r = tid / T;
  const int t = tid - r * T;
  const int R = blockDim.x / T;
  const int wpr = T >> 6;
  const int wave0 = (r * T) >> 6;
  const int N = p.N;
  const double inv_n = 1.0 / N;
  const double pad = static_cast<double>(T * V - N);
  const double off = (OP == OP_LN) ? 0.0 : static_cast<double>(p.offset);

  // The weight of this thread's columns.  Frozen instances keep it as loaded (16-bit
  // words unpacked on use: half the VGPRs of an fp32 copy, so more waves per SIMD); the
  // trainable ones, whose extra dW work makes them short of VALU issue rather than of
  // waves, keep an fp32 copy and save the unpacking, except at V = 48 with a 16-bit
  // weight and an fp64 weight path (an offset): there the copy made them spill
  // (RMSNorm 4096 x 18432 bf16 Gemma trainable step 187.1 -> 164.4 us kept packed).
  constexpr bool PACKW = NG == 0 || (V >= 48 && Ty<DW>::B == 2 && !XG);
  // The same budget argument for the row itself: a trainable launch of whole-wave
  // teams has at most one workgroup per CU (one partial row each, at most 256 of them),
  // so it can keep what the statistics pass derived from dy (V <= 32) and x (V <= 16)
  // alive for the output pass instead of unpacking and converting again (measured:
  // fused add 2048 x 8192 bf16 34.8 -> 33.4 us, LayerNorm 2048 x 4096 bf16 19.4 ->
  // 18.7 us).  Wider rows and the element-access instances would spill.
  constexpr bool KEEP_G = NG > 0 && VEC && TS == 0 && V <= 32;
  constexpr bool KEEP_X = NG > 0 && VEC && TS == 0 && V <= 16;
  FW wf;
  float wv[PACKW ? 1 : V];
  wf.load(make_rsrc(p.w, static_cast<uint32_t>(N) * Ty<DW>::B), t, T);
  if constexpr (!PACKW) {
#pragma unroll
    for (int i = 0; i < V; ++i) wv[i] = wf.get(i);
  }
  auto wget = [&](int i) -> float {
    if constexpr (PACKW) return wf.get(i);
    else return wv[i];
  };
  // Hide the weight's provenance at these points (see Frag::opaque); the fp32 copy is
  // refreshed once per row, the packed words also after the row reduction.
  auto wopaque = [&](bool after_reduction) {
    if constexpr (PACKW) wf.opaque();
    else if (!after_reduction) opaque<V>(wv);
  };
  // LDS accumulator blocks: [gradient][V/4][S][4]
  constexpr int S = ACC == 2 ? kAccS48 : bwd_max_wg(V, Ty<DX>::B);
  Acc<V, ACC >= 1 ? 1 : 0, S> accw;
  Acc<V, ACC == 1 || ACC == 2 ? 1 : 0, S> accb;
  if constexpr (CDW) accw.init(part, tid);
  if constexpr (CDB) accb.init(part + (CDW ? V * S : 0), tid);

  const int64_t row_end = p.M;
  const int iters = (p.rows_per_wg + R - 1) / R;

  // g = dy * (w + offset) in fp64 (the offset sum formed exactly), or the exact fp32
  // product when XG.
  auto gval = [&](float dys, int i) -> double {
    if constexpr (XG) return static_cast<double>(dys * wget(i));
    else if constexpr (OP == OP_LN) return static_cast<double>(dys) * static_cast<double>(wget(i));
    else {
      const double dyd = static_cast<double>(dys);
      return fma(dyd, static_cast<double>(wget(i)), dyd * off);
    }
  };

  struct In {
    FX g;   // dy
    FX x;   // x or residual_out
    FX d;   // fused add: dres_out
    double k;
  };
  auto row0_of = [&](int it) {
    return uniform((static_cast<int64_t>(it) * gridDim.x + blockIdx.x) * R);
  };
  auto row_of = [&](int it) {
    const int64_t row = (static_cast<int64_t>(it) * gridDim.x + blockIdx.x) * R + r;
    if constexpr (TS == 0) return uniform(row);
    else return row;
  };
  auto at = [&](const void* base, int64_t ld, int it) {
    return row_at<SX, TS>(base, ld, row_of(it), row0_of(it), R, r, N, row_end);
  };
  auto load = [&](In& in, int it) {
    const RowAt ax = at(p.x, p.ldx, it);
    frag_load<TS, kBwdLoadPol>(in.g, at(p.dy, p.lddy, it), t, T, N);
    frag_load<TS, kBwdLoadPol>(in.x, ax, t, T, N);
    if constexpr (OP == OP_FADD) {
      if (p.dres != nullptr)
        frag_load<TS, kBwdLoadPol>(in.d, at(p.dres, p.lddr, it), t, T, N);
      else
        in.d.zero();
    }
    if constexpr (OP == OP_LN) in.k = first_at<DX, TS>(ax);
  };

  auto process = [&](In& in, int it) {
    const int64_t row = row_of(it);
    const bool valid = row < row_end;
    wopaque(false);
    FX& gf = in.g;
    FX& xf = in.x;
    float o[V];
    if constexpr (OP == OP_RMS || OP == OP_FADD) {
      double acc[2] = {0.0, 0.0};  // sum x^2, sum g*x
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double xd = static_cast<double>(xf.get(i));
        const double gd = gval(gf.get(i), i);
        acc[0] = fma(xd, xd, acc[0]);
        acc[1] = fma(gd, xd, acc[1]);
      }
      row_sum<TS, 2>(acc, wpr, wave0, red, parity);
      if constexpr (!KEEP_X) xf.opaque();
      if constexpr (!KEEP_G) gf.opaque();
      wopaque(true);
      const double rstd = rsqrt_d(acc[0] * inv_n + static_cast<double>(p.eps));
      // dx = rstd * (g - xhat * mean(g * xhat)) = rstd * g - c * x, c = rstd^3 * mean(g * x)
      const double c = rstd * rstd * rstd * (acc[1] * inv_n);
      // rows past the share read zeros; a zero scale keeps them out of dw even when
      // rstd is infinite (eps = 0)
      const float rs = valid ? static_cast<float>(rstd) : 0.0f;
#pragma unroll
      for (int j = 0; j < V / 4; ++j) {
        float dyv[4], xh[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = 4 * j + k;
          const float xs = xf.get(i);
          const float dys = gf.get(i);
          double dxd = fma(-static_cast<double>(xs), c, gval(dys, i) * rstd);
          if constexpr (OP == OP_FADD) dxd += static_cast<double>(in.d.get(i));
          o[i] = static_cast<float>(dxd);
          dyv[k] = dys;
          xh[k] = xs * rs;
        }
        if constexpr (CDW) accw.add4(j, dyv, xh, it == 0);
      }
    } else {  // LayerNorm
      const double K = in.k;
      double acc[4] = {0.0, 0.0, 0.0, 0.0};  // sum d, sum d^2, sum g, sum g*d; d = x - K
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const double d = static_cast<double>(xf.get(i)) - K;
        const double g = gval(gf.get(i), i);
        acc[0] += d;
        acc[1] = fma(d, d, acc[1]);
        acc[2] += g;
        acc[3] = fma(g, d, acc[3]);
      }
      row_sum<TS, 4>(acc, wpr, wave0, red, parity);
      if constexpr (!KEEP_X) xf.opaque();
      if constexpr (!KEEP_G) gf.opaque();
      wopaque(true);
      acc[0] = fma(pad, K, acc[0]);          // zero-filled slots: d = -K, g = 0
      acc[1] = fma(-pad * K, K, acc[1]);
      const double delta = acc[0] * inv_n;   // mean - K
      const double var = fmax(acc[1] * inv_n - delta * delta, 0.0);
      const double rstd = rsqrt_d(var + static_cast<double>(p.eps));
      const double mean = K + delta;
      const double mg = acc[2] * inv_n;                    // mean(g)
      const double mgd = acc[3] * inv_n - delta * mg;      // mean(g * (x - mean))
      // dx = rstd * (g - mean(g) - (x - mean) * rstd^2 * mean(g * (x - mean)))
      const double c2 = mgd * rstd * rstd * rstd;
      const double nmg = -mg * rstd;
      const float rs = valid ? static_cast<float>(rstd) : 0.0f;
      const float nmr = valid ? static_cast<float>(-mean * rstd) : 0.0f;
#pragma unroll
      for (int j = 0; j < V / 4; ++j) {
        float dyv[4], xh[4];
        const float one[4] = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = 4 * j + k;
          const float xs = xf.get(i);
          const float dys = gf.get(i);
          const double e = static_cast<double>(xs) - mean;
          o[i] = static_cast<float>(fma(-e, c2, fma(gval(dys, i), rstd, nmg)));
          dyv[k] = dys;
          xh[k] = fmaf(xs, rs, nmr);
        }
        if constexpr (CDW) accw.add4(j, dyv, xh, it == 0);
        if constexpr (CDB) accb.add4(j, dyv, one, it == 0);
      }
    }
    FX of;
    of.pack(o);
    frag_store<TS, kBwdStorePol>(of, at(p.dx, p.lddx, it), t, T, N);
  };

  if constexpr (PF2) {
    // as below, two rows ahead
    In a, b, c;
    load(a, 0);
    load(b, 1);
    for (int it = 0; it < iters; it += 3) {
      load(c, it + 2);
      process(a, it);
      if (it + 1 >= iters) break;
      load(a, it + 3);
      process(b, it + 1);
      if (it + 2 >= iters) break;
      load(b, it + 4);
      process(c, it + 2);
    }
  } else if constexpr (PF) {
    // The next row's loads are issued unconditionally (past the share they read
    // zeros): a load issued on one path only makes the wait before the current row's
    // data a full vmcnt(0), which also waits for the previous row's stores.
    In a, b;
    load(a, 0);
    for (int it = 0; it < iters; it += 2) {
      load(b, it + 1);
      process(a, it);
      if (it + 1 >= iters) break;
      load(a, it + 2);
      process(b, it + 1);
    }
  } else {
    In a;
    for (int it = 0; it < iters; ++it) {
      load(a, it);
      process(a, it);
    }
  }

  float* const dst_w = CDW ? p.pw + static_cast<int64_t>(blockIdx.x) * p.ldws : nullptr;
  float* const dst_b = CDB ? p.pb + static_cast<int64_t>(blockIdx.x) * p.ldws : nullptr;
  if constexpr (ACC == 3) {
    __syncthreads();  // every accumulation has landed
    float* const dsts[1] = {dst_w};
    combine_lds<V, VEC, EVE, DX, S, 1>(part, dsts, R, T, N);
    __syncthreads();  // `part` is reused by the register combine when R > 1
    combine_regs<V, VEC, EVE, DX, S>(accb, dst_b, part, r, R, t, T, N);
  } else if constexpr (NG > 0 && ACC >= 1) {
    __syncthreads();  // every accumulation has landed
    if constexpr (CDW && CDB) {
      float* const dsts[2] = {dst_w, dst_b};
      combine_lds<V, VEC, EVE, DX, S, 2>(part, dsts, R, T, N);  // both in one pass
    } else {
      float* const dsts[1] = {CDW ? dst_w : dst_b};
      combine_lds<V, VEC, EVE, DX, S, 1>(part, dsts, R, T, N);
    }
  } else {
    if constexpr (CDW) combine_regs<V, VEC, EVE, DX, S>(accw, dst_w, part, r, R, t, T, N);
    if constexpr (CDB) {
      if constexpr (CDW) __syncthreads();  // `part` is reused
      combine_regs<V, VEC, EVE, DX, S>(accb, dst_b, part, r, R, t, T, N);
    }
  }
}

}  // namespace rn
