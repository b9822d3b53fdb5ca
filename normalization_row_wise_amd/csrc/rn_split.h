// rn_split.h — kernels for a few long rows (a decode step, a small batch): each row is
// spread over several workgroups.
//
// With one team per row, a single row of 18432 elements is the serial work of one CU
// (its fp64 passes alone take a few microseconds of that CU's vector ALUs) while the
// other CUs idle.  Here a row is cut into spans of SPLIT_WG 16-byte accesses (span s:
// lane t's access s * SPLIT_WG + t), and workgroup (c, i) of SPLIT_WG threads owns
// the `spans_per_wg` consecutive spans from c * spans_per_wg of row i.  It first walks
// the whole row and forms the row's sums itself, in the same order as every other
// workgroup of the row, so all of them hold bitwise-identical statistics and none
// waits for another.  The redundant reads come from the caches: the L2 for workgroups
// on one XCD, else the memory-side cache (when that would move many bytes across XCDs,
// a row's workgroups are renumbered onto one XCD: split_pos).  Then it writes its own
// spans of the outputs (the first one loaded before the walk, the next ones read again
// while the row's sums are reduced).  The arithmetic is the one of the row kernels
// (rn_kernels.h): fp64 sums, LayerNorm y and every dx formed in fp64 and rounded once,
// RMSNorm y in fp32 with the offset added to the weight in fp32 ([gemma], Summary).
//
// Parameter gradients: row i's products dy * xhat (and dy) for the span are written to
// partial row i, so the partial rows are the rows themselves (P = M) and the column
// sum adds them; a single row writes dw / db directly.
//
// Requirements (checked by the caller): 16-byte accesses (aligned rows, N a multiple
// of 16 / sizeof(element)), and no output that is also an input: another workgroup of
// the row may still be reading it.
#pragma once
#include "rn_kernels.h"

namespace rn {

#ifndef RN_SPLIT_U
#define RN_SPLIT_U 2
#endif
constexpr int SPLIT_WG = 256;         // threads per workgroup
constexpr int SPLIT_U = RN_SPLIT_U;   // spans per batch of the statistics walk (two batches in flight)
#ifndef RN_SPLIT_AHEAD
#define RN_SPLIT_AHEAD 4
#endif
// A workgroup's spans after the first: this many are read together right after the walk
// (their latency then overlaps the row reduction); any further ones one ahead of use.
constexpr int SPLIT_AHEAD = RN_SPLIT_AHEAD;

// Selects, at compile time, the output code path of a workgroup with more than one span.
template <bool B> struct SplitMore { static constexpr bool value = B; };

// Buffer resource over row `row` of a row tensor (N elements of SX).
template <typename SX>
__device__ __forceinline__ rsrc_t row_rsrc(const void* base, int64_t ld, int64_t row, int N) {
  return make_rsrc(static_cast<const SX*>(base) + row * ld, static_cast<uint32_t>(N) * sizeof(SX));
}

// Number of spans of a row of N elements of DX.
template <int DX> __device__ __forceinline__ int spans_of(int N) {
  constexpr int S = SPLIT_WG * (16 / Ty<DX>::B);
  return (N + S - 1) / S;
}

// Logical (span group c, row) of workgroup (blockIdx.x, blockIdx.y).  Workgroups are
// dealt to the 8 XCDs round-robin by linear id, so the workgroups of one row land on
// different XCDs and each fetches the row for its walk into its own L2.  GROUP renumbers
// them so that each XCD takes a contiguous block of logical ids: a row's workgroups then
// share one L2 and the row crosses to that XCD once.  A bijection for any grid.
template <bool GROUP> __device__ __forceinline__ void split_pos(int& c, int64_t& row) {
  if constexpr (!GROUP) {
    c = blockIdx.x;
    row = blockIdx.y;
  } else {
    const int W = gridDim.x * gridDim.y;
    const int k = blockIdx.y * gridDim.x + blockIdx.x;
    const int x = k & 7, slot = k >> 3;
    const int q = W >> 3, r = W & 7;  // XCDs below r take q + 1 workgroups, the others q
    const int L = x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
    c = L % gridDim.x;
    row = L / gridDim.x;
  }
}

// Forward.  grid = (workgroups per row, M).
template <int OP, int DX, int DW, bool GROUP>
__global__ __launch_bounds__(SPLIT_WG) void split_fwd_kernel(FwdArgs p) {
  constexpr int EVE = 16 / Ty<DX>::B;
  using FX = Frag<DX, EVE, EVE, true>;
  using FW = Frag<DW, EVE, EVE, true>;
  using SX = typename Ty<DX>::S;
  using SW = typename Ty<DW>::S;
  __shared__ double red[2][16][4];
  int parity = 0;
  const int t = threadIdx.x;
  int c;
  int64_t row;
  split_pos<GROUP>(c, row);
  const int N = p.N;
  const int NS = spans_of<DX>(N);
  const int s_first = c * p.spans_per_wg;
  const int s_end = min(s_first + p.spans_per_wg, NS);
  const double inv_n = 1.0 / N;
  const double pad = static_cast<double>(NS) * SPLIT_WG * EVE - N;

  const rsrc_t rx = row_rsrc<SX>(p.x, p.ldx, row, N);
  rsrc_t rr = rx;
  if constexpr (OP == OP_FADD) rr = row_rsrc<SX>(p.res, p.ldr, row, N);
  const uint32_t par_bytes = static_cast<uint32_t>(N) * sizeof(SW);
  const rsrc_t rw = make_rsrc(p.w, par_bytes);
  const rsrc_t rb = make_rsrc(p.b, p.b != nullptr ? par_bytes : 0u);  // no bias: zeros
  // inputs and parameters of one span of this workgroup
  struct Own {
    FX x, r;
    FW w, b;
  };
  auto load_own = [&](Own& o, int a) {
    o.x.load(rx, a, 0);
    if constexpr (OP == OP_FADD) o.r.load(rr, a, 0);
    o.w.load(rw, a, 0);
    if constexpr (OP == OP_LN) o.b.load(rb, a, 0);
  };
  Own first;  // loaded before the walk
  load_own(first, s_first * SPLIT_WG + t);
  const double K = OP == OP_LN ? first_elem<DX>(rx) : 0.0;

  // FusedAdd: the norm works on round(x + residual)
  auto summed = [&](FX& f, const FX& r) {
    if constexpr (OP == OP_FADD) {
      float s[EVE];
#pragma unroll
      for (int i = 0; i < EVE; ++i) s[i] = f.get(i) + r.get(i);
      f.pack(s);
    }
  };

  // statistics of the whole row: RMS sum x^2; LN sum d, sum d^2 with d = x - K.  Span
  // u of each batch adds into its own partial sums (independent chains of fp64 adds for
  // a workgroup of one wave per SIMD), combined in a fixed order after the walk.
  // The walk takes SPLIT_U spans per batch and loads the next batch before adding the
  // current one (loads past the row read zeros and are not added).
  double part[SPLIT_U][2];
#pragma unroll
  for (int u = 0; u < SPLIT_U; ++u) part[u][0] = part[u][1] = 0.0;
  struct Batch {
    FX x[SPLIT_U], r[SPLIT_U];
  };
  auto load_batch = [&](Batch& b, int s0) {
#pragma unroll
    for (int u = 0; u < SPLIT_U; ++u) {
      b.x[u].load(rx, (s0 + u) * SPLIT_WG + t, 0);
      if constexpr (OP == OP_FADD) b.r[u].load(rr, (s0 + u) * SPLIT_WG + t, 0);
    }
  };
  auto add_batch = [&](Batch& b, int s0) {
#pragma unroll
    for (int u = 0; u < SPLIT_U; ++u) {
      if (s0 + u >= NS) break;  // uniform
      summed(b.x[u], b.r[u]);
#pragma unroll
      for (int i = 0; i < EVE; ++i) {
        if constexpr (OP == OP_LN) {
          const double d = static_cast<double>(b.x[u].get(i)) - K;
          part[u][0] += d;
          part[u][1] = fma(d, d, part[u][1]);
        } else {
          const double v = static_cast<double>(b.x[u].get(i));
          part[u][0] = fma(v, v, part[u][0]);
        }
      }
    }
  };
  {
    Batch ba, bb;
    load_batch(ba, 0);
    for (int s0 = 0; s0 < NS; s0 += 2 * SPLIT_U) {
      load_batch(bb, s0 + SPLIT_U);
      add_batch(ba, s0);
      if (s0 + SPLIT_U >= NS) break;
      load_batch(ba, s0 + 2 * SPLIT_U);
      add_batch(bb, s0 + SPLIT_U);
    }
  }
  double acc[2] = {part[0][0], part[0][1]};
#pragma unroll
  for (int u = 1; u < SPLIT_U; ++u) {
    acc[0] += part[u][0];
    acc[1] += part[u][1];
  }
  // Reduction and output.  A workgroup of several spans reads the next ones (loads past
  // its spans or the row are harmless and unused) while the row's sums are reduced; a
  // one-span workgroup (a decode row) issues no such loads.  The two are separate code
  // paths, so neither waits for loads it does not use.
  auto finish = [&](auto more) {
    constexpr bool MORE = decltype(more)::value;
    Own ahead[MORE ? SPLIT_AHEAD : 1];
    if constexpr (MORE) {
#pragma unroll
      for (int k = 0; k < SPLIT_AHEAD; ++k) load_own(ahead[k], (s_first + 1 + k) * SPLIT_WG + t);
    }
    team_sum<2>(acc, SPLIT_WG / 64, 0, red, parity);

    double rstd, mean = 0.0;
    if constexpr (OP == OP_LN) {
      acc[0] = fma(pad, K, acc[0]);  // slots past N read as zero: d = -K each
      acc[1] = fma(-pad * K, K, acc[1]);
      const double delta = acc[0] * inv_n;
      const double var = fmax(acc[1] * inv_n - delta * delta, 0.0);
      rstd = rsqrt_d(var + static_cast<double>(p.eps));
      mean = K + delta;
    } else {
      rstd = rsqrt_d(acc[0] * inv_n + static_cast<double>(p.eps));
    }
    const float rs = static_cast<float>(rstd);
    if (c == 0 && t == 0) {
      if (p.rstd != nullptr) p.rstd[row] = rs;
      if constexpr (OP == OP_LN) {
        if (p.mean != nullptr) p.mean[row] = static_cast<float>(mean);
      }
    }
    const rsrc_t ry = row_rsrc<SX>(p.y, p.ldy, row, N);
    auto emit = [&](Own& in, int a) {
      summed(in.x, in.r);
      if constexpr (OP == OP_FADD) in.x.template store_raw<kNonTemporal>(row_rsrc<SX>(p.ro, p.ldro, row, N), a, 0);
      float o[EVE];
#pragma unroll
      for (int i = 0; i < EVE; ++i) {
        if constexpr (OP == OP_LN) {
          const double e = static_cast<double>(in.x.get(i)) - mean;
          o[i] = static_cast<float>(fma(e * rstd, static_cast<double>(in.w.get(i)),
                                        static_cast<double>(in.b.get(i))));
        } else {
          o[i] = (in.x.get(i) * rs) * (in.w.get(i) + p.offset);
        }
      }
      FX yf;
      yf.pack(o);
      yf.template store_raw<kNonTemporal>(ry, a, 0);
    };
    emit(first, s_first * SPLIT_WG + t);
    if constexpr (MORE) {
#pragma unroll
      for (int k = 0; k < SPLIT_AHEAD; ++k) {
        if (s_first + 1 + k < s_end) emit(ahead[k], (s_first + 1 + k) * SPLIT_WG + t);  // uniform
      }
      // any further spans, each one's loads issued before the previous span is written
      const int s_more = s_first + 1 + SPLIT_AHEAD;
      if (s_more < s_end) {
        Own cur;
        load_own(cur, s_more * SPLIT_WG + t);
#pragma unroll 1
        for (int sp = s_more; sp < s_end; ++sp) {
          Own nxt;
          load_own(nxt, (sp + 1) * SPLIT_WG + t);
          emit(cur, sp * SPLIT_WG + t);
          cur = nxt;
        }
      }
    }
  };
  if (s_end - s_first > 1) finish(SplitMore<true>{});
  else finish(SplitMore<false>{});
}

// Backward (stage 1).  grid = (workgroups per row, M).  pw / pb: row i of the partial
// rows (stride ldws), or dw / db themselves when M = 1.
template <int OP, int DX, int DW, bool CDW, bool CDB, bool XG, bool GROUP>
__global__ __launch_bounds__(SPLIT_WG) void split_bwd_kernel(BwdArgs p) {
  constexpr int EVE = 16 / Ty<DX>::B;
  using FX = Frag<DX, EVE, EVE, true>;
  using FW = Frag<DW, EVE, EVE, true>;
  using SX = typename Ty<DX>::S;
  using SW = typename Ty<DW>::S;
  static_assert(!(CDB && OP != OP_LN), "only LayerNorm has a bias");
  static_assert(!(XG && Ty<DW>::B != 2), "exact fp32 products need a 16-bit weight");
  __shared__ double red[2][16][4];
  int parity = 0;
  const int t = threadIdx.x;
  int c;
  int64_t row;
  split_pos<GROUP>(c, row);
  const int N = p.N;
  const int NS = spans_of<DX>(N);
  const int s_first = c * p.spans_per_wg;
  const int s_end = min(s_first + p.spans_per_wg, NS);
  const double inv_n = 1.0 / N;
  const double pad = static_cast<double>(NS) * SPLIT_WG * EVE - N;
  const double off = (OP == OP_LN) ? 0.0 : static_cast<double>(p.offset);

  const rsrc_t rg = row_rsrc<SX>(p.dy, p.lddy, row, N);
  const rsrc_t rx = row_rsrc<SX>(p.x, p.ldx, row, N);
  const rsrc_t rw = make_rsrc(p.w, static_cast<uint32_t>(N) * sizeof(SW));
  // no residual-output gradient: a zero-byte resource reads zeros
  const rsrc_t rd = OP == OP_FADD && p.dres != nullptr ? row_rsrc<SX>(p.dres, p.lddr, row, N)
                                                       : make_rsrc(p.dy, 0u);
  // inputs and weight of one span of this workgroup
  struct Own {
    FX g, x, d;
    FW w;
  };
  auto load_own = [&](Own& o, int a) {
    o.g.load(rg, a, 0);
    o.x.load(rx, a, 0);
    o.w.load(rw, a, 0);
    if constexpr (OP == OP_FADD) o.d.load(rd, a, 0);
  };
  Own first;  // loaded before the walk
  load_own(first, s_first * SPLIT_WG + t);
  const double K = OP == OP_LN ? first_elem<DX>(rx) : 0.0;

  // g = dy * (w + offset) in fp64 (the offset sum formed exactly), or the exact fp32
  // product when XG
  auto gval = [&](float dys, float w) -> double {
    if constexpr (XG) return static_cast<double>(dys * w);
    else if constexpr (OP == OP_LN) return static_cast<double>(dys) * static_cast<double>(w);
    else {
      const double dyd = static_cast<double>(dys);
      return fma(dyd, static_cast<double>(w), dyd * off);
    }
  };

  // statistics of the whole row: RMS sum x^2, sum g*x; LN sum d, sum d^2, sum g,
  // sum g*d with d = x - K (walked as in the forward: span u of each batch into its own
  // partial sums, combined in a fixed order; the next batch loaded before adding one)
  constexpr int NA = OP == OP_LN ? 4 : 2;
  double part[SPLIT_U][NA];
#pragma unroll
  for (int u = 0; u < SPLIT_U; ++u) {
#pragma unroll
    for (int j = 0; j < NA; ++j) part[u][j] = 0.0;
  }
  struct Batch {
    FX g[SPLIT_U], x[SPLIT_U];
    FW w[SPLIT_U];
  };
  auto load_batch = [&](Batch& b, int s0) {
#pragma unroll
    for (int u = 0; u < SPLIT_U; ++u) {
      const int a = (s0 + u) * SPLIT_WG + t;
      b.g[u].load(rg, a, 0);
      b.x[u].load(rx, a, 0);
      b.w[u].load(rw, a, 0);
    }
  };
  auto add_batch = [&](const Batch& b, int s0) {
#pragma unroll
    for (int u = 0; u < SPLIT_U; ++u) {
      if (s0 + u >= NS) break;  // uniform
#pragma unroll
      for (int i = 0; i < EVE; ++i) {
        const double g = gval(b.g[u].get(i), b.w[u].get(i));
        if constexpr (OP == OP_LN) {
          const double d = static_cast<double>(b.x[u].get(i)) - K;
          part[u][0] += d;
          part[u][1] = fma(d, d, part[u][1]);
          part[u][2] += g;
          part[u][3] = fma(g, d, part[u][3]);
        } else {
          const double xd = static_cast<double>(b.x[u].get(i));
          part[u][0] = fma(xd, xd, part[u][0]);
          part[u][1] = fma(g, xd, part[u][1]);
        }
      }
    }
  };
  {
    Batch ba, bb;
    load_batch(ba, 0);
    for (int s0 = 0; s0 < NS; s0 += 2 * SPLIT_U) {
      load_batch(bb, s0 + SPLIT_U);
      add_batch(ba, s0);
      if (s0 + SPLIT_U >= NS) break;
      load_batch(ba, s0 + 2 * SPLIT_U);
      add_batch(bb, s0 + SPLIT_U);
    }
  }
  double acc[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    acc[j] = part[0][j];
#pragma unroll
    for (int u = 1; u < SPLIT_U; ++u) acc[j] += part[u][j];
  }
  // Reduction and output.  A workgroup of several spans reads the next ones (loads past
  // its spans or the row are harmless and unused) while the row's sums are reduced; a
  // one-span workgroup (a decode row) issues no such loads.  The two are separate code
  // paths, so neither waits for loads it does not use.
  auto finish = [&](auto more) {
    constexpr bool MORE = decltype(more)::value;
    Own ahead[MORE ? SPLIT_AHEAD : 1];
    if constexpr (MORE) {
#pragma unroll
      for (int k = 0; k < SPLIT_AHEAD; ++k) load_own(ahead[k], (s_first + 1 + k) * SPLIT_WG + t);
    }
    team_sum<NA>(acc, SPLIT_WG / 64, 0, red, parity);

    // row constants: dx = rstd * g + c0 - x * cx (LN: c0 = -mean(g) * rstd and x taken
    // as x - mean; RMS: c0 = 0); xhat = x * rs + nmr (nmr = 0 for RMS)
    double rstd, cx, c0 = 0.0, mean = 0.0;
    if constexpr (OP == OP_LN) {
      acc[0] = fma(pad, K, acc[0]);  // slots past N: d = -K, g = 0
      acc[1] = fma(-pad * K, K, acc[1]);
      const double delta = acc[0] * inv_n;  // mean - K
      const double var = fmax(acc[1] * inv_n - delta * delta, 0.0);
      rstd = rsqrt_d(var + static_cast<double>(p.eps));
      mean = K + delta;
      const double mg = acc[2] * inv_n;                // mean(g)
      const double mgd = acc[3] * inv_n - delta * mg;  // mean(g * (x - mean))
      // dx = rstd * (g - mean(g) - (x - mean) * rstd^2 * mean(g * (x - mean)))
      cx = mgd * rstd * rstd * rstd;
      c0 = -mg * rstd;
    } else {
      rstd = rsqrt_d(acc[0] * inv_n + static_cast<double>(p.eps));
      // dx = rstd * (g - xhat * mean(g * xhat)) = rstd * g - c * x, c = rstd^3 * mean(g * x)
      cx = rstd * rstd * rstd * (acc[1] * inv_n);
    }
    const float rs = static_cast<float>(rstd);
    const float nmr = static_cast<float>(-mean * rstd);
    const rsrc_t rdx = row_rsrc<SX>(p.dx, p.lddx, row, N);
    // a span's products go to partial row `row` as 16-byte groups (N is a multiple of
    // EVE, so an access lies wholly inside the row or wholly past it, where stores vanish)
    auto put = [&](float* dst, const float (&v)[EVE], int a) {
      const rsrc_t rp = make_rsrc(dst + row * p.ldws, static_cast<uint32_t>(N) * 4u);
#pragma unroll
      for (int q = 0; q < EVE / 4; ++q) {
        const v4u w4 = {__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                        __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(w4, rp, (a * EVE + 4 * q) * 4, 0, 0);
      }
    };
    auto emit = [&](const Own& in, int a) {
      float o[EVE], dwp[EVE], dbp[EVE];
#pragma unroll
      for (int i = 0; i < EVE; ++i) {
        const float xs = in.x.get(i);
        const float dys = in.g.get(i);
        const double g = gval(dys, in.w.get(i));
        if constexpr (OP == OP_LN) {
          const double e = static_cast<double>(xs) - mean;
          o[i] = static_cast<float>(fma(-e, cx, fma(g, rstd, c0)));
          dwp[i] = dys * fmaf(xs, rs, nmr);
        } else {
          double dxd = fma(-static_cast<double>(xs), cx, g * rstd);
          if constexpr (OP == OP_FADD) dxd += static_cast<double>(in.d.get(i));
          o[i] = static_cast<float>(dxd);
          dwp[i] = dys * (xs * rs);
        }
        dbp[i] = dys;
      }
      FX of;
      of.pack(o);
      of.template store_raw<kNonTemporal>(rdx, a, 0);
      if constexpr (CDW) put(p.pw, dwp, a);
      if constexpr (CDB) put(p.pb, dbp, a);
    };
    emit(first, s_first * SPLIT_WG + t);
    if constexpr (MORE) {
#pragma unroll
      for (int k = 0; k < SPLIT_AHEAD; ++k) {
        if (s_first + 1 + k < s_end) emit(ahead[k], (s_first + 1 + k) * SPLIT_WG + t);  // uniform
      }
      // any further spans, each one's loads issued before the previous span is written
      const int s_more = s_first + 1 + SPLIT_AHEAD;
      if (s_more < s_end) {
        Own cur;
        load_own(cur, s_more * SPLIT_WG + t);
#pragma unroll 1
        for (int sp = s_more; sp < s_end; ++sp) {
          Own nxt;
          load_own(nxt, (sp + 1) * SPLIT_WG + t);
          emit(cur, sp * SPLIT_WG + t);
          cur = nxt;
        }
      }
    }
  };
  if (s_end - s_first > 1) finish(SplitMore<true>{});
  else finish(SplitMore<false>{});
}

}  // namespace rn
