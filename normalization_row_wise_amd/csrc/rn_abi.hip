// rn_abi.hip — the C ABI (include/rownorm.h): argument checks, launch shapes and
// dispatch to the kernel instances.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "../../include/rownorm.h"
#include "rn_instrument.h"
#include "rn_launch.h"

namespace rn {

// ------------------------------------------------------------------------------------
// Backward, stage 2: out[j] = sum over p = 0..P-1 of partial[p][j], in a fixed order:
// thread slice s sums p = s, s + 32, ... ascending, then the 32 slice sums are added as a
// fixed binary tree (s + 16, then + 8, + 4, + 2, + 1), so dw / db are bitwise
// reproducible.  blockIdx.y picks dw (0) or db (1).
// ------------------------------------------------------------------------------------
constexpr int CS_THREADS = 256;
constexpr int CS_C4 = 8;                  // float4 columns per workgroup: one 128-byte line
constexpr int CS_S = CS_THREADS / CS_C4;  // row slices per workgroup
constexpr int CS_BATCH = 8;               // loads a thread keeps in flight

__global__ __launch_bounds__(CS_THREADS) void colsum_kernel(const float* ws, int64_t ldws, int P,
                                                            int N, float* out0, float* out1) {
  __shared__ float4 sh[CS_S][CS_C4];
  const float* src = ws + (blockIdx.y ? static_cast<int64_t>(P) * ldws : 0);
  float* out = blockIdx.y ? out1 : out0;
  const int ci = threadIdx.x % CS_C4;
  const int s = threadIdx.x / CS_C4;
  const int c = (blockIdx.x * CS_C4 + ci) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < N) {
    const float* col = src + c;
    for (int q0 = s; q0 < P; q0 += CS_S * CS_BATCH) {
      float4 v[CS_BATCH];
#pragma unroll
      for (int k = 0; k < CS_BATCH; ++k) {
        const int q = q0 + k * CS_S;
        v[k] = q < P ? *reinterpret_cast<const float4*>(col + static_cast<int64_t>(q) * ldws)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < CS_BATCH; ++k) {
        acc.x += v[k].x;
        acc.y += v[k].y;
        acc.z += v[k].z;
        acc.w += v[k].w;
      }
    }
  }
  sh[s][ci] = acc;
#pragma unroll
  for (int h = CS_S / 2; h >= 1; h /= 2) {
    __syncthreads();
    if (s < h) {
      const float4 a = sh[s][ci];
      const float4 b = sh[s + h][ci];
      sh[s][ci] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
  }
  if (s == 0 && c < N) {
    const float4 tot = sh[0][ci];
    out[c] = tot.x;
    if (c + 1 < N) out[c + 1] = tot.y;
    if (c + 2 < N) out[c + 2] = tot.z;
    if (c + 3 < N) out[c + 3] = tot.w;
  }
}

}  // namespace rn

using namespace rn;

namespace {

// At most this many partial rows per parameter gradient.  The row-to-workgroup split
// depends only on (M, N), never on the device, so dw / db are bitwise reproducible.
// Rows of at most kNarrowN elements have small partial rows, and take more of them so
// that their many short rows spread over more workgroups.
#ifndef RN_MAX_PARTIALS
#define RN_MAX_PARTIALS 256
#endif
constexpr int64_t kMaxPartials = RN_MAX_PARTIALS;
constexpr int64_t kNarrowN = 256;
constexpr int64_t kMaxPartialsNarrow = 512;
inline int64_t max_partials(int64_t N) { return N <= kNarrowN ? kMaxPartialsNarrow : kMaxPartials; }
// Dynamic LDS a backward workgroup may use (gfx950 has 160 KiB per CU; 1 KiB is
// taken by the static row-reduction slots).
#ifndef RN_LDS_BUDGET
#define RN_LDS_BUDGET (156 * 1024)
#endif
constexpr size_t kLdsBudget = RN_LDS_BUDGET;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline int64_t ldws_of(int64_t N) { return round_up(N, 64); }

inline bool valid_dtype(int t) { return t == RN_F32 || t == RN_F16 || t == RN_BF16; }
inline int elem_bytes(int t) { return t == RN_F32 ? 4 : 2; }
inline int to_dt(int t) { return t == RN_F32 ? DT_F32 : (t == RN_F16 ? DT_F16 : DT_BF16); }

inline int check_types(rn_dtype xt, rn_dtype wt) {
  if (!valid_dtype(xt) || !valid_dtype(wt)) return RN_ERR_DTYPE;
  if (wt != xt && wt != RN_F32) return RN_ERR_DTYPE;
  return RN_OK;
}

inline int check_shape(int64_t M, int64_t N) {
  if (M < 0 || N < 1 || N > RN_MAX_N) return RN_ERR_SHAPE;
  if (M > (int64_t(1) << 40)) return RN_ERR_SHAPE;
  if (M * N > (int64_t(1) << 46)) return RN_ERR_SHAPE;
  return RN_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A row tensor allows 16-byte accesses if its base and (for M > 1) its row pitch are
// 16-byte multiples.  Null tensors (optional and absent) do not constrain.
inline bool vec_ok(const void* p, int64_t ld, int64_t M, int eb) {
  if (p == nullptr) return true;
  if (!aligned16(p)) return false;
  return M <= 1 || ((ld * eb) % 16) == 0;
}

// Elements per thread per row.  Preferred: 64 bytes of each row tensor per lane (32
// elements of a 16-bit type, 16 of fp32); the fused add moves more row tensors per
// element and prefers 16 elements of a 16-bit type (its backward then fits the next-row
// prefetch; measured faster at 2048 x 8192 bf16).  Narrow rows use the smallest V that
// still covers the row with one wave; wide rows move up to a larger V when the team
// would exceed the kernel's workgroup limit.  The choice never depends on which
// parameter gradients a backward computes: frozen and trainable calls lay the row out
// alike, add its sums in the same order and so give bit-identical dx.
inline int64_t team_of(int64_t N, int v) { return round_up(cdiv(N, v), 64); }

inline int max_wg(int kind, int v, int eb) { return kind == 0 ? fwd_max_wg(v, eb) : bwd_max_wg(v, eb); }

inline int pick_v(int kind, int op, int64_t N, int eb) {
  const int pref = eb == 2 ? (op == OP_FADD ? 16 : 32) : 16;
  for (int v : kVs) {
    if (v > pref) break;
    if (team_of(N, v) == 64) return v;  // one wave covers the row
  }
  for (int v : kVs) {
    if (v >= pref && team_of(N, v) <= max_wg(kind, v, eb)) return v;
  }
  return 0;
}

struct Shape {
  int v = 0;
  int team = 0;
  int ts = 0;              // sub-wave team width (0: teams of whole waves)
  int R = 1;               // teams per workgroup
  int64_t rows_per_wg = 1;
  int64_t grid = 0;
  int P = 0;               // partial rows (backward with grads)
  size_t shmem = 0;
  int acc = 0;             // backward with grads: accumulators in LDS (1; 2: stride 384),
                           // dW in LDS and dB in VGPRs (3), or both in VGPRs (0)
};

// Workgroups a forward launch aims for: enough to fill every CU many times over; at
// large M each workgroup then walks two rows per team with prefetch (measured best
// for 8192 x 8192 bf16: 46.0 us against 48.6 at four rows and 46.4 at one).
constexpr int64_t kTargetGrid = 4096;

// Narrow rows (N <= kNarrowN, 16-byte accesses possible): teams of 8, 16 or 32 lanes,
// several rows per wave, 8 elements per lane.  The workgroup's block of rows must stay
// addressable with 32-bit offsets (R rows of the widest row stride).  0: not narrow.
inline int narrow_team(int64_t N, bool vec, int64_t max_ld, int eb) {
  if (!vec || N > kNarrowN) return 0;
  const int ts = N <= 64 ? 8 : (N <= 128 ? 16 : 32);
  const int64_t r_max = 512 / ts;
  if (r_max * std::max(max_ld, N) * eb >= (int64_t(1) << 31)) return 0;
  return ts;
}

// kind: 0 forward, 1 backward with parameter grads, 2 backward without.
// ngrads: parameter gradients computed (kind 1).  vec: 16-byte accesses possible;
// max_ld: the widest row stride of the call's row tensors.
Shape plan(int kind, int op, int64_t M, int64_t N, int xt, int ngrads, bool vec, int64_t max_ld) {
  Shape s;
  const int eb = elem_bytes(xt);
  if (const int ts = narrow_team(N, vec, max_ld, eb)) {
    s.v = 8;
    s.team = ts;
    s.ts = ts;
    const int wg = kind == 1 ? 512 : 256;  // 512 = the LDS accumulator stride
    s.R = wg / ts;
    const int64_t R = s.R;
    int64_t rows;
    if (kind == 1) {
      s.acc = 1;
      s.shmem = static_cast<size_t>(ngrads) * 8 * 512 * sizeof(float);
      rows = cdiv(cdiv(M, R), max_partials(N)) * R;
    } else if (kind == 2) {
      rows = R;
    } else {
      rows = round_up(cdiv(M, kTargetGrid), R);
    }
    rows = std::max<int64_t>(rows, round_up(cdiv(M, int64_t(1) << 30), R));
    s.rows_per_wg = rows;
    s.grid = M > 0 ? cdiv(M, rows) : 0;
    s.P = kind == 1 ? static_cast<int>(s.grid) : 0;
    return s;
  }
  s.v = pick_v(kind, op, N, eb);
  s.team = static_cast<int>(team_of(N, s.v));
  const int wg_cap = max_wg(kind, s.v, eb);
  const int r_cap = wg_cap / s.team;
  int R;
  if (kind == 1) {
    // LDS accumulators: one [V][wg_cap] fp32 block per gradient, whatever R is
    const size_t block = static_cast<size_t>(ngrads) * s.v * wg_cap * sizeof(float);
    // both LayerNorm gradients at V = 48: blocks of stride 384 when the team fits in it
    const size_t block48 = static_cast<size_t>(ngrads) * s.v * kAccS48 * sizeof(float);
    if (block <= kLdsBudget) {
      s.acc = 1;
      R = r_cap;
      // RMSNorm over at least 8 rows per partial row, with teams of 64, 128 or 256
      // threads that cover at least 2048 elements of a row: 256-thread workgroups.
      // Graph-replayed trainable steps, us: 8192 x 8192 bf16 131.0 -> 127.1, 16384 x
      // 4096 bf16 131.8 -> 129.6, 8192 x 4096 fp16 71.3 -> 69.9, 8192 x 2048 fp32 69.7
      // -> 68.1, 8192 x 2048 bf16 41.5 -> 40.3, 2048 x 4096 bf16 28.1 -> 26.9; 2048 x
      // 8192 unchanged.  Slower: 64-thread teams over 1024 elements (8192 x 1024 25.9 ->
      // 26.2), 192-thread teams (8192 x 6144 100.7 -> 103.1) and LayerNorm (two
      // gradients; 8192 x 4096 78.9 -> 83.4).  The fused add gains from 32 rows per
      // partial row on (Gemma bf16: 8192 x 4096 109.6 -> 106.6, 16384 x 4096 208.7 ->
      // 204.5, 8192 x 2048 59.4 -> 58.7; 4096 x 4096 neutral).
      const int64_t min_rows = op == OP_RMS ? 8 * kMaxPartials : 32 * kMaxPartials;
      if (op != OP_LN && M >= min_rows && 256 % s.team == 0 &&
          static_cast<int64_t>(s.team) * s.v >= 2048)
        R = 256 / s.team;
      R = std::max(1, std::min(R, r_cap));
      s.shmem = block;
      // RMSNorm with one 256-thread team per workgroup: dW accumulates in registers (one
      // workgroup per CU leaves the VGPRs: 162 at V = 32) instead of a read-modify-write
      // of its LDS block per row.  Trainable 8192 x 8192 bf16 backward (both kernels,
      // events around the call) 91.6 -> 88.5 us.  Slower with several teams to combine
      // (LayerNorm 2048 x 4096 23.9 -> 36.1 us) and for the fused add's three-row ring
      // (2048 x 8192 37.6 -> 39.9 us), so only here.
      if (op == OP_RMS && R == 1 && s.team == 256 && (s.v == 16 || s.v == 32)) {
        s.acc = 0;
        s.shmem = 0;
      }
    } else if (s.v == 48 && ngrads == 2 && vec && s.team <= kAccS48 && block48 <= kLdsBudget) {
      s.acc = 2;
      R = 1;
      s.shmem = block48;
    } else if (s.v == 48 && ngrads == 2 && vec && block / 2 <= kLdsBudget) {
      // wider teams: dW's block in LDS, dB's accumulators in VGPRs
      s.acc = 3;
      R = r_cap;
      s.shmem = block / 2;
    } else {
      // accumulators in VGPRs; LDS only for the final team combine
      s.acc = 0;
      R = r_cap;
      while (R > 1 && static_cast<size_t>(R - 1) * s.v * s.team * sizeof(float) > kLdsBudget) --R;
      s.shmem = R > 1 ? static_cast<size_t>(R - 1) * s.v * s.team * sizeof(float) : 0;
    }
  } else if (kind == 2) {
    // frozen backward: workgroups of at least four waves
    R = std::max(1, std::min(256 / s.team, r_cap));
  } else {
    R = 1;
  }
  s.R = R;
  if (kind == 1) {
    const int64_t groups = cdiv(M, R);
    const int64_t pmax = max_partials(N);
    const int64_t rows = cdiv(groups, pmax) * R;
    s.rows_per_wg = std::max<int64_t>(rows, R);
    s.P = static_cast<int>(M > 0 ? cdiv(M, s.rows_per_wg) : 0);
    s.grid = s.P;
  } else {
    // forward: about kTargetGrid workgroups; frozen backward: one pass per workgroup
    // (short workgroups overlap each other's latency better than a persistent loop
    // without prefetch: 8192 x 8192 bf16 69.8 us against 75.7 at four rows per team)
    int64_t rows = kind == 2 ? R : round_up(cdiv(M, kTargetGrid), R);
    // keep the grid within the 2^31 workgroup limit for very tall inputs
    rows = std::max<int64_t>(rows, round_up(cdiv(M, int64_t(1) << 30), R));
    s.rows_per_wg = std::max<int64_t>(rows, R);
    s.grid = M > 0 ? cdiv(M, s.rows_per_wg) : 0;
  }
  return s;
}

// Split rows (rn_split.h): each row spread over workgroups of SPLIT_WG threads when the
// rows are too few to keep the CUs busy one team each (a decode row, a small batch).  A
// row is cut into spans of SPLIT_WG 16-byte accesses; every workgroup walks its whole
// row for the statistics and writes `spans` consecutive spans of the outputs.  A row
// takes at least two workgroups, and all rows' workgroups together stay within one per
// CU (so at most 128 rows).  The forward and both backward forms take the same
// decision; in the backward that makes dx come from the same kernel and the same sums
// with and without parameter gradients.  Needs 16-byte accesses and no output that is
// also an input.
#ifndef RN_SPLIT_MAX_WG
#define RN_SPLIT_MAX_WG 256
#endif
// A row's workgroups are renumbered onto one XCD (split_pos in rn_split.h) when their
// walks would read at least this many bytes beyond one walk per row; below it the
// renumbering measured neutral to slightly slower.  Graph-replayed fwd + bwd steps,
// trainable / frozen, us: fused add 32 x 16384 bf16 14.1 / 10.9 -> 12.1 / 9.0, RMSNorm
// 8 x 24576 fp32 12.9 / 10.1 -> 11.6 / 8.6, LayerNorm 8 x 16384 fp32 12.3 / 9.5 ->
// 11.3 / 8.2, LayerNorm 4 x 24576 fp32 13.9 / 11.0 -> 13.3 / 10.4.
#ifndef RN_SPLIT_GROUP_BYTES
#define RN_SPLIT_GROUP_BYTES (6 << 20)
#endif
struct Split {
  int64_t wgs = 0;     // workgroups per row (0: rows not split)
  int spans = 0;       // spans each workgroup writes
  bool group = false;  // a row's workgroups renumbered onto one XCD
};
inline Split split_plan(int op, int64_t M, int64_t N, int eb, bool vec, bool aliased) {
  Split sp;
  if (!vec || aliased) return sp;
  if (M > max_partials(N)) return sp;  // one partial row per row must fit the workspace
  const int64_t ns = cdiv(N, static_cast<int64_t>(SPLIT_WG) * (16 / eb));
  const int64_t g = std::min<int64_t>(ns, RN_SPLIT_MAX_WG / M);
  if (g < 2) return sp;
  const int64_t k = cdiv(ns, g);
  sp.spans = static_cast<int>(k);
  sp.wgs = cdiv(ns, k);
  // bytes the forward's walks read beyond one walk per row (x, and the residual)
  const int64_t extra = (sp.wgs - 1) * M * N * eb * (op == OP_FADD ? 2 : 1);
  sp.group = extra >= RN_SPLIT_GROUP_BYTES;
  return sp;
}

// Instrumentation (rn_instrument.h): per-thread dispatch timing events, [kernel][start,
// stop]; kernel 0 = forward, 1 = the backward's first kernel.
thread_local hipEvent_t t_timing[2][2] = {{nullptr, nullptr}, {nullptr, nullptr}};

inline int status_of(int ls) {
  return ls == LS_OK ? RN_OK : (ls == LS_HIP ? RN_ERR_HIP : RN_ERR_INTERNAL);
}

// Stage 2: the column sum of the partial rows (for M = 0: zero parameter gradients).
int colsum(const float* ws, int64_t ldws, int P, int64_t N, float* o0, float* o1,
           hipStream_t st) {
  const int n_out = (o0 != nullptr) + (o1 != nullptr);
  if (n_out == 0) return RN_OK;
  const dim3 grid(static_cast<unsigned>(cdiv(N, CS_C4 * 4)), n_out);
  int n = static_cast<int>(N);
  float* first = o0 != nullptr ? o0 : o1;
  void* args[] = {&ws, &ldws, &P, &n, &first, &o1};
  return hipLaunchKernel(reinterpret_cast<const void*>(colsum_kernel), grid, dim3(CS_THREADS), args,
                         0, st) == hipSuccess
             ? RN_OK
             : RN_ERR_HIP;
}

// ------------------------------------------------------------- no-allocation backward
// rmsnorm_bwd_noalloc keeps its partial rows of dW in this file-scope device array
// instead of a caller's workspace: every GPU the library runs on holds one copy of
// kScratchBytes until the process ends.  Host code uses the array only through the
// device address hipGetSymbolAddress returns for the current device (the name itself is
// a host-side stand-in).  Nothing in it needs to start at zero: every partial row a call
// reads is written earlier in the same call.  Calls that overlap on one GPU (different
// streams without ordering) share the array and race.
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, set once

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The current device's address of `scratch` (looked up on the first call on a device,
// with that device current).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RN_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return RN_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return RN_OK;
}

}  // namespace

extern "C" {

size_t rn_bwd_workspace_bytes(int64_t M, int64_t N, int n_param_grads) {
  if (check_shape(M, N) != RN_OK || n_param_grads <= 0 || n_param_grads > 2) return 0;
  return static_cast<size_t>(n_param_grads) * static_cast<size_t>(std::min(M, max_partials(N))) *
         static_cast<size_t>(ldws_of(N)) * sizeof(float);
}

const char* rn_status_str(int status) {
  switch (status) {
    case RN_OK: return "ok";
    case RN_ERR_NULL: return "a required pointer is NULL";
    case RN_ERR_SHAPE: return "invalid shape (need M >= 0 and 1 <= N <= RN_MAX_N)";
    case RN_ERR_DTYPE: return "invalid dtype (weight type must equal the I/O type or be F32)";
    case RN_ERR_STRIDE: return "a row stride is smaller than N";
    case RN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case RN_ERR_HIP: return "kernel launch failed";
    case RN_ERR_ALIAS: return "two outputs share storage";
    case RN_ERR_INTERNAL: return "internal error: no compiled kernel instance for this launch";
    case RN_ERR_SCRATCH:
      return "the no-allocation backward needs more than its fixed scratch (8 MiB of partial rows)";
    default: return "unknown status";
  }
}

int rn_set_timing_events(int kernel, hipEvent_t start, hipEvent_t stop) {
  if (kernel < 0 || kernel > 1) return RN_ERR_SHAPE;
  t_timing[kernel][0] = start;
  t_timing[kernel][1] = stop;
  return RN_OK;
}

// ---------------------------------------------------------------------------- forward

static int forward(int op, const void* x, int64_t ldx, const void* res, int64_t ldr,
                   const void* w, const void* b, void* y, int64_t ldy, void* ro, int64_t ldro,
                   float* rstd, float* mean, int64_t M, int64_t N, float eps, float offset,
                   rn_dtype xt, rn_dtype wt, hipStream_t st) {
  int e = check_types(xt, wt);
  if (e != RN_OK) return e;
  if ((e = check_shape(M, N)) != RN_OK) return e;
  if (M == 0) return RN_OK;
  if (x == nullptr || w == nullptr || y == nullptr) return RN_ERR_NULL;
  if (op == OP_FADD && (res == nullptr || ro == nullptr)) return RN_ERR_NULL;
  if (M > 1 && (ldx < N || ldy < N)) return RN_ERR_STRIDE;
  if (op == OP_FADD && M > 1 && (ldr < N || ldro < N)) return RN_ERR_STRIDE;
  if (op == OP_FADD && ro == y) return RN_ERR_ALIAS;
  if ((rstd != nullptr && rstd == mean)) return RN_ERR_ALIAS;
  if (M == 1) ldx = ldy = ldr = ldro = N;  // one row: its stride is never used (narrow
                                           // teams past the row must not wrap onto it)

  const int eb = elem_bytes(xt);
  const int ve = 16 / eb;
  bool vec = (N % ve) == 0 && vec_ok(x, ldx, M, eb) && vec_ok(y, ldy, M, eb) &&
             aligned16(w) && (b == nullptr || aligned16(b));
  if (op == OP_FADD) vec = vec && vec_ok(res, ldr, M, eb) && vec_ok(ro, ldro, M, eb);

  int64_t max_ld = std::max(ldx, ldy);
  if (op == OP_FADD) max_ld = std::max({max_ld, ldr, ldro});
  const bool aliased = y == x || (op == OP_FADD && (y == res || ro == x || ro == res));
  const Split sp = split_plan(op, M, N, eb, vec, aliased);
  const Shape s = plan(0, op, M, N, xt, 0, vec, max_ld);
  FwdArgs a{};
  a.x = x; a.ldx = ldx; a.res = res; a.ldr = ldr; a.w = w; a.b = b;
  a.y = y; a.ldy = ldy; a.ro = ro; a.ldro = ldro; a.rstd = rstd; a.mean = mean;
  a.M = M; a.N = static_cast<int>(N); a.team = s.team;
  a.rows_per_wg = static_cast<int>(s.rows_per_wg);
  a.eps = eps; a.offset = offset;
  a.spans_per_wg = sp.spans;
  Launch l{s.v, vec, s.ts, dim3(static_cast<unsigned>(s.grid)),
           dim3(static_cast<unsigned>(s.R * s.team)), 0};
  l.ev_start = t_timing[0][0];
  l.ev_stop = t_timing[0][1];
  if (sp.wgs > 0) {
    l.split = true;
    l.group = sp.group;
    l.grid = dim3(static_cast<unsigned>(sp.wgs), static_cast<unsigned>(M));
    l.block = dim3(SPLIT_WG);
  }
  const int dx = to_dt(xt), dw = to_dt(wt);
  if (op == OP_RMS) return status_of(launch_fwd_rms(dx, dw, l, a, st));
  if (op == OP_LN) return status_of(launch_fwd_ln(dx, dw, l, a, st));
  return status_of(launch_fwd_fadd(dx, dw, l, a, st));
}

int rmsnorm_fwd(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy, float* rstd,
                int64_t M, int64_t N, float eps, float offset, rn_dtype xt, rn_dtype wt,
                hipStream_t stream) {
  return forward(OP_RMS, x, ldx, nullptr, 0, w, nullptr, y, ldy, nullptr, 0, rstd, nullptr, M, N,
                 eps, offset, xt, wt, stream);
}

int layernorm_fwd(const void* x, int64_t ldx, const void* w, const void* b, void* y, int64_t ldy,
                  float* mean, float* rstd, int64_t M, int64_t N, float eps, rn_dtype xt,
                  rn_dtype wt, hipStream_t stream) {
  return forward(OP_LN, x, ldx, nullptr, 0, w, b, y, ldy, nullptr, 0, rstd, mean, M, N, eps, 0.0f,
                 xt, wt, stream);
}

int fused_add_rmsnorm_fwd(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                          const void* w, void* y, int64_t ldy, void* residual_out, int64_t ldro,
                          float* rstd, int64_t M, int64_t N, float eps, float offset, rn_dtype xt,
                          rn_dtype wt, hipStream_t stream) {
  return forward(OP_FADD, x, ldx, residual, ldr, w, nullptr, y, ldy, residual_out, ldro, rstd,
                 nullptr, M, N, eps, offset, xt, wt, stream);
}

// --------------------------------------------------------------------------- backward

static int backward(int op, const void* dy, int64_t lddy, const void* x, int64_t ldx,
                    const void* dres, int64_t lddr, const void* w, void* dx, int64_t lddx,
                    float* dw, float* db, void* ws, size_t ws_bytes, int64_t M, int64_t N,
                    float eps, float offset, rn_dtype xt, rn_dtype wt, hipStream_t st) {
  int e = check_types(xt, wt);
  if (e != RN_OK) return e;
  if ((e = check_shape(M, N)) != RN_OK) return e;
  const int ngrads = (dw != nullptr) + (db != nullptr);
  if (dw != nullptr && dw == db) return RN_ERR_ALIAS;
  if (ngrads > 0) {
    const size_t need = rn_bwd_workspace_bytes(M, N, ngrads);
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws))) return RN_ERR_WORKSPACE;
  }
  if (M > 0) {
    if (dy == nullptr || x == nullptr || w == nullptr || dx == nullptr) return RN_ERR_NULL;
    if (M > 1 && (lddy < N || ldx < N || lddx < N)) return RN_ERR_STRIDE;
    if (dres != nullptr && M > 1 && lddr < N) return RN_ERR_STRIDE;
  }
  if (M == 1) lddy = ldx = lddx = lddr = N;  // one row: its stride is never used
  const int64_t ldws = ldws_of(N);
  float* const part = static_cast<float*>(ws);
  if (M == 0) {  // parameter gradients of an empty batch are zero
    return colsum(part, ldws, 0, N, dw, db, st);
  }

  const int eb = elem_bytes(xt);
  const int ve = 16 / eb;
  const bool vec = (N % ve) == 0 && vec_ok(dy, lddy, M, eb) && vec_ok(x, ldx, M, eb) &&
                   vec_ok(dx, lddx, M, eb) && vec_ok(dres, lddr, M, eb) && aligned16(w);

  int64_t max_ld = std::max({lddy, ldx, lddx});
  if (dres != nullptr) max_ld = std::max(max_ld, lddr);
  const int kind = ngrads > 0 ? 1 : 2;
  const bool aliased = dx == dy || dx == x || (dres != nullptr && dx == dres);
  const Split sp = split_plan(op, M, N, eb, vec, aliased);
  const Shape s = plan(kind, op, M, N, xt, ngrads, vec, max_ld);
  // partial rows: one per workgroup, or one per row when rows are split
  const int P = sp.wgs > 0 ? static_cast<int>(M) : s.P;
  BwdArgs a{};
  a.dy = dy; a.lddy = lddy; a.x = x; a.ldx = ldx; a.dres = dres; a.lddr = lddr; a.w = w;
  a.dx = dx; a.lddx = lddx;
  // One partial row in all (a decode row, say): it is the gradient itself, written in
  // place of a partial row, and no column sum runs.  The kernels write 16-byte groups,
  // so this needs 16-byte aligned outputs.
  const bool direct = P == 1 && aligned16(dw) && aligned16(db);
  a.pw = direct ? dw : part;
  a.pb = direct ? db : part + (dw != nullptr ? static_cast<int64_t>(P) * ldws : 0);
  a.ldws = ldws;
  a.M = M; a.N = static_cast<int>(N); a.team = s.team;
  a.rows_per_wg = static_cast<int>(s.rows_per_wg);
  a.eps = eps; a.offset = offset;
  a.spans_per_wg = sp.spans;
  Launch l{s.v, vec, s.ts, dim3(static_cast<unsigned>(s.grid)),
           dim3(static_cast<unsigned>(s.R * s.team)), s.shmem};
  l.ev_start = t_timing[1][0];
  l.ev_stop = t_timing[1][1];
  if (sp.wgs > 0) {
    l.split = true;
    l.group = sp.group;
    l.grid = dim3(static_cast<unsigned>(sp.wgs), static_cast<unsigned>(M));
    l.block = dim3(SPLIT_WG);
    l.shmem = 0;
  }
  const int dxt = to_dt(xt), dwt = to_dt(wt);
  // exact fp32 products g = dy * w when the weight is 16-bit and nothing is added to it
  const bool xg = (wt != RN_F32) && (op == OP_LN || offset == 0.0f);
  const BwdVariant bv{dw != nullptr, db != nullptr, xg, s.acc};
  int ls;
  if (op == OP_RMS) ls = launch_bwd_rms(dxt, dwt, bv, l, a, st);
  else if (op == OP_LN) ls = launch_bwd_ln(dxt, dwt, bv, l, a, st);
  else ls = launch_bwd_fadd(dxt, dwt, bv, l, a, st);
  if ((e = status_of(ls)) != RN_OK) return e;
  if (ngrads == 0 || direct) return RN_OK;  // frozen, or the gradient written directly
  return colsum(part, ldws, P, N, dw, db, st);
}

int rmsnorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w, void* dx,
                int64_t lddx, float* dw, void* ws, size_t ws_bytes, int64_t M, int64_t N, float eps,
                float offset, rn_dtype xt, rn_dtype wt, hipStream_t stream) {
  return backward(OP_RMS, dy, lddy, x, ldx, nullptr, 0, w, dx, lddx, dw, nullptr, ws, ws_bytes, M,
                  N, eps, offset, xt, wt, stream);
}

int rmsnorm_bwd_noalloc(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w,
                        void* dx, int64_t lddx, float* dw, int64_t M, int64_t N, float eps,
                        float offset, rn_dtype xt, rn_dtype wt, hipStream_t stream) {
  if (dw == nullptr)  // frozen weight: no partial rows, nothing to hold
    return backward(OP_RMS, dy, lddy, x, ldx, nullptr, 0, w, dx, lddx, nullptr, nullptr, nullptr, 0,
                    M, N, eps, offset, xt, wt, stream);
  int e = check_shape(M, N);
  if (e != RN_OK) return e;
  if (rn_bwd_workspace_bytes(M, N, 1) > kScratchBytes) return RN_ERR_SCRATCH;
  void* ws = nullptr;
  if ((e = scratch_address(&ws)) != RN_OK) return e;
  return backward(OP_RMS, dy, lddy, x, ldx, nullptr, 0, w, dx, lddx, dw, nullptr, ws, kScratchBytes,
                  M, N, eps, offset, xt, wt, stream);
}

int layernorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w, void* dx,
                  int64_t lddx, float* dw, float* db, void* ws, size_t ws_bytes, int64_t M,
                  int64_t N, float eps, rn_dtype xt, rn_dtype wt, hipStream_t stream) {
  return backward(OP_LN, dy, lddy, x, ldx, nullptr, 0, w, dx, lddx, dw, db, ws, ws_bytes, M, N,
                  eps, 0.0f, xt, wt, stream);
}

int fused_add_rmsnorm_bwd(const void* dy, int64_t lddy, const void* dres_out, int64_t lddr,
                          const void* residual_out, int64_t ldro, const void* w, void* dx,
                          int64_t lddx, float* dw, void* ws, size_t ws_bytes, int64_t M, int64_t N,
                          float eps, float offset, rn_dtype xt, rn_dtype wt, hipStream_t stream) {
  return backward(OP_FADD, dy, lddy, residual_out, ldro, dres_out, lddr, w, dx, lddx, dw, nullptr,
                  ws, ws_bytes, M, N, eps, offset, xt, wt, stream);
}

}  // extern "C"
