// dl_abi.hip — the C ABI of the fused linear JSD distillation loss (include/distill.h):
// argument checks, workspace layout and the chunk loop ([distill], Summary and Details:
// tokens in chunks, the student head's weight gradient skipped when frozen).
//
// Per call: x_s^T once (dW); per chunk of C tokens: the two logits products (one launch),
// the per-token statistics, the logit gradient (bf16 columns of dz^T, fp32 column sums
// for db), the dx product (K-major operands: the chunk's columns of dz^T and W_s as
// stored); after the last chunk one dW product over all tokens.  The fp32 logits (2 C V)
// are the chunked memory; with dW, dz^T is kept for every token (2 bytes per token and
// vocabulary entry) so that dW is one product with K = tokens instead of an fp32
// read-modify-write of [V, H] per chunk; without it, for the chunk only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <set>
#include <utility>

#include "../../include/distill.h"
#include "dl_kernels.h"

using namespace dl;

namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Split of the dx product's K (= V) so that it has about one workgroup per CU (one fits
// at a time: the GEMM takes 144 KiB of LDS), a single round.  At 1024 tokens x 4096:
// 4 splits against 8 (two rounds, twice the fp32 partial slices to write and sum) took
// the call from 20.50 to 20.31 ms (trainable, V = 128256) and 15.89 to 15.73 ms
// (frozen); 6 splits (a round and a half) was slower than both.
inline int dx_splits(int64_t chunk, int64_t H) {
  const int64_t tiles = cdiv(chunk, BM) * cdiv(H, BN);
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(8, 256 / std::max<int64_t>(1, tiles))));
}

// Tokens per chunk: the caller's chunk (at most the batch and 2^22) rounded up to a
// multiple of 8, so that every chunk's first column of dz^T starts a 16-byte boundary
// (the dx product reads it as a K-major operand, 64 rows of it at a time with 32-bit
// offsets).  Chunking changes no value except the fixed summation order of db.
inline int64_t chunk_rows(int64_t chunk, int64_t BT) {
  return rup(std::min({chunk, std::max<int64_t>(BT, 1), int64_t(1) << 22}), 8);
}

// Byte offsets of the workspace parts (each 256-byte aligned); total in `end`.
struct Layout {
  size_t zs, zt, stats, dxp, gbt, xst, dbp, jt, end;
  int64_t C, ldz, vpad, ldt;  // ldt: row stride of dz^T (all tokens with dW, else a chunk)
  int splits;
};

Layout layout(int64_t BT, int64_t H, int64_t V, int64_t chunk, bool dx, bool dw, bool db) {
  Layout L{};
  const int64_t c = chunk_rows(chunk, BT);
  L.C = c;
  L.ldz = rup(V, 4);
  L.vpad = rup(V, 8);
  L.ldt = dw ? rup(std::max<int64_t>(BT, 1), 8) : c;
  L.splits = dx ? dx_splits(c, H) : 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = static_cast<size_t>(rup(static_cast<int64_t>(o + bytes), 256));
    return at;
  };
  L.zs = take(static_cast<size_t>(c) * L.ldz * 4);
  L.zt = take(static_cast<size_t>(c) * L.ldz * 4);
  L.stats = take(static_cast<size_t>(c) * 16);
  L.dxp = dx ? take(static_cast<size_t>(L.splits) * c * H * 4) : 0;
  L.gbt = (dx || dw) ? take(static_cast<size_t>(V) * L.ldt * 2) : 0;
  L.xst = dw ? take(static_cast<size_t>(H) * L.ldt * 2) : 0;
  L.dbp = db ? take(static_cast<size_t>(cdiv(c, GR_ROWS)) * V * 4) : 0;
  L.jt = take(static_cast<size_t>(std::max<int64_t>(BT, 1)) * 8);
  L.end = o;
  return L;
}

bool valid_sizes(int64_t BT, int64_t H, int64_t Ht, int64_t V, int64_t chunk, bool dw) {
  if (BT < 0 || H < 8 || Ht < 8 || V < 1 || chunk < 1) return false;
  if (H % 8 || Ht % 8) return false;
  // in-tile byte offsets of the products stay below 2^31: 256 rows of at most 2^22
  // elements (V padded, H, the input strides, the tokens padded for dW)
  if (V > (int64_t(1) << 22) - 8 || H > (int64_t(1) << 20) || Ht > (int64_t(1) << 20)) return false;
  if (BT > (int64_t(1) << 31)) return false;
  if (dw && rup(BT, 8) > (int64_t(1) << 22)) return false;
  // every buffer addressed with 32-bit byte offsets: the weights, a chunk's logits
  if (V * std::max(H, Ht) * 2 >= (int64_t(1) << 32)) return false;
  if (chunk_rows(chunk, BT) * rup(V, 4) * 4 >= (int64_t(1) << 32)) return false;
  // dz^T for a chunk (the dx product's K-major A operand)
  if (V * chunk_rows(chunk, BT) * 2 >= (int64_t(1) << 32)) return false;
  if (V * H * 4 >= (int64_t(1) << 32)) return false;  // dW
  return true;
}

inline bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename K, typename... Args>
int launch(K k, dim3 grid, dim3 block, size_t shmem, hipStream_t s, Args... args) {
  void* a[] = {&args...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, a, shmem, s) == hipSuccess
             ? RN_OK
             : RN_ERR_HIP;
}

// The GEMM's two LDS stages exceed the default dynamic LDS limit; raised once per device
// for both kernels.
bool allow_gemm_lds() {
  static std::mutex mu;
  static std::set<int> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> g(mu);
  if (done.count(dev)) return true;
  for (const void* k : {reinterpret_cast<const void*>(gemm_nt_kernel),
                        reinterpret_cast<const void*>(gemm_kk_kernel)}) {
    if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kGemmLds)) != hipSuccess)
      return false;
  }
  done.insert(dev);
  return true;
}

// Arguments of C[M x N] = A[M x K] B[N x K]^T (+ bias) with `splits` K ranges written to
// slices of C; `wgs` receives the product's workgroups per K range.  The tiles that share
// a tile of the larger operand run on one XCD (its L2 then fetches that tile once): the
// row tiles of a column tile when B is the larger (logits, dx), the column tiles of a
// row tile when A is (dW: 4.37 -> 4.27 ms at 128256 x 4096 x 4096, traced).
GemmArgs gemm_args(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                   int64_t ldc, int64_t split_stride, const uint16_t* bias, int64_t M, int64_t N,
                   int64_t K, int splits, int64_t& wgs) {
  const int by_rows = M > N ? 1 : 0;
  GemmArgs g{};
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.split_stride = split_stride; g.bias = bias;
  g.M = static_cast<int>(M); g.N = static_cast<int>(N); g.K = static_cast<int>(K);
  g.k_per_split = static_cast<int>(rup(cdiv(K, splits), BK));
  g.mt = static_cast<int>(cdiv(M, BM));
  g.nt = static_cast<int>(cdiv(N, BN));
  g.by_rows = by_rows;
  wgs = by_rows ? 8 * cdiv(g.mt, 8) * g.nt : 8 * cdiv(g.nt, 8) * g.mt;
  return g;
}

// One product.
int gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C, int64_t ldc,
         int64_t split_stride, const uint16_t* bias, int64_t M, int64_t N, int64_t K, int splits,
         hipStream_t s) {
  if (M == 0 || N == 0) return RN_OK;
  if (!allow_gemm_lds()) return RN_ERR_HIP;
  GemmLaunch gl{};
  int64_t wgs = 0;
  gl.p[0] = gemm_args(A, lda, B, ldb, C, ldc, split_stride, bias, M, N, K, splits, wgs);
  gl.p[1] = gl.p[0];
  gl.grid0 = static_cast<int>(wgs);
  const dim3 grid(static_cast<unsigned>(wgs), 1, static_cast<unsigned>(splits));
  return launch(gemm_nt_kernel, grid, dim3(GT), kGemmLds, s, gl);
}

// One product with K-major operands: A stored [K][M] (stride lda), B stored [K][N]
// (stride ldb); bases and strides 16-byte aligned.
int gemm_kk(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
            int64_t ldc, int64_t split_stride, int64_t M, int64_t N, int64_t K, int splits,
            hipStream_t s) {
  if (M == 0 || N == 0) return RN_OK;
  if (!allow_gemm_lds()) return RN_ERR_HIP;
  int64_t wgs = 0;
  const GemmArgs g = gemm_args(A, lda, B, ldb, C, ldc, split_stride, nullptr, M, N, K, splits, wgs);
  const dim3 grid(static_cast<unsigned>(wgs), 1, static_cast<unsigned>(splits));
  return launch(gemm_kk_kernel, grid, dim3(GT), kGemmLds, s, g);
}

// Two products of the same M x N (no split) in one launch: C0 = A0 B0^T (+ bias0) with
// K0, and C1 = A1 B1^T (+ bias1) with K1.
int gemm_pair(const uint16_t* A0, int64_t lda0, const uint16_t* B0, int64_t ldb0, float* C0,
              const uint16_t* bias0, int64_t K0, const uint16_t* A1, int64_t lda1,
              const uint16_t* B1, int64_t ldb1, float* C1, const uint16_t* bias1, int64_t K1,
              int64_t ldc, int64_t M, int64_t N, hipStream_t s) {
  if (M == 0 || N == 0) return RN_OK;
  if (!allow_gemm_lds()) return RN_ERR_HIP;
  GemmLaunch gl{};
  int64_t w0 = 0, w1 = 0;
  gl.p[0] = gemm_args(A0, lda0, B0, ldb0, C0, ldc, 0, bias0, M, N, K0, 1, w0);
  gl.p[1] = gemm_args(A1, lda1, B1, ldb1, C1, ldc, 0, bias1, M, N, K1, 1, w1);
  gl.grid0 = static_cast<int>(w0);
  return launch(gemm_nt_kernel, dim3(static_cast<unsigned>(w0 + w1)), dim3(GT), kGemmLds, s, gl);
}

// out[c][r] = in[r][c] for R x Cc, zeros for r in [R, Rpad)
int transpose(const uint16_t* in, int64_t ldi, int64_t R, int64_t Cc, uint16_t* out, int64_t ldo,
              int64_t Rpad, hipStream_t s) {
  return launch(transpose_bf16_kernel,
                dim3(static_cast<unsigned>(cdiv(Cc, 64)), static_cast<unsigned>(cdiv(Rpad, 64))),
                dim3(256), 0, s, in, ldi, static_cast<int>(R), static_cast<int>(Cc), out, ldo,
                static_cast<int>(Rpad));
}

}  // namespace

extern "C" {

size_t fused_linear_jsd_workspace_bytes(int64_t BT, int64_t H, int64_t Ht, int64_t V,
                                        int64_t chunk, int want_dx, int want_dw, int want_db) {
  if (!valid_sizes(BT, H, Ht, V, chunk, want_dw != 0)) return 0;
  return layout(BT, H, V, chunk, want_dx != 0, want_dw != 0, want_db != 0).end;
}

int fused_linear_jsd(const void* xs, int64_t ldxs, const void* ws_weight, const void* bs,
                     const void* xt, int64_t ldxt, const void* wt, const void* bt, int64_t BT,
                     int64_t H, int64_t Ht, int64_t V, float beta, float temperature,
                     int64_t chunk, float* loss, void* dxs, int64_t lddx, float* dws, float* dbs,
                     void* ws, size_t ws_bytes, hipStream_t st) {
  const bool want_dx = dxs != nullptr, want_dw = dws != nullptr, want_db = dbs != nullptr;
  if (!valid_sizes(BT, H, Ht, V, chunk, want_dw)) return RN_ERR_SHAPE;
  if (!(beta >= 0.0f && beta <= 1.0f) || !(temperature > 0.0f)) return RN_ERR_SHAPE;
  if (loss == nullptr || ws == nullptr) return RN_ERR_NULL;
  if (dbs != nullptr && bs == nullptr) return RN_ERR_NULL;
  const Layout L = layout(BT, H, V, chunk, want_dx, want_dw, want_db);
  if (ws_bytes < L.end || (reinterpret_cast<uintptr_t>(ws) & 255u)) return RN_ERR_WORKSPACE;
  if (BT > 0) {
    if (xs == nullptr || ws_weight == nullptr || xt == nullptr || wt == nullptr) return RN_ERR_NULL;
    if ((BT > 1 && (ldxs < H || ldxt < Ht)) || (want_dx && BT > 1 && lddx < H))
      return RN_ERR_STRIDE;
    if (ldxs % 8 || ldxt % 8 || ldxs > (int64_t(1) << 22) || ldxt > (int64_t(1) << 22))
      return RN_ERR_STRIDE;
    if (!a16(xs) || !a16(ws_weight) || !a16(xt) || !a16(wt)) return RN_ERR_STRIDE;
  }
  if (want_dw && dws == loss) return RN_ERR_ALIAS;

  char* base = static_cast<char*>(ws);
  float* zs = reinterpret_cast<float*>(base + L.zs);
  float* zt = reinterpret_cast<float*>(base + L.zt);
  float* stats = reinterpret_cast<float*>(base + L.stats);
  float* dxp = want_dx ? reinterpret_cast<float*>(base + L.dxp) : nullptr;
  uint16_t* gbt = (want_dx || want_dw) ? reinterpret_cast<uint16_t*>(base + L.gbt) : nullptr;
  uint16_t* xst = want_dw ? reinterpret_cast<uint16_t*>(base + L.xst) : nullptr;
  float* dbp = want_db ? reinterpret_cast<float*>(base + L.dbp) : nullptr;
  double* jt = reinterpret_cast<double*>(base + L.jt);
  const auto* Xs = static_cast<const uint16_t*>(xs);
  const auto* Ws = static_cast<const uint16_t*>(ws_weight);
  const auto* Bs = static_cast<const uint16_t*>(bs);
  const auto* Xt = static_cast<const uint16_t*>(xt);
  const auto* Wt = static_cast<const uint16_t*>(wt);
  const auto* Bt = static_cast<const uint16_t*>(bt);
  auto* Dx = static_cast<uint16_t*>(dxs);
  int e = RN_OK;

  if (BT == 0) {  // empty batch: loss 0, gradients 0
    if ((e = launch(loss_sum_kernel, dim3(1), dim3(1024), 0, st, static_cast<const double*>(jt),
                    int64_t(0), loss)) != RN_OK)
      return e;
    if (want_dw && (e = launch(fill_zero_kernel, dim3(static_cast<unsigned>(cdiv(V * H, 256))),
                               dim3(256), 0, st, dws, V * H)) != RN_OK)
      return e;
    if (want_db && (e = launch(fill_zero_kernel, dim3(static_cast<unsigned>(cdiv(V, 256))), dim3(256),
                               0, st, dbs, V)) != RN_OK)
      return e;
    return RN_OK;
  }

  // x_s^T [H][ldt] (zero columns past BT): the second operand of the dW product
  if (want_dw && (e = transpose(Xs, ldxs, BT, H, xst, L.ldt, L.ldt, st)) != RN_OK) return e;

  const bool want_grad = want_dx || want_dw || want_db;
  const float inv_tau = 1.0f / temperature;
  for (int64_t c0 = 0; c0 < BT; c0 += L.C) {
    const int64_t cr = std::min(L.C, BT - c0);
    const bool last = c0 + cr == BT;
    // logits of the chunk, both heads in one launch (fp32; the bias added in the epilogue).
    // Against one launch per head (1024 tokens x 4096): V = 151936 (2400 workgroups per
    // head, a last round a third full) 24.3-24.8 -> 23.9-24.0 ms trainable, 19.0-19.2 ->
    // 18.5-18.6 ms frozen; V = 128256 about 0.5 % faster.
    if ((e = gemm_pair(Xs + c0 * ldxs, ldxs, Ws, H, zs, Bs, H, Xt + c0 * ldxt, ldxt, Wt, Ht, zt, Bt,
                       Ht, L.ldz, cr, V, st)) != RN_OK)
      return e;
    // per token: log-sum-exps, J, A
    StatArgs sa{};
    sa.zs = zs; sa.zt = zt; sa.ldz = L.ldz; sa.stats = stats; sa.jtok = jt + c0;
    sa.rows = static_cast<int>(cr); sa.V = static_cast<int>(V);
    sa.beta = beta; sa.inv_tau = inv_tau;
    if ((e = launch(jsd_stats_kernel, dim3(static_cast<unsigned>(cr)), dim3(JT), 0, st, sa)) != RN_OK)
      return e;
    if (!want_grad) continue;
    // dL/dz: bf16 columns of dz^T (dx and dW: all tokens' columns with dW, the last chunk
    // also zeroing the token padding; the chunk's alone without), fp32 column sums per
    // 64 rows (db)
    const int64_t tok0 = want_dw ? c0 : 0;  // the chunk's first column of dz^T
    GradArgs ga{};
    ga.zs = zs; ga.zt = zt; ga.ldz = L.ldz; ga.stats = stats;
    ga.rows = static_cast<int>(cr); ga.V = static_cast<int>(V);
    ga.beta = beta; ga.inv_tau = inv_tau;
    ga.grad_scale = static_cast<float>(1.0 / (static_cast<double>(temperature) * static_cast<double>(BT)));
    ga.gbt = gbt; ga.ldt = L.ldt; ga.tok0 = tok0;
    ga.tok_rows = static_cast<int>(want_dw && last ? L.ldt - c0 : cr);
    ga.dbp = dbp;
    const int64_t grid_rows = std::max<int64_t>(cr, ga.tok_rows);
    if ((e = launch(jsd_grad_kernel,
                    dim3(static_cast<unsigned>(cdiv(L.vpad, GR_COLS)),
                         static_cast<unsigned>(cdiv(grid_rows, GR_ROWS))),
                    dim3(GR_T), 0, st, ga)) != RN_OK)
      return e;
    if (want_dx) {
      // dx[c0 .. c0 + cr) = dz W_s with K-major operands (dz^T's chunk columns, W_s as
      // stored): K = V in `splits` ranges, then their fixed-order sum
      if ((e = gemm_kk(gbt + tok0, L.ldt, Ws, H, dxp, H, cr * H, cr, H, V, L.splits, st)) != RN_OK)
        return e;
      if ((e = launch(split_sum_bf16_kernel, dim3(static_cast<unsigned>(cdiv(cr * H, 256))),
                      dim3(256), 0, st, static_cast<const float*>(dxp), cr * H, L.splits,
                      static_cast<int>(cr), static_cast<int>(H), H, Dx + c0 * lddx, lddx)) != RN_OK)
        return e;
    }
    if (want_db &&
        (e = launch(colsum_rows_kernel, dim3(static_cast<unsigned>(cdiv(V, 256))), dim3(256), 0, st,
                    static_cast<const float*>(dbp), V, static_cast<int>(cdiv(cr, GR_ROWS)),
                    static_cast<int>(V), dbs, static_cast<int>(c0 != 0))) != RN_OK)
      return e;
  }
  // dW = dz^T x_s over all tokens (K padded with zeros to a multiple of 8).  Skipped
  // entirely, with its buffers, for a frozen weight.
  if (want_dw && (e = gemm(gbt, L.ldt, xst, L.ldt, dws, H, 0, nullptr, V, H, L.ldt, 1, st)) != RN_OK)
    return e;
  return launch(loss_sum_kernel, dim3(1), dim3(1024), 0, st, static_cast<const double*>(jt), BT, loss);
}

}  // extern "C"
