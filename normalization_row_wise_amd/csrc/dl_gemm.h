// dl_gemm.h — bf16 matrix product on the MFMA units of gfx950 for the fused linear
// distillation loss: C[M x N] = A[M x K] * B[N x K]^T (+ bias[N]), fp32 accumulation and
// fp32 C.  Two operand layouts, both bf16 with row strides lda, ldb in elements:
//   gemm_nt_kernel: A stored [M][K] and B stored [N][K] (K contiguous);
//   gemm_kk_kernel: A stored [K][M] and B stored [K][N] (K-major: M, N contiguous).
// The products of the loss:
//   logits  z[C x V]  = x[C x H] * W[V x H]^T                         (NT)
//   dx      [C x H]   = dz[C x V] * W[V x H]: A = dz^T [V][C], B = W (K-major)
//   dW      [V x H]   = (dz^T)[V x T] * (x^T)[H x T]^T                  (NT; T: all tokens)
// so neither W nor dz is ever transposed for dx.
//
// Tiling.  A workgroup of 512 threads (eight waves in a 2 x 4 grid) owns a 256 x 256
// tile of C; each wave owns 128 x 64 of it as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16.
// Lane layout of that instruction (checked on the GPU): lane l holds A[l % 32][8 (l / 32)
// + e] and B^T[l % 32][8 (l / 32) + e] for e = 0..7, and accumulator r is
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  K advances 64 at a time through two LDS
// stages (rows padded to 72 elements, which keeps the 16-byte fragment reads free of
// bank conflicts): the next 256 x 64 slices of A and B are loaded from HBM into
// registers during the products of the current stage and written to the other stage
// after them, so one barrier per slice suffices.  Per CU and slice the LDS serves 192 KiB
// of fragment reads and 64 KiB of stores against 2 x 32 MFMAs per SIMD; the 128 x 128
// tile of four waves needed a third more LDS traffic per product and was 11-20 % slower
// on these shapes.  The two stages (144 KiB) leave room for one workgroup per CU.
// Loads go through buffer resources: rows past M (N) and columns past K read zero, so
// ragged edges need no branches; K must be a multiple of 8, and 256 rows of A or B must
// span less than 2^31 bytes (lda, ldb <= 2^22).
//
// K-major operands.  A 64-deep slice is 64 rows of 256 contiguous elements, stored in LDS
// at that shape (row pitch 288 elements, 576 bytes) and read with ds_read_b64_tr_b16,
// CDNA4's transposing LDS read: within each group of 16 lanes, lane i receives element e
// of the 8 bytes addressed by lane 4 e + i / 4, at position i % 4 (checked on the GPU).
// Lane j of a group addresses row k0 + j / 4, columns r0 + 4 (j % 4) .. + 3, so lane i
// gets rows k0 .. k0 + 3 of column r0 + i: half of the instruction's 8-deep fragment;
// two reads make a fragment.  Each 32-lane half of a read covers 4 rows x 64 bytes, the
// 64 banks once (measured: no bank conflicts).  The stage has the same size as the NT
// one.  A 16-byte load that crosses the end of its resource reads zero as a whole, so a
// slice's resource ends at column M (N) rounded up to 8 of its last row: every row of a
// K-major operand must be readable that far, and nothing past that is read.  Columns
// past M (N) may hold any values: they reach only rows (columns) of C that are not
// stored.  M, N strides and the operands' bases must be 16-byte aligned; K needs no
// padding.  Measured against the NT form on the same products: level at
// 1024 x 4096 x 128256 (split 4) and 4096^3.
//
// Placement.  Workgroups are dealt to the 8 XCDs round-robin by id.  The ids are mapped
// so that all row tiles of one column tile of C run on the same XCD at about the same
// time: the column tile of B is then fetched from HBM once into that XCD's L2 and reused
// by every row tile.  With `by_rows` the roles swap (all column tiles of one row tile on
// one XCD), for products whose A is the larger operand.
//
// Split K (grid.z > 1): workgroup z adds K range z and writes its own fp32 slice of C;
// a fixed-order sum of the slices follows (deterministic).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

struct GemmArgs {
  const uint16_t* A; int64_t lda;   // [M][lda] bf16 bits
  const uint16_t* B; int64_t ldb;   // [N][ldb] bf16 bits
  float* C; int64_t ldc;            // [M][ldc]; split K: slices of split_stride elements
  int64_t split_stride;
  const uint16_t* bias;             // [N] bf16 added to every row (slice 0 only), or null
  int M, N, K;
  int k_per_split;                  // multiple of 64
  int mt, nt;                       // row / column tiles of C
  int by_rows;                      // placement: 0 column tiles per XCD, 1 row tiles
};

constexpr int GT = 512;            // threads per workgroup
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LP = BK + 8;         // LDS row pitch in elements (144 bytes)
constexpr int kStage = (BM + BN) * LP;                          // elements per LDS stage
constexpr size_t kGemmLds = static_cast<size_t>(2) * kStage * 2;  // 147456 bytes, dynamic

// The size is the same in every lane but may be computed with vector instructions (a
// clamp becomes v_med3); readfirstlane keeps the resource in scalar registers, without
// which every load through it is compiled as a loop over the lanes' distinct resources.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           __builtin_amdgcn_readfirstlane(static_cast<int>(n)),
                                           0x00020000);
}

__device__ __forceinline__ float bf16_to_f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round to nearest even
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {f, 0.0f};
  return static_cast<uint16_t>(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2)) &
                               0xffffu);
}

// Tile (mi, ni) of workgroup `id` (see Placement).  Returns false for the ids that
// round the grid up to a multiple of 8 column tiles.
__device__ __forceinline__ bool tile_of(int id, int mt, int nt, int by_rows, int& mi, int& ni) {
  const int x = id & 7;
  const int q = id >> 3;
  if (by_rows) {
    ni = q % nt;
    mi = (q / nt) * 8 + x;
    return mi < mt;
  }
  mi = q % mt;
  ni = (q / mt) * 8 + x;
  return ni < nt;
}

// One launch computes one product, or two independent ones (the two heads' logits of a
// chunk): workgroups below `grid0` take p[0], the others p[1].  Each product's share of
// the grid is a multiple of 8 workgroups, so its placement over the XCDs is the same as
// in a launch of its own; the second product fills the first one's last partial round.
struct GemmLaunch {
  GemmArgs p[2];
  int grid0;  // workgroups of p[0] (all of them for a single product)
};

// The NT kernel keeps its own body: its schedule is tuned instruction by instruction, and
// sharing the tile code with the K-major form changed its code and cost 2-3 % on the
// logits products.
__global__ __launch_bounds__(GT) void gemm_nt_kernel(GemmLaunch gl) {
  extern __shared__ u32x4 gemm_lds[];
  uint16_t* const stage0 = reinterpret_cast<uint16_t*>(gemm_lds);
  const bool second = static_cast<int>(blockIdx.x) >= gl.grid0;  // uniform per workgroup
  const GemmArgs g = second ? gl.p[1] : gl.p[0];
  const int id = static_cast<int>(blockIdx.x) - (second ? gl.grid0 : 0);
  int mi, ni;
  if (!tile_of(id, g.mt, g.nt, g.by_rows, mi, ni)) return;  // uniform per workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = mi * BM, n0 = ni * BN;
  const int kb = blockIdx.z * g.k_per_split;
  const int ke = min(g.K, kb + g.k_per_split);

  // resources over the workgroup's rows of A and B (rows past M / N read zero)
  const rsrc_t ra = make_rsrc(g.A + static_cast<int64_t>(m0) * g.lda,
                              static_cast<uint64_t>(max(0, min(BM, g.M - m0))) * g.lda * 2);
  const rsrc_t rb = make_rsrc(g.B + static_cast<int64_t>(n0) * g.ldb,
                              static_cast<uint64_t>(max(0, min(BN, g.N - n0))) * g.ldb * 2);

  // global -> register staging: 256 rows x 64 elements = 2048 chunks of 8 elements per
  // operand; thread t takes chunks t + 512 i, i = 0..3
  u32x4 ra_st[4], rb_st[4];
  auto load_slice = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + GT * i;
      const int row = c >> 3;
      const int kc = k0 + (c & 7) * 8;
      const bool kin = kc < ke;
      const uint32_t oa = kin ? static_cast<uint32_t>((row * g.lda + kc) * 2) : 0x80000000u;
      const uint32_t ob = kin ? static_cast<uint32_t>((row * g.ldb + kc) * 2) : 0x80000000u;
      ra_st[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, oa, 0, 0);
      rb_st[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, ob, 0, 0);
    }
  };
  auto store_slice = [&](uint16_t* As) {
    uint16_t* Bs = As + BM * LP;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + GT * i;
      const int row = c >> 3;
      const int kc = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&As[row * LP + kc]) = ra_st[i];
      *reinterpret_cast<u32x4*>(&Bs[row * LP + kc]) = rb_st[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int arow = wm * 128 + (lane & 31);
  const int brow = wn * 64 + (lane & 31);
  const int kl = (lane >> 5) * 8;
  // The products of one slice, four 16-deep steps of 8 MFMAs.  The fragments of step
  // q + 1 are read during step q (two register sets), one read after each product, and
  // the next slice's 8 global loads are issued one per product of step 0: the scheduling
  // groups below fix that interleave (it measured 2-4 % faster than the compiler's own
  // order, which issued each step's reads in one block ahead of its products).
  auto multiply = [&](const uint16_t* As, bool more, int knext) {
    const uint16_t* Bs = As + BM * LP;
    bf16x8 af[2][4], bfr[2][2];
    auto frags = [&](int kk, int d) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[d][i] = *reinterpret_cast<const bf16x8*>(&As[(arow + 32 * i) * LP + kk + kl]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[d][j] = *reinterpret_cast<const bf16x8*>(&Bs[(brow + 32 * j) * LP + kk + kl]);
    };
    frags(0, 0);
#pragma unroll
    for (int q = 0; q < BK / 16; ++q) {
      const int cur = q & 1;
      if (q == 0 && more) load_slice(knext);  // in flight during the products
      if (q + 1 < BK / 16) frags(16 * (q + 1), cur ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
      if (q == 0 && more) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        }
      }
      if (q + 1 < BK / 16) {
#pragma unroll
        for (int t = 0; t < 6; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS fragment read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
  };

  if (kb < ke) {
    load_slice(kb);
    store_slice(stage0);
  }
  __syncthreads();
  int s = 0;
  for (int k0 = kb; k0 < ke; k0 += BK) {
    const bool more = k0 + BK < ke;
    multiply(stage0 + s * kStage, more, k0 + BK);  // also issues the next slice's loads
    // the other stage was last read before the previous barrier
    if (more) store_slice(stage0 + (s ^ 1) * kStage);
    __syncthreads();
    s ^= 1;
  }

  // epilogue: accumulator r of block (i, j) is C[m][n] with
  // m = m0 + 128 wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4, n = n0 + 64 wn + 32 j + lane % 32
  float* const c = g.C + blockIdx.z * g.split_stride;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + 32 * j + (lane & 31);
    if (n >= g.N) continue;
    const float bn = (g.bias != nullptr && blockIdx.z == 0) ? bf16_to_f(g.bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= g.M) continue;
        c[static_cast<int64_t>(m) * g.ldc + n] = acc[i][j][r] + bn;
      }
    }
  }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
constexpr int KP = BM + 32;  // K-major LDS row pitch (elements): 576 bytes
static_assert(BK * KP == BM * LP, "both layouts take the same LDS stage");

// K-major slice of one operand, global -> registers: K rows k0 .. k0 + nr - 1 of
// [K][ldx], columns r0 .. r0 + 255; the slice's resource ends at column R rounded up to
// 8 of its last row (a 16-byte load that crosses a resource's end reads zero as a
// whole).  Thread t takes 16-byte chunks t + 512 i, i = 0..3.
__device__ __forceinline__ void km_load(u32x4 (&st)[4], const uint16_t* X, int64_t ldx, int r0,
                                        int R, int k0, int ke, int tid) {
  const int nr = max(0, min(BK, ke - k0));
  const int64_t bytes =
      nr > 0 ? (static_cast<int64_t>(nr - 1) * ldx + ((max(0, R - r0) + 7) & ~7)) * 2 : 0;
  const rsrc_t rs = make_rsrc(X + static_cast<int64_t>(k0) * ldx + r0, static_cast<uint64_t>(bytes));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + GT * i;
    const int row = c >> 5;
    const uint32_t o = row < nr ? static_cast<uint32_t>((row * ldx + (c & 31) * 8) * 2) : 0x80000000u;
    st[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
  }
}
// ... and registers -> LDS at the slice's own shape, 64 rows of pitch KP
__device__ __forceinline__ void km_store(const u32x4 (&st)[4], uint16_t* S, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + GT * i;
    *reinterpret_cast<u32x4*>(&S[(c >> 5) * KP + (c & 31) * 8]) = st[i];
  }
}
// The fragment of rows rb .. rb + 31 (M or N) and depth kk + 8 (lane / 32) .. + 7: two
// transposing reads of 4 rows each.
__device__ __forceinline__ bf16x8 km_frag(const uint16_t* S, int rb, int kk, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int k = kk + 8 * (g >> 1) + (j >> 2);
  const int r = rb + 16 * (g & 1) + 4 * (j & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(S + k * KP + r));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(S + (k + 4) * KP + r));
  const v4i16 both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, both);
}

// C = A B with A stored [K][M] and B stored [K][N]: the NT kernel's tiling, placement,
// two-stage pipeline and epilogue (no bias), with K-major slices.
__global__ __launch_bounds__(GT) void gemm_kk_kernel(GemmArgs g) {
  extern __shared__ u32x4 gemm_lds_kk[];
  uint16_t* const stage0 = reinterpret_cast<uint16_t*>(gemm_lds_kk);
  int mi, ni;
  if (!tile_of(static_cast<int>(blockIdx.x), g.mt, g.nt, g.by_rows, mi, ni)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = mi * BM, n0 = ni * BN;
  const int kb = blockIdx.z * g.k_per_split;
  const int ke = min(g.K, kb + g.k_per_split);

  u32x4 ra_st[4], rb_st[4];
  auto load_slice = [&](int k0) {
    km_load(ra_st, g.A, g.lda, m0, g.M, k0, ke, tid);
    km_load(rb_st, g.B, g.ldb, n0, g.N, k0, ke, tid);
  };
  auto store_slice = [&](uint16_t* As) {
    km_store(ra_st, As, tid);
    km_store(rb_st, As + BM * LP, tid);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // As in the NT kernel, with 12 reads per 16-deep step (8 for A, 4 for B) spread one or
  // two per product.
  auto multiply = [&](const uint16_t* As, bool more, int knext) {
    const uint16_t* Bs = As + BM * LP;
    bf16x8 af[2][4], bfr[2][2];
    auto frags = [&](int kk, int d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) af[d][i] = km_frag(As, wm * 128 + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[d][j] = km_frag(Bs, wn * 64 + 32 * j, kk, lane);
    };
    frags(0, 0);
#pragma unroll
    for (int q = 0; q < BK / 16; ++q) {
      const int cur = q & 1;
      if (q == 0 && more) load_slice(knext);  // in flight during the products
      if (q + 1 < BK / 16) frags(16 * (q + 1), cur ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
      if (q == 0 && more) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        }
      }
      if (q + 1 < BK / 16) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one transposing read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    }
  };

  if (kb < ke) {
    load_slice(kb);
    store_slice(stage0);
  }
  __syncthreads();
  int s = 0;
  for (int k0 = kb; k0 < ke; k0 += BK) {
    const bool more = k0 + BK < ke;
    multiply(stage0 + s * kStage, more, k0 + BK);
    if (more) store_slice(stage0 + (s ^ 1) * kStage);
    __syncthreads();
    s ^= 1;
  }

  float* const c = g.C + blockIdx.z * g.split_stride;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + 32 * j + (lane & 31);
    if (n >= g.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= g.M) continue;
        c[static_cast<int64_t>(m) * g.ldc + n] = acc[i][j][r];
      }
    }
  }
}

}  // namespace dl
