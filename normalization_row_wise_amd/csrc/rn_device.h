// rn_device.h — device-side building blocks of the row-wise normalisation kernels
// (gfx950 / CDNA4, wave64).
//
// Layout of one row across a "team" of T threads (T a multiple of 64, one or more
// whole waves): each thread owns V elements, taken as V/VE loads of VE contiguous
// elements.  Load l of thread t covers columns (l*T + t)*VE .. +VE-1, so for every l
// the team reads one contiguous span of T*VE elements (fully coalesced 16-byte
// accesses when VE = 16 / sizeof(element)).  VE = 1 is the same code for rows that
// are not 16-byte aligned or whose length is not a multiple of the vector width.
//
// The whole row stays in VGPRs between the reduction and the output pass, so every
// tensor is read from HBM exactly once per kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rn {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum : int { OP_RMS = 0, OP_LN = 1, OP_FADD = 2 };

template <int DT> struct Ty;
template <> struct Ty<DT_F32> { using S = uint32_t; static constexpr int B = 4; };
template <> struct Ty<DT_F16> { using S = uint16_t; static constexpr int B = 2; };
template <> struct Ty<DT_BF16> { using S = uint16_t; static constexpr int B = 2; };

typedef float f2v __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

// Buffer resource over `bytes` bytes at `base` (raw, no stride; gfx9 word 3).  `base`
// must be uniform across the wave.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// A row index every lane of the wave agrees on, moved to scalar registers.
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// Stored bits (low 16 bits for 16-bit types) -> float.  Exact.
template <int DT> __device__ __forceinline__ float bits_to_f(uint32_t b) {
  if constexpr (DT == DT_F32) return __uint_as_float(b);
  else if constexpr (DT == DT_BF16) return __uint_as_float(b << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// Two floats -> one word holding two 16-bit values (a in the low half), round to
// nearest even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950).
template <int DT> __device__ __forceinline__ uint32_t pack2(float a, float b) {
  f2v v = {a, b};
  if constexpr (DT == DT_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2v));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2v));
}

// One float -> stored bits of DT (low 16 bits for 16-bit types), round to nearest even.
template <int DT> __device__ __forceinline__ uint32_t f_to_bits(float a) {
  if constexpr (DT == DT_F32) return __float_as_uint(a);
  else return pack2<DT>(a, 0.0f) & 0xffffu;
}

// V elements of one row of type DT owned by one thread.  VEC selects 16-byte loads
// (VE = 16 / sizeof) or element loads (VE = 1).  EVE is the element count per load
// of the row's I/O tensor; weights use the same column mapping with their own type.
template <int DT, int V, int EVE, bool VEC> struct Frag {
  static constexpr int B = Ty<DT>::B;
  static constexpr int VE = VEC ? EVE : 1;   // elements per access
  static constexpr int NL = V / VE;          // accesses per row
  static constexpr int WPL = VEC ? (VE * B + 3) / 4 : 1;  // 32-bit words per access
  static constexpr int NW = NL * WPL;
  static_assert(V % VE == 0, "V must be a multiple of the vector width");
  uint32_t w[NW];

  __device__ __forceinline__ float get(int i) const {
    if constexpr (!VEC) return bits_to_f<DT>(w[i]);
    else if constexpr (B == 4) return __uint_as_float(w[i]);
    else if constexpr (DT == DT_BF16)
      return (i & 1) ? __uint_as_float(w[i >> 1] & 0xffff0000u) : __uint_as_float(w[i >> 1] << 16);
    else return bits_to_f<DT>((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu));
  }

  // Column of element i for thread t in a team of T threads.
  static __device__ __forceinline__ int col(int i, int t, int T) {
    return ((i / VE) * T + t) * VE + (i % VE);
  }
  // Is access l in range?  (Vector path: N is a multiple of VE, so an access is
  // either wholly inside the row or wholly outside.)
  static __device__ __forceinline__ bool inb(int l, int t, int T, int N) {
    return (l * T + t) * VE < N;
  }

  // Hide the words' provenance from the optimiser: values derived from them after
  // this point are recomputed instead of being kept alive (in fp64) across the row
  // reduction, which would cost 4 VGPRs per element.
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int j = 0; j < NW; ++j) asm volatile("" : "+v"(w[j]));
  }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < NW; ++j) w[j] = 0u;
  }

  // Load this thread's elements through a buffer resource covering the row: offsets
  // at or past the resource's byte count read as zero (row tails, rows past M), so
  // there is no per-access branch and no 64-bit address arithmetic.  POL is the buffer
  // instructions' cache-policy operand (0 default, 2 non-temporal), here and below.
  template <int POL = 0>
  __device__ __forceinline__ void load(rsrc_t rs, int t, int T) {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int off = (l * T + t) * VE * B;
      if constexpr (VEC) {
        static_assert(WPL % 4 == 0, "vector access is a whole number of 16-byte loads");
#pragma unroll
        for (int q = 0; q < WPL / 4; ++q) {
          const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + q * 16, 0, POL);
          w[l * WPL + q * 4 + 0] = v.x;
          w[l * WPL + q * 4 + 1] = v.y;
          w[l * WPL + q * 4 + 2] = v.z;
          w[l * WPL + q * 4 + 3] = v.w;
        }
      } else if constexpr (B == 2) {
        w[l] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, POL);
      } else {
        w[l] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, POL);
      }
    }
  }

  // Several rows per wave (teams narrower than a wave): `rs` covers a block of rows,
  // `base` is this lane's row offset in bytes, and accesses at or past column N are
  // pushed out of the resource, so they read zero and are not stored.  (Vector path: N
  // is a multiple of VE, so an access is wholly inside the row or wholly outside.)
  static __device__ __forceinline__ uint32_t off_at(int l, uint32_t base, int t, int T, int N) {
    const int col = (l * T + t) * VE;
    return col < N ? base + static_cast<uint32_t>(col * B) : 0x80000000u;
  }
  template <int POL = 0>
  __device__ __forceinline__ void load_at(rsrc_t rs, uint32_t base, int t, int T, int N) {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const uint32_t off = off_at(l, base, t, T, N);
      if constexpr (VEC) {
        static_assert(WPL % 4 == 0, "vector access is a whole number of 16-byte loads");
#pragma unroll
        for (int q = 0; q < WPL / 4; ++q) {
          const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + q * 16, 0, POL);
          w[l * WPL + q * 4 + 0] = v.x;
          w[l * WPL + q * 4 + 1] = v.y;
          w[l * WPL + q * 4 + 2] = v.z;
          w[l * WPL + q * 4 + 3] = v.w;
        }
      } else if constexpr (B == 2) {
        w[l] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, POL);
      } else {
        w[l] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, POL);
      }
    }
  }
  template <int POL = 0>
  __device__ __forceinline__ void store_at(rsrc_t rs, uint32_t base, int t, int T, int N) const {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const uint32_t off = off_at(l, base, t, T, N);
      if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < WPL / 4; ++q) {
          const v4u v = {w[l * WPL + q * 4], w[l * WPL + q * 4 + 1], w[l * WPL + q * 4 + 2],
                         w[l * WPL + q * 4 + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, off + q * 16, 0, POL);
        }
      } else if constexpr (B == 2) {
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(w[l]), rs, off, 0, POL);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(w[l], rs, off, 0, POL);
      }
    }
  }

  // Store the words as they are; stores past the resource's byte count are dropped.
  template <int POL = 0>
  __device__ __forceinline__ void store_raw(rsrc_t rs, int t, int T) const {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int off = (l * T + t) * VE * B;
      if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < WPL / 4; ++q) {
          const v4u v = {w[l * WPL + q * 4], w[l * WPL + q * 4 + 1], w[l * WPL + q * 4 + 2],
                         w[l * WPL + q * 4 + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, off + q * 16, 0, POL);
        }
      } else if constexpr (B == 2) {
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(w[l]), rs, off, 0, POL);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(w[l], rs, off, 0, POL);
      }
    }
  }

  // Round V floats to DT and pack them into this fragment's words.
  __device__ __forceinline__ void pack(const float (&o)[V]) {
    if constexpr (!VEC) {
#pragma unroll
      for (int i = 0; i < V; ++i) w[i] = f_to_bits<DT>(o[i]);
    } else if constexpr (B == 4) {
#pragma unroll
      for (int i = 0; i < V; ++i) w[i] = __float_as_uint(o[i]);
    } else {
#pragma unroll
      for (int j = 0; j < V / 2; ++j) w[j] = pack2<DT>(o[2 * j], o[2 * j + 1]);
    }
  }
};

// Make per-column parameters look modified each row, so their fp64 conversions are
// redone per row instead of being hoisted out of the row loop (which would pin two
// VGPRs per element for the whole kernel).
template <int V> __device__ __forceinline__ void opaque(float (&a)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) asm volatile("" : "+v"(a[i]));
}

// fp64 value moved across lanes with a DPP pattern (two 32-bit moves).
template <int CTRL> __device__ __forceinline__ double dpp_mov(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  // every pattern used reads a lane that exists, so no lane keeps an old value
  const uint32_t lo = __builtin_amdgcn_mov_dpp(static_cast<int>(b), CTRL, 0xF, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_mov_dpp(static_cast<int>(b >> 32), CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ double read_lane(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(b), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(b >> 32), lane);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Sum over the 64 lanes of a wave; every lane ends with the same bits.
// Inside each row of 16 lanes: swap neighbours (quad_perm [1,0,3,2]), swap pairs
// ([2,3,0,1]), then rotate by 8 and by 4 lanes.  After the two quad swaps all lanes of
// quad k hold Q_k; rotating by 8 pairs quad k with quad k^2 (Q_k + Q_{k^2}, the same
// two operands in both quads, and a + b == b + a exactly); rotating by 4 then adds the
// other pair, again the same two operands everywhere.  The four row sums are read as
// scalars and added in one fixed order, so the result is uniform.
template <int NV> __device__ __forceinline__ void wave_sum(double (&v)[NV]) {
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] += dpp_mov<0xB1>(v[j]);
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] += dpp_mov<0x4E>(v[j]);
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] += dpp_mov<0x128>(v[j]);
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] += dpp_mov<0x124>(v[j]);
#pragma unroll
  for (int j = 0; j < NV; ++j)
    v[j] = (read_lane(v[j], 0) + read_lane(v[j], 16)) + (read_lane(v[j], 32) + read_lane(v[j], 48));
}

// Sum over each aligned group of TS lanes (TS = 8, 16 or 32: teams narrower than a
// wave, one row each); every lane of a group ends with the same bits.  Quad swaps give
// every lane its quad's sum; row_half_mirror (lane i <-> 7 - i inside 8 lanes) pairs
// the two quads of an 8-lane group, row_mirror (i <-> 15 - i) the two halves of a
// 16-lane row -- each step adds the same two operands in both lanes of a pair.  For 32
// lanes the four row sums are read as scalars and added in one fixed order.
template <int TS, int NV> __device__ __forceinline__ void group_sum(double (&v)[NV]) {
  static_assert(TS == 8 || TS == 16 || TS == 32, "sub-wave teams of 8, 16 or 32 lanes");
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] += dpp_mov<0xB1>(v[j]);
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] += dpp_mov<0x4E>(v[j]);
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] += dpp_mov<0x141>(v[j]);
  if constexpr (TS >= 16) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] += dpp_mov<0x140>(v[j]);
  }
  if constexpr (TS == 32) {
    const bool hi = (threadIdx.x & 63) >= 32;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const double lo2 = read_lane(v[j], 0) + read_lane(v[j], 16);
      const double hi2 = read_lane(v[j], 32) + read_lane(v[j], 48);
      v[j] = hi ? hi2 : lo2;
    }
  }
}

// Sum over the team's waves.  `red` is a workgroup-shared [2][16][4] buffer used in
// ping-pong: a slot written in one call is not rewritten before every thread has
// passed the next call's barrier, hence has finished reading it.  All threads of the
// workgroup must call this the same number of times (the team width is uniform).
template <int NV>
__device__ __forceinline__ void team_sum(double (&v)[NV], int wpr, int wave0,
                                         double (*red)[16][4], int& parity) {
  wave_sum<NV>(v);
  if (wpr == 1) return;
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) red[parity][wave][j] = v[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    double s = red[parity][wave0][j];
#pragma unroll 1
    for (int q = 1; q < wpr; ++q) s += red[parity][wave0 + q][j];
    v[j] = s;
  }
  parity ^= 1;
}

// 1 / sqrt(a) for a > 0: fp32 hardware estimate refined by two Newton steps in fp64
// (each step squares the relative error: ~2^-22 -> 2^-44 -> below fp64 rounding).
// Outside the range where the fp32 estimate is meaningful, the exact library path.
__device__ __forceinline__ double rsqrt_d(double a) {
  if (!(a > 1e-30 && a < 1e30)) return 1.0 / sqrt(a);
  double r = static_cast<double>(__builtin_amdgcn_rsqf(static_cast<float>(a)));
  const double h = 0.5 * a;
  r = r * fma(-h * r, r, 1.5);
  r = r * fma(-h * r, r, 1.5);
  return r;
}

}  // namespace rn
