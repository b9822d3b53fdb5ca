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

  __device__ __forceinline__ void load(const void* rowp, int t, int T, int N, bool valid) {
    const typename Ty<DT>::S* row = static_cast<const typename Ty<DT>::S*>(rowp);
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int c = (l * T + t) * VE;
      if constexpr (VEC) {
        static_assert(WPL % 4 == 0, "vector access is a whole number of 16-byte loads");
#pragma unroll
        for (int q = 0; q < WPL / 4; ++q) {
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (valid && c < N) v = *reinterpret_cast<const uint4*>(row + c + q * (16 / B));
          w[l * WPL + q * 4 + 0] = v.x;
          w[l * WPL + q * 4 + 1] = v.y;
          w[l * WPL + q * 4 + 2] = v.z;
          w[l * WPL + q * 4 + 3] = v.w;
        }
      } else {
        w[l] = (valid && c < N) ? static_cast<uint32_t>(row[c]) : 0u;
      }
    }
  }

  // Store words as they are (used for the rounded residual of the fused add).
  __device__ __forceinline__ void store_raw(void* rowp, int t, int T, int N, bool valid) const {
    typename Ty<DT>::S* row = static_cast<typename Ty<DT>::S*>(rowp);
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int c = (l * T + t) * VE;
      if (!(valid && c < N)) continue;
      if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < WPL / 4; ++q)
          *reinterpret_cast<uint4*>(row + c + q * (16 / B)) =
              make_uint4(w[l * WPL + q * 4], w[l * WPL + q * 4 + 1], w[l * WPL + q * 4 + 2],
                         w[l * WPL + q * 4 + 3]);
      } else {
        row[c] = static_cast<typename Ty<DT>::S>(w[l]);
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

// Butterfly sum over the 64 lanes of a wave.  Every lane ends with the same value
// (a + b == b + a exactly), so no broadcast is needed.
template <int NV> __device__ __forceinline__ void wave_sum(double (&v)[NV]) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] += __shfl_xor(v[j], m, 64);
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
    for (int q = 1; q < wpr; ++q) s += red[parity][wave0 + q][j];
    v[j] = s;
  }
  parity ^= 1;
}

}  // namespace rn
