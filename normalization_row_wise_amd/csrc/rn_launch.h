// rn_launch.h — internal launch interface between the C ABI and the kernel instances.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include "rn_split.h"

namespace rn {

// Elements per thread per row that are compiled (for every type and both access modes).
constexpr int kVs[] = {8, 16, 32, 48};

struct Launch {
  int v;          // elements per thread per row (one of kVs)
  bool vec;       // 16-byte accesses (else element accesses)
  int ts;         // 0: teams of whole waves; 8, 16, 32: sub-wave teams (V = 8, vec only)
  dim3 grid, block;
  size_t shmem;   // dynamic LDS bytes
  hipEvent_t ev_start = nullptr, ev_stop = nullptr;  // optional kernel timing
  bool split = false;  // rows spread over workgroups (rn_split.h; v, ts unused)
  bool group = false;  // split: a row's workgroups renumbered onto one XCD
};

// Launch through hipExtLaunchKernel when timing events are attached.
template <typename K, typename A>
inline void launch_kernel(K k, const Launch& l, hipStream_t s, const A& a) {
  if (l.ev_start != nullptr && l.ev_stop != nullptr)
    hipExtLaunchKernelGGL(k, l.grid, l.block, l.shmem, s, l.ev_start, l.ev_stop, 0, a);
  else
    k<<<l.grid, l.block, l.shmem, s>>>(a);
}

// Each returns false when (dx, dw, v) has no compiled instance.
bool launch_fwd_rms(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
bool launch_fwd_ln(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
bool launch_fwd_fadd(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
// Backward variants: xg = exact fp32 product g = dy * w (16-bit weight, no offset);
// acc = 1 keeps the dw / db accumulators in LDS, 2 in LDS blocks of stride 384 (V = 48,
// both LayerNorm gradients), 3 dw in LDS and db in registers (V = 48, both LayerNorm
// gradients, wider teams), 0 both in registers (V = 48 only).
struct BwdVariant {
  bool cdw, cdb, xg;
  int acc;
};
bool launch_bwd_rms(int dx, int dw, const BwdVariant& b, const Launch& l, const BwdArgs& a,
                    hipStream_t s);
bool launch_bwd_ln(int dx, int dw, const BwdVariant& b, const Launch& l, const BwdArgs& a,
                   hipStream_t s);
bool launch_bwd_fadd(int dx, int dw, const BwdVariant& b, const Launch& l, const BwdArgs& a,
                     hipStream_t s);

// Type pairs that are compiled: (x type, weight type).
#define RN_FOR_TYPE_PAIRS(X)                                                    \
  X(DT_F32, DT_F32) X(DT_F16, DT_F16) X(DT_BF16, DT_BF16) X(DT_F16, DT_F32)     \
  X(DT_BF16, DT_F32)

template <int OP, int DX, int DW>
inline bool fwd_v(const Launch& l, const FwdArgs& a, hipStream_t s) {
  if (l.split) {
    if (!l.vec) return false;
    launch_kernel(l.group ? split_fwd_kernel<OP, DX, DW, true> : split_fwd_kernel<OP, DX, DW, false>,
                  l, s, a);
    return true;
  }
  if (l.ts != 0) {  // sub-wave teams: V = 8, 16-byte accesses
    if (l.v != 8 || !l.vec) return false;
    switch (l.ts) {
      case 8: launch_kernel(fwd_kernel<OP, DX, DW, 8, true, 8>, l, s, a); return true;
      case 16: launch_kernel(fwd_kernel<OP, DX, DW, 8, true, 16>, l, s, a); return true;
      case 32: launch_kernel(fwd_kernel<OP, DX, DW, 8, true, 32>, l, s, a); return true;
      default: return false;
    }
  }
#define RN_CASE(V)                                                                       \
  case V:                                                                                \
    launch_kernel(l.vec ? fwd_kernel<OP, DX, DW, V, true> : fwd_kernel<OP, DX, DW, V, false>, \
                  l, s, a);                                                              \
    return true;
  switch (l.v) {
    RN_CASE(8) RN_CASE(16) RN_CASE(32) RN_CASE(48)
    default: return false;
  }
#undef RN_CASE
}

template <typename K> inline bool bwd_go(K k, const Launch& l, const BwdArgs& a, hipStream_t s) {
  if (l.shmem > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(l.shmem)) != hipSuccess)
    return false;
  launch_kernel(k, l, s, a);
  return true;
}

template <int OP, int DX, int DW, bool CDW, bool CDB, bool XG, int ACC, int V>
inline bool bwd_one(const Launch& l, const BwdArgs& a, hipStream_t s) {
  if constexpr (ACC == 0 && (CDW || CDB) && V < 48) {
    // up to V = 32 the LDS accumulator blocks always fit
    return false;
  } else if constexpr (ACC >= 2 && !(V == 48 && CDW && CDB)) {
    // the 384-stride blocks and the split homes only serve both LayerNorm gradients at
    // V = 48
    return false;
  } else if constexpr (ACC >= 2) {
    if (l.ts != 0 || !l.vec) return false;
    return bwd_go(bwd_kernel<OP, DX, DW, V, true, CDW, CDB, XG, ACC>, l, a, s);
  } else {
    if constexpr (V == 8 && (ACC == 1 || (!CDW && !CDB))) {
      if (l.ts != 0) {  // sub-wave teams: V = 8, 16-byte accesses
        if (!l.vec) return false;
        switch (l.ts) {
          case 8: return bwd_go(bwd_kernel<OP, DX, DW, 8, true, CDW, CDB, XG, ACC, 8>, l, a, s);
          case 16: return bwd_go(bwd_kernel<OP, DX, DW, 8, true, CDW, CDB, XG, ACC, 16>, l, a, s);
          case 32: return bwd_go(bwd_kernel<OP, DX, DW, 8, true, CDW, CDB, XG, ACC, 32>, l, a, s);
          default: return false;
        }
      }
    }
    if (l.ts != 0) return false;
    return bwd_go(l.vec ? bwd_kernel<OP, DX, DW, V, true, CDW, CDB, XG, ACC>
                        : bwd_kernel<OP, DX, DW, V, false, CDW, CDB, XG, ACC>,
                  l, a, s);
  }
}

template <int OP, int DX, int DW, bool CDW, bool CDB, bool XG, int ACC>
inline bool bwd_v(const Launch& l, const BwdArgs& a, hipStream_t s) {
  switch (l.v) {
    case 8: return bwd_one<OP, DX, DW, CDW, CDB, XG, ACC, 8>(l, a, s);
    case 16: return bwd_one<OP, DX, DW, CDW, CDB, XG, ACC, 16>(l, a, s);
    case 32: return bwd_one<OP, DX, DW, CDW, CDB, XG, ACC, 32>(l, a, s);
    case 48: return bwd_one<OP, DX, DW, CDW, CDB, XG, ACC, 48>(l, a, s);
    default: return false;
  }
}

template <int OP, int DX, int DW, bool CDW, bool CDB, bool XG>
inline bool bwd_acc(int acc, const Launch& l, const BwdArgs& a, hipStream_t s) {
  switch (acc) {
    case 0: return bwd_v<OP, DX, DW, CDW, CDB, XG, 0>(l, a, s);
    case 1: return bwd_v<OP, DX, DW, CDW, CDB, XG, 1>(l, a, s);
    case 2: return bwd_v<OP, DX, DW, CDW, CDB, XG, 2>(l, a, s);
    case 3: return bwd_v<OP, DX, DW, CDW, CDB, XG, 3>(l, a, s);
    default: return false;
  }
}

// Dispatch over the gradient flags, the exact-product path and the accumulator home.
template <int OP, int DX, int DW, bool CDW, bool CDB>
inline bool bwd_flags(const BwdVariant& b, const Launch& l, const BwdArgs& a, hipStream_t s) {
  constexpr bool can_xg = Ty<DW>::B == 2;
  if (l.split) {
    if (!l.vec) return false;
    if constexpr (can_xg) {
      if (b.xg) {
        launch_kernel(l.group ? split_bwd_kernel<OP, DX, DW, CDW, CDB, true, true>
                              : split_bwd_kernel<OP, DX, DW, CDW, CDB, true, false>,
                      l, s, a);
        return true;
      }
    }
    launch_kernel(l.group ? split_bwd_kernel<OP, DX, DW, CDW, CDB, false, true>
                          : split_bwd_kernel<OP, DX, DW, CDW, CDB, false, false>,
                  l, s, a);
    return true;
  }
  if constexpr (!CDW && !CDB) {
    if constexpr (can_xg) {
      if (b.xg) return bwd_v<OP, DX, DW, false, false, true, 0>(l, a, s);
    }
    return bwd_v<OP, DX, DW, false, false, false, 0>(l, a, s);
  } else {
    if constexpr (can_xg) {
      if (b.xg) return bwd_acc<OP, DX, DW, CDW, CDB, true>(b.acc, l, a, s);
    }
    return bwd_acc<OP, DX, DW, CDW, CDB, false>(b.acc, l, a, s);
  }
}

}  // namespace rn
