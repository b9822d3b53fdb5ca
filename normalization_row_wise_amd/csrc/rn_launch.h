// rn_launch.h — internal launch interface between the C ABI and the kernel instances.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>
#include <set>
#include <utility>

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
  bool split = false;  // rows spread over workgroups (rn_split.h; v, ts unused)
  bool group = false;  // split: a row's workgroups renumbered onto one XCD
  hipEvent_t ev_start = nullptr, ev_stop = nullptr;  // optional dispatch timing events
};

// Outcome of a dispatch: launched, no compiled instance for the request (an internal
// error: the planner only asks for compiled shapes), or the HIP runtime refused it.
enum LaunchStatus : int { LS_OK = 0, LS_NO_INSTANCE = 1, LS_HIP = 2 };

// Launch one kernel; the status is this launch's own (the launch call's return value),
// not whatever error an earlier, unrelated HIP call may have left behind.  With timing
// events attached (rn_instrument.h) the dispatch itself records them.
template <typename A>
inline int launch_kernel(void (*k)(A), const Launch& l, hipStream_t s, const A& a) {
  void* args[] = {const_cast<A*>(&a)};
  const hipError_t e =
      l.ev_start != nullptr && l.ev_stop != nullptr
          ? hipExtLaunchKernel(reinterpret_cast<const void*>(k), l.grid, l.block, args, l.shmem, s,
                               l.ev_start, l.ev_stop, 0)
          : hipLaunchKernel(reinterpret_cast<const void*>(k), l.grid, l.block, args, l.shmem, s);
  return e == hipSuccess ? LS_OK : LS_HIP;
}

// Kernels that take more than 64 KiB of dynamic LDS must be allowed to, once per kernel
// and device: the attribute is set on the first such launch on a device and remembered.
template <typename A>
inline bool allow_big_lds(void (*k)(A)) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const auto key = std::make_pair(reinterpret_cast<const void*>(k), dev);
  std::lock_guard<std::mutex> g(mu);
  if (done.count(key)) return true;
  // the whole LDS a workgroup may take (160 KiB on gfx950) less the static row slots
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 156 * 1024) != hipSuccess)
    return false;
  done.insert(key);
  return true;
}

// Each returns a LaunchStatus.
int launch_fwd_rms(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
int launch_fwd_ln(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
int launch_fwd_fadd(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
// Backward variants: xg = exact fp32 product g = dy * w (16-bit weight, no offset);
// acc = 1 keeps the dw / db accumulators in LDS, 2 in LDS blocks of stride 384 (V = 48,
// both LayerNorm gradients), 3 dw in LDS and db in registers (V = 48, both LayerNorm
// gradients, wider teams), 0 both in registers (V = 48 only).
struct BwdVariant {
  bool cdw, cdb, xg;
  int acc;
};
int launch_bwd_rms(int dx, int dw, const BwdVariant& b, const Launch& l, const BwdArgs& a,
                   hipStream_t s);
int launch_bwd_ln(int dx, int dw, const BwdVariant& b, const Launch& l, const BwdArgs& a,
                  hipStream_t s);
int launch_bwd_fadd(int dx, int dw, const BwdVariant& b, const Launch& l, const BwdArgs& a,
                    hipStream_t s);

// Type pairs that are compiled: (x type, weight type).
#define RN_FOR_TYPE_PAIRS(X)                                                    \
  X(DT_F32, DT_F32) X(DT_F16, DT_F16) X(DT_BF16, DT_BF16) X(DT_F16, DT_F32)     \
  X(DT_BF16, DT_F32)

template <int OP, int DX, int DW>
inline int fwd_v(const Launch& l, const FwdArgs& a, hipStream_t s) {
  if (l.split) {
    if (!l.vec) return LS_NO_INSTANCE;
    return launch_kernel(
        l.group ? split_fwd_kernel<OP, DX, DW, true> : split_fwd_kernel<OP, DX, DW, false>, l, s, a);
  }
  if (l.ts != 0) {  // sub-wave teams: V = 8, 16-byte accesses
    if (l.v != 8 || !l.vec) return LS_NO_INSTANCE;
    switch (l.ts) {
      case 8: return launch_kernel(fwd_kernel<OP, DX, DW, 8, true, 8>, l, s, a);
      case 16: return launch_kernel(fwd_kernel<OP, DX, DW, 8, true, 16>, l, s, a);
      case 32: return launch_kernel(fwd_kernel<OP, DX, DW, 8, true, 32>, l, s, a);
      default: return LS_NO_INSTANCE;
    }
  }
#define RN_CASE(V)                                                                       \
  case V:                                                                                \
    return launch_kernel(                                                                \
        l.vec ? fwd_kernel<OP, DX, DW, V, true> : fwd_kernel<OP, DX, DW, V, false>, l, s, a);
  switch (l.v) {
    RN_CASE(8) RN_CASE(16) RN_CASE(32) RN_CASE(48)
    default: return LS_NO_INSTANCE;
  }
#undef RN_CASE
}

inline int bwd_go(void (*k)(BwdArgs), const Launch& l, const BwdArgs& a, hipStream_t s) {
  if (l.shmem > 64 * 1024 && !allow_big_lds(k)) return LS_HIP;
  return launch_kernel(k, l, s, a);
}

template <int OP, int DX, int DW, bool CDW, bool CDB, bool XG, int ACC, int V>
inline int bwd_one(const Launch& l, const BwdArgs& a, hipStream_t s) {
  if constexpr (ACC == 0 && (CDW || CDB) && V < 48 && !(OP == OP_RMS && V >= 16)) {
    // up to V = 32 the LDS accumulator blocks always fit; register accumulators below
    // V = 48 only serve RMSNorm workgroups of a single team (rn_abi.hip, plan)
    return LS_NO_INSTANCE;
  } else if constexpr (ACC >= 2 && !(V == 48 && CDW && CDB)) {
    // the 384-stride blocks and the split homes only serve both LayerNorm gradients at
    // V = 48
    return LS_NO_INSTANCE;
  } else if constexpr (ACC >= 2) {
    if (l.ts != 0 || !l.vec) return LS_NO_INSTANCE;
    return bwd_go(bwd_kernel<OP, DX, DW, V, true, CDW, CDB, XG, ACC>, l, a, s);
  } else {
    if constexpr (V == 8 && (ACC == 1 || (!CDW && !CDB))) {
      if (l.ts != 0) {  // sub-wave teams: V = 8, 16-byte accesses
        if (!l.vec) return LS_NO_INSTANCE;
        switch (l.ts) {
          case 8: return bwd_go(bwd_kernel<OP, DX, DW, 8, true, CDW, CDB, XG, ACC, 8>, l, a, s);
          case 16: return bwd_go(bwd_kernel<OP, DX, DW, 8, true, CDW, CDB, XG, ACC, 16>, l, a, s);
          case 32: return bwd_go(bwd_kernel<OP, DX, DW, 8, true, CDW, CDB, XG, ACC, 32>, l, a, s);
          default: return LS_NO_INSTANCE;
        }
      }
    }
    if (l.ts != 0) return LS_NO_INSTANCE;
    return bwd_go(l.vec ? bwd_kernel<OP, DX, DW, V, true, CDW, CDB, XG, ACC>
                        : bwd_kernel<OP, DX, DW, V, false, CDW, CDB, XG, ACC>,
                  l, a, s);
  }
}

template <int OP, int DX, int DW, bool CDW, bool CDB, bool XG, int ACC>
inline int bwd_v(const Launch& l, const BwdArgs& a, hipStream_t s) {
  switch (l.v) {
    case 8: return bwd_one<OP, DX, DW, CDW, CDB, XG, ACC, 8>(l, a, s);
    case 16: return bwd_one<OP, DX, DW, CDW, CDB, XG, ACC, 16>(l, a, s);
    case 32: return bwd_one<OP, DX, DW, CDW, CDB, XG, ACC, 32>(l, a, s);
    case 48: return bwd_one<OP, DX, DW, CDW, CDB, XG, ACC, 48>(l, a, s);
    default: return LS_NO_INSTANCE;
  }
}

template <int OP, int DX, int DW, bool CDW, bool CDB, bool XG>
inline int bwd_acc(int acc, const Launch& l, const BwdArgs& a, hipStream_t s) {
  switch (acc) {
    case 0: return bwd_v<OP, DX, DW, CDW, CDB, XG, 0>(l, a, s);
    case 1: return bwd_v<OP, DX, DW, CDW, CDB, XG, 1>(l, a, s);
    case 2: return bwd_v<OP, DX, DW, CDW, CDB, XG, 2>(l, a, s);
    case 3: return bwd_v<OP, DX, DW, CDW, CDB, XG, 3>(l, a, s);
    default: return LS_NO_INSTANCE;
  }
}

// Dispatch over the gradient flags, the exact-product path and the accumulator home.
template <int OP, int DX, int DW, bool CDW, bool CDB>
inline int bwd_flags(const BwdVariant& b, const Launch& l, const BwdArgs& a, hipStream_t s) {
  constexpr bool can_xg = Ty<DW>::B == 2;
  if (l.split) {
    if (!l.vec) return LS_NO_INSTANCE;
    if constexpr (can_xg) {
      if (b.xg) {
        return launch_kernel(l.group ? split_bwd_kernel<OP, DX, DW, CDW, CDB, true, true>
                                     : split_bwd_kernel<OP, DX, DW, CDW, CDB, true, false>,
                             l, s, a);
      }
    }
    return launch_kernel(l.group ? split_bwd_kernel<OP, DX, DW, CDW, CDB, false, true>
                                 : split_bwd_kernel<OP, DX, DW, CDW, CDB, false, false>,
                         l, s, a);
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
