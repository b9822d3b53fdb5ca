// rn_launch.h — internal launch interface between the C ABI and the kernel instances.
#pragma once
#include <hip/hip_runtime.h>
#include "rn_kernels.h"

namespace rn {

// Elements per thread per row that are compiled (for every type and both access modes).
constexpr int kVs[] = {8, 16, 24, 32};

struct Launch {
  int v;          // elements per thread per row (one of kVs)
  bool vec;       // 16-byte accesses (else element accesses)
  dim3 grid, block;
  size_t shmem;   // dynamic LDS bytes
};

// Each returns false when (dx, dw, v) has no compiled instance.
bool launch_fwd_rms(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
bool launch_fwd_ln(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
bool launch_fwd_fadd(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s);
bool launch_bwd_rms(int dx, int dw, bool cdw, const Launch& l, const BwdArgs& a, hipStream_t s);
bool launch_bwd_ln(int dx, int dw, bool cdw, bool cdb, const Launch& l, const BwdArgs& a,
                   hipStream_t s);
bool launch_bwd_fadd(int dx, int dw, bool cdw, const Launch& l, const BwdArgs& a, hipStream_t s);

// Type pairs that are compiled: (x type, weight type).
#define RN_FOR_TYPE_PAIRS(X)                                                    \
  X(DT_F32, DT_F32) X(DT_F16, DT_F16) X(DT_BF16, DT_BF16) X(DT_F16, DT_F32)     \
  X(DT_BF16, DT_F32)

template <int OP, int DX, int DW>
inline bool fwd_v(const Launch& l, const FwdArgs& a, hipStream_t s) {
#define RN_CASE(V)                                                                   \
  case V:                                                                            \
    if (l.vec) fwd_kernel<OP, DX, DW, V, true><<<l.grid, l.block, l.shmem, s>>>(a);  \
    else fwd_kernel<OP, DX, DW, V, false><<<l.grid, l.block, l.shmem, s>>>(a);       \
    return true;
  switch (l.v) { RN_CASE(8) RN_CASE(16) RN_CASE(24) RN_CASE(32) default: return false; }
#undef RN_CASE
}

template <int OP, int DX, int DW, bool CDW, bool CDB>
inline bool bwd_v(const Launch& l, const BwdArgs& a, hipStream_t s) {
#define RN_CASE(V)                                                                            \
  case V:                                                                                     \
    if (l.vec) bwd_kernel<OP, DX, DW, V, true, CDW, CDB><<<l.grid, l.block, l.shmem, s>>>(a); \
    else bwd_kernel<OP, DX, DW, V, false, CDW, CDB><<<l.grid, l.block, l.shmem, s>>>(a);      \
    return true;
  switch (l.v) { RN_CASE(8) RN_CASE(16) RN_CASE(24) RN_CASE(32) default: return false; }
#undef RN_CASE
}

}  // namespace rn
