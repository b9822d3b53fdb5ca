// Forward kernel instances for one operation (split per file to compile in parallel).
#include "rn_launch.h"

namespace rn {
int launch_fwd_fadd(int dx, int dw, const Launch& l, const FwdArgs& a, hipStream_t s) {
#define RN_PAIR(X, W) if (dx == X && dw == W) return fwd_v<OP_FADD, X, W>(l, a, s);
  RN_FOR_TYPE_PAIRS(RN_PAIR)
#undef RN_PAIR
  return LS_NO_INSTANCE;
}
}  // namespace rn
