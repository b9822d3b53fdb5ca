// Backward (stage 1) kernel instances for RMSNorm: dw computed or pruned.
#include "rn_launch.h"

namespace rn {
int launch_bwd_rms(int dx, int dw, const BwdVariant& b, const Launch& l, const BwdArgs& a,
                   hipStream_t s) {
#define RN_PAIR(X, W)                                                           \
  if (dx == X && dw == W)                                                       \
    return b.cdw ? bwd_flags<OP_RMS, X, W, true, false>(b, l, a, s)             \
                 : bwd_flags<OP_RMS, X, W, false, false>(b, l, a, s);
  RN_FOR_TYPE_PAIRS(RN_PAIR)
#undef RN_PAIR
  return LS_NO_INSTANCE;
}
}  // namespace rn
