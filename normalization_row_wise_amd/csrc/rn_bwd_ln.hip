// Backward (stage 1) kernel instances for LayerNorm: dw and db each computed or pruned.
#include "rn_launch.h"

namespace rn {
int launch_bwd_ln(int dx, int dw, const BwdVariant& b, const Launch& l, const BwdArgs& a,
                   hipStream_t s) {
#define RN_PAIR(X, W)                                                                  \
  if (dx == X && dw == W) {                                                            \
    if (b.cdw && b.cdb) return bwd_flags<OP_LN, X, W, true, true>(b, l, a, s);         \
    if (b.cdw) return bwd_flags<OP_LN, X, W, true, false>(b, l, a, s);                 \
    if (b.cdb) return bwd_flags<OP_LN, X, W, false, true>(b, l, a, s);                 \
    return bwd_flags<OP_LN, X, W, false, false>(b, l, a, s);                           \
  }
  RN_FOR_TYPE_PAIRS(RN_PAIR)
#undef RN_PAIR
  return LS_NO_INSTANCE;
}
}  // namespace rn
