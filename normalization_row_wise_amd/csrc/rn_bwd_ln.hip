// Backward (stage 1) kernel instances for LayerNorm: dw and db each computed or pruned.
#include "rn_launch.h"

namespace rn {
bool launch_bwd_ln(int dx, int dw, bool cdw, bool cdb, const Launch& l, const BwdArgs& a,
                   hipStream_t s) {
#define RN_PAIR(X, W)                                                                  \
  if (dx == X && dw == W) {                                                            \
    if (cdw && cdb) return bwd_v<OP_LN, X, W, true, true>(l, a, s);                    \
    if (cdw) return bwd_v<OP_LN, X, W, true, false>(l, a, s);                          \
    if (cdb) return bwd_v<OP_LN, X, W, false, true>(l, a, s);                          \
    return bwd_v<OP_LN, X, W, false, false>(l, a, s);                                  \
  }
  RN_FOR_TYPE_PAIRS(RN_PAIR)
#undef RN_PAIR
  return false;
}
}  // namespace rn
