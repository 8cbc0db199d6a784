// Routed-expert GEMV for 2..8 tokens (instantiations of gemv_kernel's MoE
// form with grouped slots, the matrix-core form; the design
// notes are in gemv.hip).
#include "gemv_kernel.h"

namespace rfp2 {
namespace gemv_detail {

GemvFn pick_moe_tokens(int T, bool mf) {
  switch (T) {
    case 2: return mf ? gemv_kernel<2, 1, true, 0, true> : gemv_kernel<2, 1, true, 0>;
    case 3: return mf ? gemv_kernel<3, 1, true, 0, true> : gemv_kernel<3, 1, true, 0>;
    case 4: return mf ? gemv_kernel<4, 1, true, 0, true> : gemv_kernel<4, 1, true, 0>;
    case 5: return mf ? gemv_kernel<5, 1, true, 0, true> : gemv_kernel<5, 1, true, 0>;
    case 6: return mf ? gemv_kernel<6, 1, true, 0, true> : gemv_kernel<6, 1, true, 0>;
    case 7: return mf ? gemv_kernel<7, 1, true, 0, true> : gemv_kernel<7, 1, true, 0>;
    default: return mf ? gemv_kernel<8, 1, true, 0, true> : gemv_kernel<8, 1, true, 0>;
  }
}

}  // namespace gemv_detail
}  // namespace rfp2
