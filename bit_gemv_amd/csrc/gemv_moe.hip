// Routed-expert GEMV for 2..8 tokens (instantiations of gemv_kernel's MoE
// form with grouped slots; the design notes are in gemv.hip).
#include "gemv_kernel.h"

namespace rfp2 {
namespace gemv_detail {

GemvFn pick_moe_tokens(int T) {
  switch (T) {
    case 2: return gemv_kernel<2, 1, true, false>;
    case 3: return gemv_kernel<3, 1, true, false>;
    case 4: return gemv_kernel<4, 1, true, false>;
    case 5: return gemv_kernel<5, 1, true, false>;
    case 6: return gemv_kernel<6, 1, true, false>;
    case 7: return gemv_kernel<7, 1, true, false>;
    default: return gemv_kernel<8, 1, true, false>;
  }
}

}  // namespace gemv_detail
}  // namespace rfp2
