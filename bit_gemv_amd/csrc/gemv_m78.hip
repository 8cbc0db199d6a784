// Instantiations of the GEMV kernel for 7 and 8 activation columns.
#include "gemv_kernel.h"

namespace rfp2 {
namespace gemv_detail {

GemvFn pick_m7(int jt) { return pick<7, false>(jt); }
GemvFn pick_m8(int jt) { return pick<8, false>(jt); }
GemvFn pick_m7_mf(int jt) { return pick<7, false, true>(jt); }
GemvFn pick_m8_mf(int jt) { return pick<8, false, true>(jt); }

}  // namespace gemv_detail
}  // namespace rfp2
