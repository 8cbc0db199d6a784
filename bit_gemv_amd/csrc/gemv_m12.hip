// Instantiations of the GEMV kernel for 1 and 2 activation columns.
#include "gemv_kernel.h"

namespace rfp2 {
namespace gemv_detail {

GemvFn pick_m1(int jt) { return pick<1, false>(jt); }
GemvFn pick_m2(int jt) { return pick<2, false>(jt); }
GemvFn pick_m2_mf(int jt) { return pick<2, false, true>(jt); }

}  // namespace gemv_detail
}  // namespace rfp2
