// Instantiations of the GEMV kernel for 5 and 6 activation columns.
#include "gemv_kernel.h"

namespace rfp2 {
namespace gemv_detail {

GemvFn pick_m5(int jt) { return pick<5, false>(jt); }
GemvFn pick_m6(int jt) { return pick<6, false>(jt); }
GemvFn pick_m5_mf(int jt) { return pick<5, false, true>(jt); }
GemvFn pick_m6_mf(int jt) { return pick<6, false, true>(jt); }

}  // namespace gemv_detail
}  // namespace rfp2
