// Instantiations of the GEMV kernel for 3 and 4 activation columns.
#include "gemv_kernel.h"

namespace rfp2 {
namespace gemv_detail {

GemvFn pick_m3(int jt) { return pick<3, false>(jt); }
GemvFn pick_m4(int jt) { return pick<4, false>(jt); }
GemvFn pick_m3_mf(int jt) { return pick<3, false, true>(jt); }
GemvFn pick_m4_mf(int jt) { return pick<4, false, true>(jt); }

}  // namespace gemv_detail
}  // namespace rfp2
