// Multi-row dot path for 8-bit codes, plain product and fused residual sum
// (kernels in qgemv_dot_impl.h; compiled apart so the widths build in
// parallel).
#include "qgemv_dot_impl.h"

namespace qgemv {

int launch_dot8(const QgemvArgs &a, hipStream_t stream) {
  return a.res ? launch_dot_bits<8, true>(a, stream) : launch_dot_bits<8, false>(a, stream);
}

}  // namespace qgemv
