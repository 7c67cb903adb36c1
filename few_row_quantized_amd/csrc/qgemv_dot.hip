// Multi-row dot path: the plain product (kernels in qgemv_dot_impl.h).  The
// fused residual sum's instantiations are compiled in qgemv_dot_add.hip.
#include "qgemv_dot_impl.h"

namespace qgemv {

int launch_dot(const QgemvArgs &a, hipStream_t stream) {
  if (a.res) return launch_dot_add(a, stream);
  return launch_dot_impl<false>(a, stream);
}

}  // namespace qgemv
