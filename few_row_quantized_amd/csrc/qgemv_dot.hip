// Multi-row dot path: the plain product of 2- and 4-bit codes (kernels in
// qgemv_dot_impl.h).  The fused residual sum's instantiations are compiled in
// qgemv_dot_add.hip, those of 8-bit codes in qgemv_dot8.hip and those of the
// block-scaled FP formats in qgemv_dot_fp.hip.
#include "qgemv_dot_impl.h"

namespace qgemv {

int launch_dot(const QgemvArgs &a, hipStream_t stream) {
  if (a.fmt != 0) return launch_dot_fp(a, stream);
  if (a.bits == 8) return launch_dot8(a, stream);
  if (a.res) return launch_dot_add(a, stream);
  return launch_dot_impl<false>(a, stream);
}

}  // namespace qgemv
