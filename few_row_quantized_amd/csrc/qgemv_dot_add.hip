// Multi-row dot path with the fused residual sum, y = x W^T + r (kernels in
// qgemv_dot_impl.h; compiled apart from the plain product so the two halves
// of the instantiations build in parallel).
#include "qgemv_dot_impl.h"

namespace qgemv {

int launch_dot_add(const QgemvArgs &a, hipStream_t stream) { return launch_dot_impl<true>(a, stream); }

}  // namespace qgemv
