// Multi-row dot path for the block-scaled FP formats (mxfp4, nvfp4, mxfp8),
// plain product and fused residual sum (kernels in qgemv_dot_impl.h; compiled
// apart so the formats build in parallel with the affine codes).
#include "qgemv_dot_impl.h"

namespace qgemv {

namespace {
template <bool ADD>
int launch_dot_fp_add(const QgemvArgs &a, hipStream_t stream) {
  switch (a.fmt) {
    case kMxfp4: return launch_dot_bits<4, ADD, kMxfp4>(a, stream);
    case kNvfp4: return launch_dot_bits<4, ADD, kNvfp4>(a, stream);
    case kMxfp8: return launch_dot_bits<8, ADD, kMxfp8>(a, stream);
    default: return QGEMV_EINVAL;
  }
}
}  // namespace

int launch_dot_fp(const QgemvArgs &a, hipStream_t stream) {
  return a.res ? launch_dot_fp_add<true>(a, stream) : launch_dot_fp_add<false>(a, stream);
}

}  // namespace qgemv
