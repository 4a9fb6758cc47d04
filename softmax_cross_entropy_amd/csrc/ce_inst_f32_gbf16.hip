// f32 instantiations of the split-row kernel that writes a bf16 gradient
// (wide_kernel_gbf16), used by the linear layer fused with the
// cross-entropy: row pairs of 512-thread workgroups (8 or 16 slots per
// thread) and of 1024-thread ones (16 slots), and quarter rows.
#include "ce_launch_impl.hpp"

namespace cehost {
bool gbf16_shape(int shape) {
  return shape == kPair8Shape || shape == kPair512Shape || shape == kPair1024Shape ||
         shape == kQuadShape;
}

hipError_t launch_wide_gbf16(int shape, const cedev::Params& p, const float* gscale,
                             int per_row, hipStream_t st) {
  switch (shape) {
    case kQuadShape: return launch_wide_gbf16_h<cedev::F32, 512, 16, 4>(p, gscale, per_row, st);
    case kPair1024Shape:
      return launch_wide_gbf16_h<cedev::F32, 1024, 16, 2>(p, gscale, per_row, st);
    case kPair512Shape:
      return launch_wide_gbf16_h<cedev::F32, 512, 16, 2>(p, gscale, per_row, st);
    case kPair8Shape: return launch_wide_gbf16_h<cedev::F32, 512, 8, 2>(p, gscale, per_row, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace cehost
