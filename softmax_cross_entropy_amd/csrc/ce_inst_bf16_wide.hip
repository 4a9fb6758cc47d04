// bf16 instantiations of the 1024-thread wide row kernel (one workgroup per
// row, or a row pair).
#include "ce_launch_impl.hpp"

namespace cehost {
hipError_t launch_wide_bf16(int halves, const cedev::Params& p, hipStream_t st) {
  return halves == 2 ? launch_wide_h<cedev::BF16, 2>(p, st) : launch_wide_h<cedev::BF16, 1>(p, st);
}
}  // namespace cehost
