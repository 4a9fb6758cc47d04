// bf16 instantiations of the 1024-thread wide row kernel (one workgroup per
// row, or a row pair).
#include "ce_launch_impl.hpp"

namespace cehost {
hipError_t launch_wide_bf16(int nreg, int halves, const cedev::Params& p, hipStream_t st) {
  if (halves == 2) return launch_wide_h<cedev::BF16, 16, 2>(p, st);
  switch (nreg) {
    case 4: return launch_wide_h<cedev::BF16, 4, 1>(p, st);
    case 8: return launch_wide_h<cedev::BF16, 8, 1>(p, st);
    default: return launch_wide_h<cedev::BF16, 16, 1>(p, st);
  }
}
}  // namespace cehost
