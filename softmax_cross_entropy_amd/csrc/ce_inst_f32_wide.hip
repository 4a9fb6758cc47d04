// f32 instantiations of the wide row kernel (1024-thread workgroups holding
// a whole row or half of one, 512-thread workgroups holding a quarter).
#include "ce_launch_impl.hpp"

namespace cehost {
hipError_t launch_wide_f32(int nreg, int halves, const cedev::Params& p, hipStream_t st) {
  if (halves == 4) return launch_wide_h<cedev::F32, 512, 16, 4>(p, st);
  if (halves == 2) return launch_wide_h<cedev::F32, 1024, 16, 2>(p, st);
  switch (nreg) {
    case 4: return launch_wide_h<cedev::F32, 1024, 4, 1>(p, st);
    case 8: return launch_wide_h<cedev::F32, 1024, 8, 1>(p, st);
    default: return launch_wide_h<cedev::F32, 1024, 16, 1>(p, st);
  }
}
}  // namespace cehost
