// f32 instantiations of the wide row kernel: 512-thread workgroups holding
// half a row (8 or 16 slots per thread) or a quarter (16 slots), 1024-thread
// workgroups holding half a row (16 slots) or a whole one (4 slots).
#include "ce_launch_impl.hpp"

namespace cehost {
hipError_t launch_wide_f32(const Shape& s, const cedev::Params& p, hipStream_t st) {
  if (s.parts == 4) return launch_wide_h<cedev::F32, 512, 16, 4>(p, st);
  if (s.parts == 2) {
    if (s.block == 1024) return launch_wide_h<cedev::F32, 1024, 16, 2>(p, st);
    return s.nreg == 8 ? launch_wide_h<cedev::F32, 512, 8, 2>(p, st)
                       : launch_wide_h<cedev::F32, 512, 16, 2>(p, st);
  }
  return launch_wide_h<cedev::F32, 1024, 4, 1>(p, st);
}
}  // namespace cehost
