// bf16 instantiations of the wide row kernel: 1024-thread workgroups holding
// a whole row (4 or 8 slots per thread) or half of one, 512-thread
// workgroups holding half or a quarter of one (16 slots).
#include "ce_launch_impl.hpp"

namespace cehost {
hipError_t launch_wide_bf16(const Shape& s, const cedev::Params& p, hipStream_t st) {
  if (s.halves == 4) return launch_wide_h<cedev::BF16, 512, 16, 4>(p, st);
  if (s.halves == 2) {
    return s.block == 512 ? launch_wide_h<cedev::BF16, 512, 16, 2>(p, st)
                          : launch_wide_h<cedev::BF16, 1024, 16, 2>(p, st);
  }
  return s.nreg == 4 ? launch_wide_h<cedev::BF16, 1024, 4, 1>(p, st)
                     : launch_wide_h<cedev::BF16, 1024, 8, 1>(p, st);
}
}  // namespace cehost
