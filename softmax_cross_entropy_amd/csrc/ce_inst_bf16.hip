// bf16 instantiations of the forward and backward kernels.
#include "ce_launch_impl.hpp"

namespace cehost {
hipError_t launch_forward_bf16(const Plan& plan, const cedev::Params& p, hipStream_t st) {
  return launch_forward<cedev::BF16>(plan, p, st);
}
hipError_t launch_recompute_bf16(const cedev::Params& p, void* grad, int64_t grad_stride,
                                 const float* go, int per_row, bool vec, hipStream_t st) {
  return launch_recompute<cedev::BF16>(p, grad, grad_stride, go, per_row, vec, st);
}
hipError_t launch_backward_bf16(void* grad, int64_t rows, int64_t V, int64_t stride,
                                const float* go, int per_row, bool vec, hipStream_t st) {
  return launch_backward<cedev::BF16>(grad, rows, V, stride, go, per_row, vec, st);
}
}  // namespace cehost
