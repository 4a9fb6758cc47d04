// fp32 instantiations of the forward and backward kernels.
#include "ce_launch_impl.hpp"

namespace cehost {
hipError_t launch_prologue(const cedev::Params& p, hipStream_t st) {
  cedev::prologue_kernel<cedev::kPrologueBlock><<<1, cedev::kPrologueBlock, 0, st>>>(p);
  return hipGetLastError();
}
hipError_t launch_forward_f32(const Plan& plan, const cedev::Params& p, hipStream_t st) {
  return launch_forward<cedev::F32>(plan, p, st);
}
hipError_t launch_recompute_f32(const cedev::Params& p, void* grad, int64_t grad_stride,
                                const float* go, int per_row, bool vec, hipStream_t st) {
  return launch_recompute<cedev::F32>(p, grad, grad_stride, go, per_row, vec, st);
}
hipError_t launch_backward_f32(void* grad, int64_t rows, int64_t V, int64_t stride,
                               const float* go, int per_row, bool vec, hipStream_t st) {
  return launch_backward<cedev::F32>(grad, rows, V, stride, go, per_row, vec, st);
}
}  // namespace cehost
