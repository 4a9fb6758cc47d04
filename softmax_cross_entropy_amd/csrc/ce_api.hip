// C ABI of the fused softmax cross-entropy library (declared in include/ce.h):
// argument validation, path planning, workspace layout and the launch
// sequence prologue -> row kernel(s) (with the last-block epilogue).
#include <mutex>

#include "ce_plan.hpp"

#define CE_API extern "C" __attribute__((visibility("default")))

using namespace ceplan;
using cehost::kShapes;
using cehost::Plan;


CE_API size_t ce_workspace_bytes(int64_t rows, int64_t V, int dtype, uint32_t flags) {
  if (dtype != CE_F32 && dtype != CE_BF16) return 0;
  if (!valid_shape(rows, V, V)) return 0;
  // The largest layout any path of this shape can take (the vector paths
  // need 16-byte alignment, which is known only at the call).
  Plan pl;
  plan_aligned(rows, V, dtype, flags, &pl);
  return layout(rows, pl).total;
}

CE_API int ce_plan_path(const void* logits, int dtype, int64_t rows, int64_t V,
                        int64_t row_stride, const float* weight, float label_smoothing,
                        uint32_t flags) {
  if (dtype != CE_F32 && dtype != CE_BF16) return CE_E_DTYPE;
  if (!valid_shape(rows, V, row_stride)) return CE_E_SHAPE;
  Plan pl;
  make_plan(logits, dtype, rows, V, row_stride, weight, label_smoothing, flags, &pl);
  return pl.path;
}


// Device memory of ce_forward_noalloc: its workspace, one copy per device
// that loads the library, held until the process ends. Host code never
// passes the name itself to a kernel (on the host it is only a stand-in for
// the symbol): it uses the device address hipGetSymbolAddress returns for
// the current device, kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[CE_FORWARD_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of scratch per device; null until set up

__global__ void scratch_zero_kernel(uint4* p, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

// The current device's scratch address. The first call on a device looks
// the address up and enqueues one zero fill of the whole array on `st` (a
// kernel, ahead of that call's own kernels), which is the zero fill every
// workspace needs before its first use.
ce_status current_scratch(hipStream_t st, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CE_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CE_E_HIP;
  if (st != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(st, &sdev) != hipSuccess || sdev != dev) return CE_E_PARAM;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return CE_E_HIP;
    constexpr size_t n = CE_FORWARD_NOALLOC_MAX_BYTES / sizeof(uint4);
    scratch_zero_kernel<<<dim3(1024), dim3(256), 0, st>>>(static_cast<uint4*>(ptr), n);
    if (hipGetLastError() != hipSuccess) return CE_E_HIP;
    g_scratch[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch[dev]);
  return CE_OK;
}

// ce_forward's body on a given workspace; `noalloc`: the workspace is the
// scratch array (too small a problem is CE_E_SCRATCH, not CE_E_WORKSPACE).
ce_status forward_on(void* logits, int dtype, int64_t rows, int64_t V, int64_t row_stride,
                     const int64_t* target, const float* weight, int64_t ignore_index,
                     float label_smoothing, float lse_square_scale, float softcap, int reduction,
                     uint32_t flags, float* loss, float* z_loss, float* token_accuracy,
                     int64_t* argmax, int64_t* counts, float* row_stats, void* workspace,
                     size_t workspace_bytes, bool noalloc, void* stream) {
  const ce_status bad = check_options(dtype, rows, V, row_stride, label_smoothing,
                                      lse_square_scale, softcap, reduction);
  if (bad != CE_OK) return bad;
  if (loss == nullptr) return CE_E_NULL;
  if (rows > 0 && (logits == nullptr || target == nullptr)) return CE_E_NULL;

  Plan pl;
  make_plan(logits, dtype, rows, V, row_stride, weight, label_smoothing, flags, &pl);
  if (rows * (plan_partials(pl) > 0 ? plan_partials(pl) : 1) > kMaxInt) return CE_E_SHAPE;
  const Layout L = layout(rows, pl);
  if (noalloc) {
    if (L.total > CE_FORWARD_NOALLOC_MAX_BYTES) return CE_E_SCRATCH;
    const ce_status sc = current_scratch(static_cast<hipStream_t>(stream),
                                         reinterpret_cast<char**>(&workspace));
    if (sc != CE_OK) return sc;
    workspace_bytes = CE_FORWARD_NOALLOC_MAX_BYTES;
  }
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return CE_E_WORKSPACE;
  if (workspace_bytes < L.total) return CE_E_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  cedev::Params p;
  fill_options(p, logits, rows, V, row_stride, target, weight, ignore_index, label_smoothing,
               lse_square_scale, softcap, reduction);
  p.grad = (flags & CE_F_GRAD) ? 1 : 0;
  p.epilogue = (reduction != CE_RED_NONE || counts != nullptr) ? 1 : 0;
  // The prologue is needed before any gradient is written only for the mean
  // scales (1/D, 1/n), the weight sum of weighted smoothing and the target
  // check; an empty batch also takes it (it writes the reductions).
  p.has_hdr = (reduction == CE_RED_MEAN || (weight != nullptr && label_smoothing > 0.0f) ||
               (flags & CE_F_CHECK_TARGETS) || rows == 0)
                  ? 1
                  : 0;
  // A mean whose only batch-wide inputs are n and D (no weighted smoothing,
  // no target check) on the fused path: every persistent workgroup counts
  // them itself (a read of the targets from L2) instead of waiting for a
  // prologue launch. Up to kSelfScaleRows rows, so that read stays small.
  if (reduction == CE_RED_MEAN && !(weight != nullptr && label_smoothing > 0.0f) &&
      !(flags & CE_F_CHECK_TARGETS) && rows > 0 && rows <= kSelfScaleRows &&
      pl.path == CE_PATH_FUSED) {
    p.has_hdr = 0;
    p.self_scales = 1;
  }
  p.loss = loss;
  p.z_loss = z_loss;
  p.acc = token_accuracy;
  p.argmax = argmax;
  p.counts = counts;
  p.row_stats = row_stats;
  p.hdr = reinterpret_cast<cedev::Header*>(ws);
  p.row_ce = reinterpret_cast<float*>(ws + L.row_ce);
  p.row_z = reinterpret_cast<float*>(ws + L.row_z);
  p.row_ok = reinterpret_cast<int32_t*>(ws + L.row_ok);
  p.part = reinterpret_cast<cedev::Partial*>(ws + L.part);
  const uint32_t ep = next_epoch();
  p.epoch = ep;
  p.xstamp = ep;
  p.spin_limit = (flags & CE_F_EXCHANGE_ONE_POLL) ? 1 : 0;
  p.S = pl.S;
  p.chunk_vec = pl.chunk_vec;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.has_hdr && cehost::launch_prologue(p, st) != hipSuccess) return CE_E_HIP;
  if (rows > 0) {
    const hipError_t e = dtype == CE_BF16 ? cehost::launch_forward_bf16(pl, p, st)
                                          : cehost::launch_forward_f32(pl, p, st);
    if (e != hipSuccess) return CE_E_HIP;
  }
  if (flags & CE_F_CHECK_TARGETS) return check_status(p.hdr, ep, st);
  return CE_OK;
}

}  // namespace

CE_API ce_status ce_forward(void* logits, int dtype, int64_t rows, int64_t V, int64_t row_stride,
                            const int64_t* target, const float* weight, int64_t ignore_index,
                            float label_smoothing, float lse_square_scale, float softcap,
                            int reduction, uint32_t flags, float* loss, float* z_loss,
                            float* token_accuracy, int64_t* argmax, int64_t* counts,
                            float* row_stats, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return forward_on(logits, dtype, rows, V, row_stride, target, weight, ignore_index,
                    label_smoothing, lse_square_scale, softcap, reduction, flags, loss, z_loss,
                    token_accuracy, argmax, counts, row_stats, workspace, workspace_bytes, false,
                    stream);
}

CE_API ce_status ce_forward_noalloc(void* logits, int dtype, int64_t rows, int64_t V,
                                    int64_t row_stride, const int64_t* target,
                                    const float* weight, int64_t ignore_index,
                                    float label_smoothing, float lse_square_scale, float softcap,
                                    int reduction, uint32_t flags, float* loss, float* z_loss,
                                    float* token_accuracy, int64_t* argmax, int64_t* counts,
                                    float* row_stats, void* stream) {
  return forward_on(logits, dtype, rows, V, row_stride, target, weight, ignore_index,
                    label_smoothing, lse_square_scale, softcap, reduction, flags, loss, z_loss,
                    token_accuracy, argmax, counts, row_stats, nullptr, 0, true, stream);
}

CE_API ce_status ce_backward(void* grad, int dtype, int64_t rows, int64_t V, int64_t row_stride,
                             const float* grad_output, int per_row, void* stream) {
  if (dtype != CE_F32 && dtype != CE_BF16) return CE_E_DTYPE;
  if (!valid_shape(rows, V, row_stride)) return CE_E_SHAPE;
  if (grad_output == nullptr) return CE_E_NULL;
  if (rows > 0 && grad == nullptr) return CE_E_NULL;
  if (rows == 0) return CE_OK;
  const bool vec = reinterpret_cast<uintptr_t>(grad) % 16 == 0 &&
                   (row_stride * elem_bytes(dtype)) % 16 == 0;
  const int64_t span = static_cast<int64_t>(cedev::kBwdBlock) * cedev::kBwdUnroll;
  const int64_t units = vec ? V / elems_per_vec(dtype) : V;
  const int64_t bpr = units / span + 1;
  if (rows * bpr > kMaxInt) return CE_E_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e =
      dtype == CE_BF16
          ? cehost::launch_backward_bf16(grad, rows, V, row_stride, grad_output, per_row, vec, st)
          : cehost::launch_backward_f32(grad, rows, V, row_stride, grad_output, per_row, vec, st);
  return e == hipSuccess ? CE_OK : CE_E_HIP;
}

CE_API ce_status ce_backward_recompute(const void* logits, int dtype, int64_t rows, int64_t V,
                                       int64_t row_stride, const int64_t* target,
                                       const float* weight, int64_t ignore_index,
                                       float label_smoothing, float lse_square_scale,
                                       float softcap, int reduction, const float* row_stats,
                                       const float* grad_output, int per_row, void* grad,
                                       int64_t grad_stride, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const ce_status bad = check_options(dtype, rows, V, row_stride, label_smoothing,
                                      lse_square_scale, softcap, reduction);
  if (bad != CE_OK) return bad;
  if (!valid_shape(rows, V, grad_stride)) return CE_E_SHAPE;
  if (grad_output == nullptr) return CE_E_NULL;
  if (rows > 0 && (logits == nullptr || target == nullptr || row_stats == nullptr ||
                   grad == nullptr))
    return CE_E_NULL;
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0 ||
      workspace_bytes < kAlign)
    return CE_E_WORKSPACE;
  if (grad == logits && grad_stride != row_stride) return CE_E_SHAPE;
  if (rows == 0) return CE_OK;
  const int eb = elem_bytes(dtype);
  const bool vec = reinterpret_cast<uintptr_t>(logits) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(grad) % 16 == 0 && (row_stride * eb) % 16 == 0 &&
                   (grad_stride * eb) % 16 == 0 &&
                   !(weight && label_smoothing > 0.0f && reinterpret_cast<uintptr_t>(weight) % 16);
  const int64_t span = static_cast<int64_t>(cedev::kBwdBlock) * cedev::kBwdUnroll;
  const int64_t units = vec ? V / elems_per_vec(dtype) : V;
  const int64_t bpr = units / span + 1;
  if (rows * bpr > kMaxInt) return CE_E_SHAPE;

  cedev::Params p;
  fill_options(p, const_cast<void*>(logits), rows, V, row_stride, target, weight, ignore_index,
               label_smoothing, lse_square_scale, softcap, reduction);
  p.row_stats = const_cast<float*>(row_stats);
  p.hdr = reinterpret_cast<cedev::Header*>(workspace);
  // The same scales as the forward: the mean's 1/D and 1/n, and W for
  // weighted smoothing, from the prologue.
  p.has_hdr = (reduction == CE_RED_MEAN || (weight != nullptr && label_smoothing > 0.0f)) ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.has_hdr && cehost::launch_prologue(p, st) != hipSuccess) return CE_E_HIP;
  const hipError_t e =
      dtype == CE_BF16
          ? cehost::launch_recompute_bf16(p, grad, grad_stride, grad_output, per_row, vec, st)
          : cehost::launch_recompute_f32(p, grad, grad_stride, grad_output, per_row, vec, st);
  return e == hipSuccess ? CE_OK : CE_E_HIP;
}

CE_API const char* ce_status_string(int status) {
  switch (status) {
    case CE_OK: return "ok";
    case CE_E_NULL: return "a required pointer is NULL";
    case CE_E_SHAPE: return "invalid shape (rows < 0, V < 1, row_stride < V, or too large)";
    case CE_E_DTYPE: return "unknown dtype";
    case CE_E_PARAM: return "invalid reduction, label_smoothing, softcap or lse_square_scale";
    case CE_E_WORKSPACE: return "workspace NULL, too small or not 256-byte aligned";
    case CE_E_HIP: return "HIP runtime or kernel launch error";
    case CE_E_TARGET_RANGE: return "a target is outside [0, V) and not ignore_index";
    case CE_E_EXCHANGE:
      return "a row split over workgroups gave up waiting for one of its parts (NaN results)";
    case CE_E_SCRATCH:
      return "the problem needs more workspace than ce_forward_noalloc's static scratch holds";
    default: return "unknown status";
  }
}
