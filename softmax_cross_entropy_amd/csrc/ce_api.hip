// C ABI of the fused softmax cross-entropy library (declared in include/ce.h):
// argument validation, path planning, workspace layout and the launch
// sequence prologue -> row kernel(s) (with the last-block epilogue).
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "ce.h"
#include "ce_launch.hpp"

#define CE_API extern "C" __attribute__((visibility("default")))

namespace {

using cehost::kShapes;
using cehost::Plan;

constexpr int64_t kMaxInt = 0x7fffffffLL;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dtype) { return dtype == CE_BF16 ? 2 : 4; }
int elems_per_vec(int dtype) { return dtype == CE_BF16 ? 8 : 4; }

bool valid_shape(int64_t rows, int64_t V, int64_t row_stride) {
  if (rows < 0 || V < 1 || row_stride < V) return false;
  if (rows > kMaxInt || V > kMaxInt) return false;
  return true;
}

// Split-V partition for nvec vectors per row: S chunks of chunk_vec vectors,
// each within the capacity of its stage-1 shape.
void split_plan(int64_t rows, int64_t nvec, bool forced, Plan* pl) {
  pl->path = CE_PATH_SPLITV;
  if (forced) {
    // Test hook: several small chunks even for short rows.
    int64_t cv = (nvec + 3) / 4;
    if (cv < 1) cv = 1;
    if (cv > kShapes[cehost::kSplitShapeSmall].cap()) cv = kShapes[cehost::kSplitShapeSmall].cap();
    pl->chunk_vec = static_cast<int>(cv);
    pl->shape = cehost::kSplitShapeSmall;
  } else {
    // Aim for about 1024 workgroups in total, chunks of at most 8192 vectors.
    int64_t S = rows > 0 ? (1024 + rows - 1) / rows : 1;
    const int64_t smax = (nvec + 1023) / 1024;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    int64_t cv = (nvec + S - 1) / S;
    const int64_t big = kShapes[cehost::kSplitShapeLarge].cap();
    if (cv > big) cv = big;
    if (cv < 1) cv = 1;
    pl->chunk_vec = static_cast<int>(cv);
    pl->shape = cv <= kShapes[cehost::kSplitShapeSmall].cap() ? cehost::kSplitShapeSmall
                                                              : cehost::kSplitShapeLarge;
  }
  int64_t S = (nvec + pl->chunk_vec - 1) / pl->chunk_vec;
  pl->S = static_cast<int>(S < 1 ? 1 : S);
}

// Fused shape for rows of nvec vectors: the smallest capacity that holds the
// row. Rows of 8 K to 32 K vectors take the 1024-thread layouts (one
// workgroup, or a row pair), measured faster on MI355X than 512-thread
// workgroups holding the whole row; CE_F_SHAPE_ALT takes the 512-thread
// layouts instead (a test hook for comparing them). -1: no fused shape.
int fused_shape(int64_t nvec, uint32_t flags) {
  const bool alt = (flags & CE_F_SHAPE_ALT) != 0;
  for (int s = 0; s <= 3; ++s)
    if (nvec <= kShapes[s].cap()) return s;
  if (nvec <= kShapes[4].cap()) return alt ? 4 : cehost::kWideShape;
  if (nvec <= kShapes[cehost::kPairShape].cap()) {
    if (!alt) return cehost::kPairShape;
    return nvec <= kShapes[6].cap() ? 6 : 7;
  }
  return -1;
}

// Path choice for an aligned problem (alignment is checked by the caller).
void plan_aligned(int64_t rows, int64_t V, int dtype, uint32_t flags, Plan* pl) {
  const int64_t nvec = V / elems_per_vec(dtype);
  if (flags & CE_F_FORCE_SPLITV) {
    split_plan(rows, nvec, true, pl);
    return;
  }
  const int fit = fused_shape(nvec, flags);
  const bool few_rows = rows < 256 && nvec >= 4096;
  if (fit >= 0 && ((flags & CE_F_FORCE_FUSED) || !few_rows)) {
    pl->path = CE_PATH_FUSED;
    pl->shape = fit;
    pl->S = 1;
    pl->chunk_vec = static_cast<int>(nvec);
    return;
  }
  split_plan(rows, nvec, false, pl);
}

bool is_aligned(const void* logits, int dtype, int64_t row_stride, const float* weight,
                float eps) {
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0) return false;
  if ((row_stride * elem_bytes(dtype)) % 16 != 0) return false;
  if (weight && eps > 0.0f && reinterpret_cast<uintptr_t>(weight) % 16 != 0) return false;
  return true;
}

void make_plan(const void* logits, int dtype, int64_t rows, int64_t V, int64_t row_stride,
               const float* weight, float eps, uint32_t flags, Plan* pl) {
  // The vector paths need at least one whole 16-byte vector per row.
  if ((flags & CE_F_FORCE_SCALAR) || V < elems_per_vec(dtype) ||
      !is_aligned(logits, dtype, row_stride, weight, eps)) {
    pl->path = CE_PATH_SCALAR;
    pl->shape = 0;
    pl->S = 1;
    pl->chunk_vec = 0;
    return;
  }
  plan_aligned(rows, V, dtype, flags, pl);
}

struct Layout {
  size_t row_ce, row_z, row_ok, part, total;
};

// Partials per row: S for split-V, 2 for a row pair, none otherwise.
int plan_partials(const Plan& pl) {
  if (pl.path == CE_PATH_SPLITV) return pl.S;
  if (pl.path == CE_PATH_FUSED && kShapes[pl.shape].halves == 2) return 4;  // 64 B per half
  return 0;
}

Layout layout(int64_t rows, const Plan& pl) {
  const int S = plan_partials(pl);
  Layout L;
  size_t off = kAlign;  // header
  L.row_ce = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  L.row_z = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  L.row_ok = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  L.part = off;
  off += align_up(static_cast<size_t>(rows) * static_cast<size_t>(S) * sizeof(cedev::Partial));
  L.total = off;
  return L;
}

}  // namespace

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

namespace {

// Checks shared by the forward and the recomputed backward.
ce_status check_options(int dtype, int64_t rows, int64_t V, int64_t row_stride,
                        float label_smoothing, float lse_square_scale, float softcap,
                        int reduction) {
  if (dtype != CE_F32 && dtype != CE_BF16) return CE_E_DTYPE;
  if (!valid_shape(rows, V, row_stride)) return CE_E_SHAPE;
  if (reduction != CE_RED_NONE && reduction != CE_RED_MEAN && reduction != CE_RED_SUM)
    return CE_E_PARAM;
  if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f)) return CE_E_PARAM;
  if (!(softcap >= 0.0f) || !isfinite(softcap)) return CE_E_PARAM;
  if (!(lse_square_scale >= 0.0f) || !isfinite(lse_square_scale)) return CE_E_PARAM;
  return CE_OK;
}

// The launch parameters of the per-row options (both directions).
void fill_options(cedev::Params& p, void* logits, int64_t rows, int64_t V, int64_t row_stride,
                  const int64_t* target, const float* weight, int64_t ignore_index,
                  float label_smoothing, float lse_square_scale, float softcap, int reduction) {
  memset(&p, 0, sizeof(p));
  p.logits = logits;
  p.rows = rows;
  p.V = V;
  p.row_stride = row_stride;
  p.target = target;
  p.weight = weight;
  p.ignore_index = ignore_index;
  p.eps = label_smoothing;
  p.lam = lse_square_scale;
  p.one_minus_eps = 1.0 - static_cast<double>(label_smoothing);
  p.eps_over_v = static_cast<double>(label_smoothing) / static_cast<double>(V);
  p.lam_d = lse_square_scale;
  p.softcap = softcap;
  p.inv_softcap = softcap > 0.0f ? 1.0f / softcap : 0.0f;
  p.reduction = reduction;
}

}  // namespace

CE_API ce_status ce_forward(void* logits, int dtype, int64_t rows, int64_t V, int64_t row_stride,
                            const int64_t* target, const float* weight, int64_t ignore_index,
                            float label_smoothing, float lse_square_scale, float softcap,
                            int reduction, uint32_t flags, float* loss, float* z_loss,
                            float* token_accuracy, int64_t* argmax, int64_t* counts,
                            float* row_stats, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const ce_status bad = check_options(dtype, rows, V, row_stride, label_smoothing,
                                      lse_square_scale, softcap, reduction);
  if (bad != CE_OK) return bad;
  if (loss == nullptr) return CE_E_NULL;
  if (rows > 0 && (logits == nullptr || target == nullptr)) return CE_E_NULL;

  Plan pl;
  make_plan(logits, dtype, rows, V, row_stride, weight, label_smoothing, flags, &pl);
  if (rows * (plan_partials(pl) > 0 ? plan_partials(pl) : 1) > kMaxInt) return CE_E_SHAPE;
  const Layout L = layout(rows, pl);
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
  // Row pairs stamp their partials with a number unique to this call, so no
  // reset is needed between calls that share the workspace. Stamps are taken
  // from [0xC0000001, 0xFFFFFFFF]: as fp32 bit patterns these are negative
  // numbers, which no per-row loss array holds, and no other workspace word
  // (counts, flags, split-V padding) takes such values either.
  static std::atomic<uint32_t> calls{0};
  const uint32_t ep = 0xC0000000u | (calls.fetch_add(1, std::memory_order_relaxed) % 0x3FFFFFFFu + 1u);
  p.epoch = ep;
  p.S = pl.S;
  p.chunk_vec = pl.chunk_vec;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.has_hdr && cehost::launch_prologue(p, st) != hipSuccess) return CE_E_HIP;
  if (rows > 0) {
    const hipError_t e = dtype == CE_BF16 ? cehost::launch_forward_bf16(pl, p, st)
                                          : cehost::launch_forward_f32(pl, p, st);
    if (e != hipSuccess) return CE_E_HIP;
  }
  if (flags & CE_F_CHECK_TARGETS) {
    uint32_t err = 0;
    if (hipMemcpyAsync(&err, &p.hdr->err, sizeof(err), hipMemcpyDeviceToHost, st) != hipSuccess)
      return CE_E_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return CE_E_HIP;
    if (err) return CE_E_TARGET_RANGE;
  }
  return CE_OK;
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
    default: return "unknown status";
  }
}
