// Template launchers shared by the per-dtype instantiation units.
#pragma once

#include "ce_kernels.hpp"
#include "ce_launch.hpp"
#include "ce_wide.hpp"

namespace cehost {

using cedev::Params;

// Workgroups of `kernel` (BLOCK threads) resident on the current device at
// once: occupancy x compute units, cached per device and kernel.
template <class K>
hipError_t resident_blocks(K kernel, int block, int* cache, int* out) {
  constexpr int kMaxDevices = 64;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int r = (dev >= 0 && dev < kMaxDevices) ? cache[dev] : 0;
  if (r == 0) {
    int per_cu = 0, ncu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    r = (per_cu > 0 ? per_cu : 1) * (ncu > 0 ? ncu : 1);
    if (dev >= 0 && dev < kMaxDevices) cache[dev] = r;
  }
  *out = r;
  return hipSuccess;
}

// Persistent grid for `units` rows (or row groups) of which at most
// `resident` run at once: the fewest workers that need no more rounds than
// `resident` would. Each worker then gets the same number of units, give or
// take one, so the last round is not left to a small share of the device
// (4096 rows on 1280 resident workgroups: 1024 workgroups of 4 rows, not
// 256 of 4 and 1024 of 3).
inline int64_t balanced_grid(int64_t units, int64_t resident) {
  if (resident < 1) resident = 1;
  if (units <= resident) return units;
  const int64_t rounds = (units + resident - 1) / resident;
  return (units + rounds - 1) / rounds;
}

// Persistent row kernel: at most as many workgroups as fit on the device at
// once (occupancy x compute units, cached per device), balanced over rows.
template <class E, int SC, int SM, int BLOCK, int NREG>
hipError_t launch_rows(const Params& p, hipStream_t st) {
  static int cache[64] = {};
  int r = 0;
  const hipError_t e =
      resident_blocks(cedev::rows_kernel<E, BLOCK, NREG, SC, SM>, BLOCK, cache, &r);
  if (e != hipSuccess) return e;
  const int64_t grid = balanced_grid(p.rows, r);
  cedev::rows_kernel<E, BLOCK, NREG, SC, SM>
      <<<dim3(static_cast<unsigned>(grid)), BLOCK, 0, st>>>(p);
  return hipGetLastError();
}

template <class E, int SC, int SM>
hipError_t launch_fused(int shape, const Params& p, hipStream_t st) {
  switch (shape) {
    case 0: return launch_rows<E, SC, SM, 256, 4>(p, st);
    case 1: return launch_rows<E, SC, SM, 256, 8>(p, st);
    case 2: return launch_rows<E, SC, SM, 256, 16>(p, st);
    case 3: return launch_rows<E, SC, SM, 512, 16>(p, st);
    case 4: return launch_rows<E, SC, SM, 512, 32>(p, st);
    case kPair512Shape:
    case kPair8Shape:
    case kQuadShape:
      // Without the gradient nothing is written back, so these rows stream
      // through one workgroup each instead of being split over a group (the
      // alternative layouts keep the split-row kernels).
      if (!p.grad) {
        if constexpr (E::EPV == 4) return launch_nograd_f32(p, st);
        return launch_nograd_bf16(p, st);
      }
      [[fallthrough]];
    case kPair1024Shape:
    case kWide4Shape:
      if constexpr (E::EPV == 4) return launch_wide_f32(kShapes[shape], p, st);
      return launch_wide_bf16(kShapes[shape], p, st);
    default: return hipErrorInvalidValue;
  }
}

// wide_kernel launch (instantiated in the ce_inst_*_wide units): persistent,
// at most one workgroup per part; rows split over G parts take a multiple
// of G workgroups (fixed groups G j ... G j + G - 1), at least one group,
// balanced over rows like the row kernel.
template <class E, int BLOCK, int NREG, int PARTS, int SC, int SM>
hipError_t launch_wide_t(const Params& p, hipStream_t st) {
  static int cache[64] = {};
  int r = 0;
  const hipError_t e =
      resident_blocks(cedev::wide_kernel<E, BLOCK, NREG, PARTS, SC, SM>, BLOCK, cache, &r);
  if (e != hipSuccess) return e;
  const int64_t groups = balanced_grid(p.rows, r / PARTS);
  const int64_t grid = (groups > 0 ? groups : 1) * PARTS;
  cedev::wide_kernel<E, BLOCK, NREG, PARTS, SC, SM>
      <<<dim3(static_cast<unsigned>(grid)), BLOCK, 0, st>>>(p);
  return hipGetLastError();
}

template <class E, int BLOCK, int NREG, int PARTS>
hipError_t launch_wide_h(const Params& p, hipStream_t st) {
  const bool sc = p.softcap > 0.0f;
  const bool sm = p.eps > 0.0f;
  if (sc) {
    return sm ? launch_wide_t<E, BLOCK, NREG, PARTS, 1, 1>(p, st)
              : launch_wide_t<E, BLOCK, NREG, PARTS, 1, 0>(p, st);
  }
  return sm ? launch_wide_t<E, BLOCK, NREG, PARTS, 0, 1>(p, st)
            : launch_wide_t<E, BLOCK, NREG, PARTS, 0, 0>(p, st);
}

// wide_kernel_gbf16: the same grid as wide_kernel.
template <class E, int BLOCK, int NREG, int PARTS, int SC, int SM>
hipError_t launch_wide_gbf16_t(const Params& p, const float* gscale, int per_row,
                               hipStream_t st) {
  static int cache[64] = {};
  int r = 0;
  const hipError_t e = resident_blocks(cedev::wide_kernel_gbf16<E, BLOCK, NREG, PARTS, SC, SM>,
                                       BLOCK, cache, &r);
  if (e != hipSuccess) return e;
  const int64_t groups = balanced_grid(p.rows, r / PARTS);
  const int64_t grid = (groups > 0 ? groups : 1) * PARTS;
  cedev::wide_kernel_gbf16<E, BLOCK, NREG, PARTS, SC, SM>
      <<<dim3(static_cast<unsigned>(grid)), BLOCK, 0, st>>>(p, gscale, per_row);
  return hipGetLastError();
}

template <class E, int BLOCK, int NREG, int PARTS>
hipError_t launch_wide_gbf16_h(const Params& p, const float* gscale, int per_row,
                               hipStream_t st) {
  const bool sc = p.softcap > 0.0f;
  const bool sm = p.eps > 0.0f;
  if (sc) {
    return sm ? launch_wide_gbf16_t<E, BLOCK, NREG, PARTS, 1, 1>(p, gscale, per_row, st)
              : launch_wide_gbf16_t<E, BLOCK, NREG, PARTS, 1, 0>(p, gscale, per_row, st);
  }
  return sm ? launch_wide_gbf16_t<E, BLOCK, NREG, PARTS, 0, 1>(p, gscale, per_row, st)
            : launch_wide_gbf16_t<E, BLOCK, NREG, PARTS, 0, 0>(p, gscale, per_row, st);
}

template <class E, int SC, int SM>
hipError_t launch_splitv(int shape, const Params& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.rows * p.S));
  switch (shape) {
    case kSplitShapeSmall:
      cedev::splitv_partial_kernel<E, 256, 4, SC, SM><<<grid, 256, 0, st>>>(p);
      break;
    case kSplitShapeLarge:
      cedev::splitv_partial_kernel<E, 512, 16, SC, SM><<<grid, 512, 0, st>>>(p);
      break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  cedev::splitv_finish_kernel<E, kSplitBlock, SC, SM><<<grid, kSplitBlock, 0, st>>>(p);
  return hipGetLastError();
}

template <class E, int SC, int SM>
hipError_t launch_path(const Plan& plan, const Params& p, hipStream_t st) {
  switch (plan.path) {
    case 1: return launch_fused<E, SC, SM>(plan.shape, p, st);
    case 2: return launch_splitv<E, SC, SM>(plan.shape, p, st);
    case 3:
      cedev::row_scalar_kernel<E, kScalarBlock, SC, SM>
          <<<dim3(static_cast<unsigned>(p.rows)), kScalarBlock, 0, st>>>(p);
      return hipGetLastError();
    default: return hipErrorInvalidValue;
  }
}

template <class E>
hipError_t launch_forward(const Plan& plan, const Params& p, hipStream_t st) {
  const bool sc = p.softcap > 0.0f;
  const bool sm = p.eps > 0.0f;
  if (sc) return sm ? launch_path<E, 1, 1>(plan, p, st) : launch_path<E, 1, 0>(plan, p, st);
  return sm ? launch_path<E, 0, 1>(plan, p, st) : launch_path<E, 0, 0>(plan, p, st);
}

template <class E, int SC, int SM>
hipError_t launch_recompute_t(const Params& p, void* grad, int64_t grad_stride, const float* go,
                              int per_row, bool vec, hipStream_t st) {
  const int64_t span = static_cast<int64_t>(cedev::kBwdBlock) * cedev::kBwdUnroll;
  const int64_t units = vec ? (p.V / E::EPV) : p.V;
  int64_t bpr = (units + span - 1) / span;
  if (bpr < 1) bpr = 1;
  const dim3 grid(static_cast<unsigned>(p.rows * bpr));
  if (vec) {
    cedev::recompute_kernel<E, SC, SM, true><<<grid, cedev::kBwdBlock, 0, st>>>(
        p, grad, grad_stride, go, per_row, static_cast<int>(bpr));
  } else {
    cedev::recompute_kernel<E, SC, SM, false><<<grid, cedev::kBwdBlock, 0, st>>>(
        p, grad, grad_stride, go, per_row, static_cast<int>(bpr));
  }
  return hipGetLastError();
}

template <class E>
hipError_t launch_recompute(const Params& p, void* grad, int64_t grad_stride, const float* go,
                            int per_row, bool vec, hipStream_t st) {
  const bool sc = p.softcap > 0.0f;
  const bool sm = p.eps > 0.0f;
  if (sc) {
    return sm ? launch_recompute_t<E, 1, 1>(p, grad, grad_stride, go, per_row, vec, st)
              : launch_recompute_t<E, 1, 0>(p, grad, grad_stride, go, per_row, vec, st);
  }
  return sm ? launch_recompute_t<E, 0, 1>(p, grad, grad_stride, go, per_row, vec, st)
            : launch_recompute_t<E, 0, 0>(p, grad, grad_stride, go, per_row, vec, st);
}

template <class E>
hipError_t launch_backward(void* grad, int64_t rows, int64_t V, int64_t stride, const float* go,
                           int per_row, bool vec, hipStream_t st) {
  const int64_t span = static_cast<int64_t>(cedev::kBwdBlock) * cedev::kBwdUnroll;
  int64_t units = vec ? (V / E::EPV) : V;
  int64_t bpr = (units + span - 1) / span;
  if (bpr < 1) bpr = 1;
  const int64_t total = rows * bpr;
  const dim3 grid(static_cast<unsigned>(total < cedev::kBwdMaxGrid ? total : cedev::kBwdMaxGrid));
  if (vec) {
    cedev::backward_kernel<E, true><<<grid, cedev::kBwdBlock, 0, st>>>(
        grad, rows, V, stride, go, per_row, static_cast<int>(bpr));
  } else {
    cedev::backward_kernel<E, false><<<grid, cedev::kBwdBlock, 0, st>>>(
        grad, rows, V, stride, go, per_row, static_cast<int>(bpr));
  }
  return hipGetLastError();
}

}  // namespace cehost
