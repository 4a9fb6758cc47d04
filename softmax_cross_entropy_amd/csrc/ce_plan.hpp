// Host-side planning shared by the C ABI translation units: argument
// checks, the kernel path and fused shape for a problem, the workspace
// layout and the launch parameters of the per-row options.
#pragma once

#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#include <atomic>

#include "ce.h"
#include "ce_launch.hpp"

namespace ceplan {

using cehost::kShapes;
using cehost::Plan;

constexpr int64_t kMaxInt = 0x7fffffffLL;
constexpr int64_t kSelfScaleRows = 65536;  // rows a workgroup counts itself (self_scales)
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline int elem_bytes(int dtype) { return dtype == CE_BF16 ? 2 : 4; }
inline int elems_per_vec(int dtype) { return dtype == CE_BF16 ? 8 : 4; }

inline bool valid_shape(int64_t rows, int64_t V, int64_t row_stride) {
  if (rows < 0 || V < 1 || row_stride < V) return false;
  if (rows > kMaxInt || V > kMaxInt) return false;
  return true;
}

// Split-V partition for nvec vectors per row: S chunks of chunk_vec vectors,
// each within the capacity of its stage-1 shape.
inline void split_plan(int64_t rows, int64_t nvec, bool forced, Plan* pl) {
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
// row. Rows of 4 K to 16 K vectors take a pair of 512-thread workgroups, rows
// of 16 K to 32 K four of them (two workgroups per CU, so one streams while
// the other waits for its group), measured faster on MI355X than one
// workgroup per row or per CU; rows of up to 4 K vectors stay with the
// 256/512-thread row kernel. CE_F_SHAPE_ALT takes the other layout where a
// row size has two (a test hook for comparing them). -1: no fused shape.
inline int fused_shape(int64_t nvec, uint32_t flags) {
  const bool alt = (flags & CE_F_SHAPE_ALT) != 0;
  for (int s = 0; s <= 1; ++s)
    if (nvec <= kShapes[s].cap()) return s;
  if (nvec <= kShapes[2].cap()) return alt ? cehost::kWide4Shape : 2;
  if (nvec <= kShapes[3].cap()) return alt ? 3 : cehost::kPair8Shape;
  if (nvec <= kShapes[4].cap()) return alt ? 4 : cehost::kPair512Shape;
  if (nvec <= kShapes[cehost::kQuadShape].cap())
    return alt ? cehost::kPair1024Shape : cehost::kQuadShape;
  return -1;
}

// Path choice for an aligned problem (alignment is checked by the caller).
inline void plan_aligned(int64_t rows, int64_t V, int dtype, uint32_t flags, Plan* pl) {
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

inline bool is_aligned(const void* logits, int dtype, int64_t row_stride, const float* weight,
                float eps) {
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0) return false;
  if ((row_stride * elem_bytes(dtype)) % 16 != 0) return false;
  if (weight && eps > 0.0f && reinterpret_cast<uintptr_t>(weight) % 16 != 0) return false;
  return true;
}

inline void make_plan(const void* logits, int dtype, int64_t rows, int64_t V, int64_t row_stride,
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
inline int plan_partials(const Plan& pl) {
  if (pl.path == CE_PATH_SPLITV) return pl.S;
  if (pl.path == CE_PATH_FUSED && kShapes[pl.shape].parts > 1)
    return 2 * kShapes[pl.shape].parts;  // 64 B per part
  return 0;
}

inline Layout layout(int64_t rows, const Plan& pl) {
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


// Checks shared by the forward and the recomputed backward.
inline ce_status check_options(int dtype, int64_t rows, int64_t V, int64_t row_stride,
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
inline void fill_options(cedev::Params& p, void* logits, int64_t rows, int64_t V, int64_t row_stride,
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


// Split rows stamp their exchanged words with a number unique to each
// launch, so no reset is needed between calls that share the workspace.
// Stamps are taken from [0xC0000001, 0xFFFFFFFF]: as fp32 bit patterns these
// are negative numbers, which no per-row loss array holds, and no other
// workspace word (counts, flags, split-V padding) takes such values either.
// They repeat after 2^30 - 1 calls: a slot could be misread only if it was
// last written exactly that many calls earlier and no call since reached its
// row.
inline uint32_t next_epoch() {
  static std::atomic<uint32_t> calls{0};
  return 0xC0000000u | (calls.fetch_add(1, std::memory_order_relaxed) % 0x3FFFFFFFu + 1u);
}

// CE_F_CHECK_TARGETS: wait for the call, then report a target out of range
// (the prologue's error bit) or a split row's exchange that gave up (the
// call's stamp in the header).
inline ce_status check_status(const cedev::Header* hdr, uint32_t stamp, hipStream_t st) {
  uint32_t w[2] = {0u, 0u};
  static_assert(offsetof(cedev::Header, xerr_epoch) == offsetof(cedev::Header, err) + 4,
                "err and xerr_epoch are adjacent");
  if (hipMemcpyAsync(w, &hdr->err, sizeof(w), hipMemcpyDeviceToHost, st) != hipSuccess)
    return CE_E_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return CE_E_HIP;
  if (w[1] == stamp) return CE_E_EXCHANGE;
  if (w[0] & 1u) return CE_E_TARGET_RANGE;
  return CE_OK;
}

}  // namespace ceplan
