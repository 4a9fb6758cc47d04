// Host-side launch plan and the per-dtype launchers (defined in the
// ce_inst_*.hip translation units, which instantiate the kernel templates).
#pragma once

#include <hip/hip_runtime.h>

#include "ce_device.hpp"

namespace cehost {

// Fused row shapes: BLOCK threads, each holding NREG vectors in VGPRs and
// NLDS in LDS; capacity = BLOCK * (NREG + NLDS) 16-byte vectors per row.
struct Shape {
  int block, nreg, nlds;
  int cap() const { return block * (nreg + nlds); }
};
constexpr int kNumShapes = 7;
constexpr Shape kShapes[kNumShapes] = {
    {256, 4, 0},    // 1024 vectors:  16 KiB rows
    {256, 8, 0},    // 2048 vectors:  32 KiB
    {256, 16, 0},   // 4096 vectors:  64 KiB
    {512, 16, 0},   // 8192 vectors: 128 KiB
    {512, 32, 0},   // 16384 vectors: 256 KiB
    {512, 44, 19},  // 32256 vectors: 504 KiB (176 VGPRs + 152 KiB LDS)
    {512, 45, 19},  // 32768 vectors: 512 KiB (180 VGPRs + 152 KiB LDS)
};
constexpr int kSplitShapeSmall = 0;  // split-V chunk shapes
constexpr int kSplitShapeLarge = 3;
constexpr int kSplitBlock = 256;     // block of the split-V second stage
constexpr int kScalarBlock = 256;

struct Plan {
  int path;       // CE_PATH_*
  int shape;      // index into kShapes (fused, or split-V stage 1)
  int S;          // chunks per row (split-V)
  int chunk_vec;  // vectors per chunk (split-V)
};

hipError_t launch_prologue(const cedev::Params& p, hipStream_t st);
hipError_t launch_forward_f32(const Plan& plan, const cedev::Params& p, hipStream_t st);
hipError_t launch_forward_bf16(const Plan& plan, const cedev::Params& p, hipStream_t st);
hipError_t launch_recompute_f32(const cedev::Params& p, void* grad, int64_t grad_stride,
                                const float* go, int per_row, bool vec, hipStream_t st);
hipError_t launch_recompute_bf16(const cedev::Params& p, void* grad, int64_t grad_stride,
                                 const float* go, int per_row, bool vec, hipStream_t st);
hipError_t launch_backward_f32(void* grad, int64_t rows, int64_t V, int64_t stride,
                               const float* go, int per_row, bool vec, hipStream_t st);
hipError_t launch_backward_bf16(void* grad, int64_t rows, int64_t V, int64_t stride,
                                const float* go, int per_row, bool vec, hipStream_t st);

}  // namespace cehost
