// Host-side launch plan and the per-dtype launchers (defined in the
// ce_inst_*.hip translation units, which instantiate the kernel templates).
#pragma once

#include <hip/hip_runtime.h>

#include "ce_device.hpp"

namespace cedev {
struct ShardArgs;
}

namespace cehost {

// Fused row shapes: BLOCK threads, each holding NREG vectors in VGPRs,
// PARTS workgroups per row (2: a row pair of wide_kernel, 4: four quarter
// rows); capacity = BLOCK * NREG * PARTS 16-byte vectors per row.
struct Shape {
  int block, nreg, parts;
  int cap() const { return block * nreg * parts; }
};
constexpr int kNumShapes = 10;
constexpr Shape kShapes[kNumShapes] = {
    {256, 4, 1},    // 1024 vectors:  16 KiB rows
    {256, 8, 1},    // 2048 vectors:  32 KiB
    {256, 16, 1},   // 4096 vectors:  64 KiB
    {512, 16, 1},   // 8192 vectors: 128 KiB
    {512, 32, 1},   // 16384 vectors: 256 KiB
    {512, 16, 2},   // 16384 vectors: 256 KiB (row pair of 512-thread workgroups, two per CU)
    {1024, 16, 2},  // 32768 vectors: 512 KiB (row pair of 1024-thread workgroups)
    {1024, 4, 1},   // 4096 vectors:  64 KiB (wide_kernel, 16 waves)
    {512, 8, 2},    // 8192 vectors: 128 KiB (row pair of 512-thread workgroups, two per CU)
    {512, 16, 4},   // 32768 vectors: 512 KiB (four 512-thread workgroups, two per CU)
};
constexpr int kPair512Shape = 5;
constexpr int kPair1024Shape = 6;
constexpr int kWide4Shape = 7;
constexpr int kPair8Shape = 8;
constexpr int kQuadShape = 9;
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
// wide_kernel with block threads, nreg VGPR slots per thread and parts
// (1, 2 or 4) workgroups per row: one of the wide shapes of kShapes.
hipError_t launch_wide_f32(const Shape& s, const cedev::Params& p, hipStream_t st);
hipError_t launch_wide_bf16(const Shape& s, const cedev::Params& p, hipStream_t st);
// wide_kernel_gbf16 (fp32 logits, gradient times gscale written as bf16 rows
// compacted in place) for the split-row shapes (parts 2 or 4):
// hipErrorInvalidValue for any other shape.
bool gbf16_shape(int shape);
hipError_t launch_wide_gbf16(int shape, const cedev::Params& p, const float* gscale,
                             int per_row, hipStream_t st);
// nograd_rows_kernel (ce_nograd.hpp): rows of the default split-row shapes
// when no gradient is asked for, each streamed through one workgroup.
hipError_t launch_nograd_f32(const cedev::Params& p, hipStream_t st);
hipError_t launch_nograd_bf16(const cedev::Params& p, hipStream_t st);
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
// The vocabulary-shard finish (ce_shard.hip): fold each row's partials in
// shard order, write the outputs, and with p.grad the slice's gradient.
hipError_t launch_shard_finish(int dtype, const cedev::Params& p, const cedev::ShardArgs& sa,
                               bool vec, hipStream_t st);

}  // namespace cehost
