// C ABI of the vocabulary-parallel cross-entropy (declared in include/ce.h):
// stage 1 (per-row partials over this device's columns) and stage 2
// (combine the gathered partials, outputs, gradient of the columns).
#include "ce_plan.hpp"
#include "ce_shard.hpp"

#define CE_API extern "C" __attribute__((visibility("default")))

using namespace ceplan;

namespace {

template <class E, int SC, int SM>
hipError_t launch_partials_t(const cedev::Params& p, const cedev::ShardArgs& sa, bool vec,
                             hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.rows));
  if (vec) {
    cedev::shard_partial_kernel<E, SC, SM, true><<<grid, cedev::kShardBlock, 0, st>>>(p, sa);
  } else {
    cedev::shard_partial_kernel<E, SC, SM, false><<<grid, cedev::kShardBlock, 0, st>>>(p, sa);
  }
  return hipGetLastError();
}

template <class E, int SC, int SM>
hipError_t launch_finish_t(const cedev::Params& p, const cedev::ShardArgs& sa, bool vec,
                           hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.rows));
  if (vec) {
    cedev::shard_finish_kernel<E, SC, SM, true><<<grid, cedev::kShardBlock, 0, st>>>(p, sa);
  } else {
    cedev::shard_finish_kernel<E, SC, SM, false><<<grid, cedev::kShardBlock, 0, st>>>(p, sa);
  }
  return hipGetLastError();
}

// Dispatch on dtype and the per-element options (softcap, smoothing).
template <template <class, int, int> class L, class... A>
hipError_t dispatch(int dtype, const cedev::Params& p, A... a) {
  const int sc = p.softcap > 0.0f, sm = p.eps > 0.0f;
#define CE_SHARD_CASE(E)                                                     \
  if (sc) return sm ? L<E, 1, 1>::run(p, a...) : L<E, 1, 0>::run(p, a...);   \
  return sm ? L<E, 0, 1>::run(p, a...) : L<E, 0, 0>::run(p, a...);
  if (dtype == CE_BF16) {
    CE_SHARD_CASE(cedev::BF16)
  }
  CE_SHARD_CASE(cedev::F32)
#undef CE_SHARD_CASE
}

template <class E, int SC, int SM>
struct Partials {
  static hipError_t run(const cedev::Params& p, cedev::ShardArgs sa, bool vec, hipStream_t st) {
    return launch_partials_t<E, SC, SM>(p, sa, vec, st);
  }
};
template <class E, int SC, int SM>
struct Finish {
  static hipError_t run(const cedev::Params& p, cedev::ShardArgs sa, bool vec, hipStream_t st) {
    return launch_finish_t<E, SC, SM>(p, sa, vec, st);
  }
};

// Shape and option checks shared by both stages.
ce_status check_shard(int dtype, int64_t rows, int64_t V, int64_t row_stride, int64_t v_offset,
                      int64_t V_total, float label_smoothing, float softcap) {
  if (dtype != CE_F32 && dtype != CE_BF16) return CE_E_DTYPE;
  if (!valid_shape(rows, V, row_stride)) return CE_E_SHAPE;
  if (v_offset < 0 || V_total < 1 || V_total > kMaxInt || v_offset + V > V_total) return CE_E_SHAPE;
  if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f)) return CE_E_PARAM;
  if (!(softcap >= 0.0f) || !isfinite(softcap)) return CE_E_PARAM;
  return CE_OK;
}

// 16-byte rows and, with weighted smoothing, 16-byte aligned slice weights.
bool shard_vec(const void* logits, int dtype, int64_t row_stride, const float* weight,
               int64_t v_offset, float eps) {
  if (reinterpret_cast<uintptr_t>(logits) % 16 || (row_stride * elem_bytes(dtype)) % 16)
    return false;
  if (weight && eps > 0.0f && reinterpret_cast<uintptr_t>(weight + v_offset) % 16) return false;
  return true;
}

}  // namespace

namespace cehost {
hipError_t launch_shard_finish(int dtype, const cedev::Params& p, const cedev::ShardArgs& sa,
                               bool vec, hipStream_t st) {
  return dispatch<Finish>(dtype, p, sa, vec, st);
}
}  // namespace cehost

CE_API size_t ce_shard_workspace_bytes(int64_t rows) {
  if (rows < 0 || rows > kMaxInt) return 0;
  return kAlign + 3 * align_up(static_cast<size_t>(rows) * 4);
}

CE_API ce_status ce_shard_partials(const void* logits, int dtype, int64_t rows, int64_t V,
                                   int64_t row_stride, int64_t v_offset, int64_t V_total,
                                   const int64_t* target, const float* weight,
                                   int64_t ignore_index, float label_smoothing, float softcap,
                                   void* partials, void* stream) {
  const ce_status bad = check_shard(dtype, rows, V, row_stride, v_offset, V_total,
                                    label_smoothing, softcap);
  if (bad != CE_OK) return bad;
  if (rows > 0 && (logits == nullptr || target == nullptr || partials == nullptr))
    return CE_E_NULL;
  if (rows == 0) return CE_OK;
  cedev::Params p;
  fill_options(p, const_cast<void*>(logits), rows, V, row_stride, target,
               weight ? weight + v_offset : nullptr, ignore_index, label_smoothing, 0.0f,
               softcap, CE_RED_NONE);
  cedev::ShardArgs sa{};
  sa.v_offset = v_offset;
  sa.V_total = V_total;
  sa.weight_g = weight;
  sa.out = static_cast<cedev::Partial*>(partials);
  const bool vec = shard_vec(logits, dtype, row_stride, weight, v_offset, label_smoothing);
  const hipError_t e =
      dispatch<Partials>(dtype, p, sa, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CE_OK : CE_E_HIP;
}

CE_API ce_status ce_shard_finish(void* logits, int dtype, int64_t rows, int64_t V,
                                 int64_t row_stride, int64_t v_offset, int64_t V_total,
                                 const int64_t* target, const float* weight,
                                 int64_t ignore_index, float label_smoothing,
                                 float lse_square_scale, float softcap, int reduction,
                                 uint32_t flags, const void* partials_all, int num_shards,
                                 float* loss, float* z_loss, float* token_accuracy,
                                 int64_t* argmax, int64_t* counts, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  ce_status bad = check_shard(dtype, rows, V, row_stride, v_offset, V_total, label_smoothing,
                              softcap);
  if (bad != CE_OK) return bad;
  bad = check_options(dtype, rows, V, row_stride, label_smoothing, lse_square_scale, softcap,
                      reduction);
  if (bad != CE_OK) return bad;
  if (num_shards < 1) return CE_E_PARAM;
  if (loss == nullptr) return CE_E_NULL;
  if (rows > 0 && (logits == nullptr || target == nullptr || partials_all == nullptr))
    return CE_E_NULL;
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0 ||
      workspace_bytes < ce_shard_workspace_bytes(rows))
    return CE_E_WORKSPACE;
  const bool vec = shard_vec(logits, dtype, row_stride, weight, v_offset, label_smoothing);

  char* ws = static_cast<char*>(workspace);
  const size_t arr = align_up(static_cast<size_t>(rows) * 4);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The prologue over all targets and class weights (V_total classes): n, D,
  // W, the mean's scales and the target check.
  cedev::Params pp;
  fill_options(pp, logits, rows, V_total, V_total, target, weight, ignore_index, label_smoothing,
               lse_square_scale, softcap, reduction);
  pp.hdr = reinterpret_cast<cedev::Header*>(ws);
  pp.epilogue = (reduction != CE_RED_NONE || counts != nullptr) ? 1 : 0;
  pp.loss = loss;
  pp.z_loss = z_loss;
  pp.acc = token_accuracy;
  pp.counts = counts;
  const bool has_hdr = reduction == CE_RED_MEAN || (weight != nullptr && label_smoothing > 0.0f) ||
                       (flags & CE_F_CHECK_TARGETS) || rows == 0;
  if (has_hdr && cehost::launch_prologue(pp, st) != hipSuccess) return CE_E_HIP;
  if (rows > 0) {
    cedev::Params p;
    fill_options(p, logits, rows, V, row_stride, target, weight ? weight + v_offset : nullptr,
                 ignore_index, label_smoothing, lse_square_scale, softcap, reduction);
    p.eps_over_v = static_cast<double>(label_smoothing) / static_cast<double>(V_total);
    p.grad = 1;
    p.epilogue = pp.epilogue;
    p.has_hdr = has_hdr ? 1 : 0;
    p.loss = loss;
    p.z_loss = z_loss;
    p.acc = token_accuracy;
    p.argmax = argmax;
    p.counts = counts;
    p.hdr = pp.hdr;
    p.row_ce = reinterpret_cast<float*>(ws + kAlign);
    p.row_z = reinterpret_cast<float*>(ws + kAlign + arr);
    p.row_ok = reinterpret_cast<int32_t*>(ws + kAlign + 2 * arr);
    p.xstamp = next_epoch();
    cedev::ShardArgs sa{};
    sa.v_offset = v_offset;
    sa.V_total = V_total;
    sa.weight_g = weight;
    sa.parts = static_cast<const cedev::Partial*>(partials_all);
    sa.G = num_shards;
    if (dispatch<Finish>(dtype, p, sa, vec, st) != hipSuccess)
      return CE_E_HIP;
  }
  // (no exchange here: a fresh stamp, which the header never holds)
  if (flags & CE_F_CHECK_TARGETS) return check_status(pp.hdr, next_epoch(), st);
  return CE_OK;
}
