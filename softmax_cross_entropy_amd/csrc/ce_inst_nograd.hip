// Instantiations of the streaming no-gradient row kernel (ce_nograd.hpp).
#include "ce_launch_impl.hpp"
#include "ce_nograd.hpp"

namespace cehost {
namespace {

// 512 threads with two sets of 8 slots (one chunk loading while the other is
// reduced), two workgroups per CU, persistent over the rows.
constexpr int kNogradBlock = 512;
constexpr int kNogradSlots = 8;

template <class E, int SC, int SM>
hipError_t launch_nograd_t(const Params& p, hipStream_t st) {
  static int cache[64] = {};
  int r = 0;
  const hipError_t e = resident_blocks(
      cedev::nograd_rows_kernel<E, kNogradBlock, kNogradSlots, SC, SM>, kNogradBlock, cache, &r);
  if (e != hipSuccess) return e;
  const int64_t grid = balanced_grid(p.rows, r);
  cedev::nograd_rows_kernel<E, kNogradBlock, kNogradSlots, SC, SM>
      <<<dim3(static_cast<unsigned>(grid)), kNogradBlock, 0, st>>>(p);
  return hipGetLastError();
}

template <class E>
hipError_t launch_nograd_h(const Params& p, hipStream_t st) {
  const bool sc = p.softcap > 0.0f;
  const bool sm = p.eps > 0.0f;
  if (sc) return sm ? launch_nograd_t<E, 1, 1>(p, st) : launch_nograd_t<E, 1, 0>(p, st);
  return sm ? launch_nograd_t<E, 0, 1>(p, st) : launch_nograd_t<E, 0, 0>(p, st);
}

}  // namespace

hipError_t launch_nograd_f32(const Params& p, hipStream_t st) {
  return launch_nograd_h<cedev::F32>(p, st);
}
hipError_t launch_nograd_bf16(const Params& p, hipStream_t st) {
  return launch_nograd_h<cedev::BF16>(p, st);
}

}  // namespace cehost
