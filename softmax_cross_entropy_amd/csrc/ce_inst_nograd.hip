// Instantiations of the streaming no-gradient row kernel (ce_nograd.hpp).
#include "ce_launch_impl.hpp"
#include "ce_nograd.hpp"

namespace cehost {
namespace {

// Two sets of 8 slots per thread (one chunk loading while the other is
// reduced), persistent over the rows: 512 threads (two workgroups per CU)
// for fp32, 256 (four per CU) for bf16, whose 8 elements per vector give a
// chunk more arithmetic. Measured on MI355X: 256 threads took bf16 rows
// 4 % faster and fp32 rows 3.5 % slower than 512; 512 x 4 slots matched
// 512 x 8, and 1024 x 8 was 17-18 % slower.
constexpr int kNogradSlots = 8;

template <class E, int SC, int SM>
hipError_t launch_nograd_t(const Params& p, hipStream_t st) {
  constexpr int kBlock = E::EPV == 4 ? 512 : 256;
  static int cache[64] = {};
  int r = 0;
  const hipError_t e = resident_blocks(
      cedev::nograd_rows_kernel<E, kBlock, kNogradSlots, SC, SM>, kBlock, cache, &r);
  if (e != hipSuccess) return e;
  const int64_t grid = balanced_grid(p.rows, r);
  cedev::nograd_rows_kernel<E, kBlock, kNogradSlots, SC, SM>
      <<<dim3(static_cast<unsigned>(grid)), kBlock, 0, st>>>(p);
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
