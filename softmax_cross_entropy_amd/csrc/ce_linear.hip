// C ABI of the linear layer fused with the cross-entropy (declared in
// include/ce.h): logits = hidden @ weight^T in row chunks (rocBLAS, bf16 in,
// fp32 out on the matrix cores), the fused cross-entropy kernels on each
// chunk's fp32 logits (gradient in place), the gradient narrowed to bf16,
// and the two gradient products d hidden = G @ weight, d weight = G^T @
// hidden. The Liger-Kernel page "Kernel Profile: CrossEntropy (Tier 3 -
// Fused/Complex)", Classification, names this fusion as the one the
// cross-entropy kernel extends with a linear layer.
#include <rocblas/rocblas.h>

#include <mutex>

#include "ce_linear_mfma.hpp"
#include "ce_plan.hpp"

#define CE_API extern "C" __attribute__((visibility("default")))

using namespace ceplan;

namespace {

// Default chunk: at most 2048 rows, and the fp32 logits, bf16 gradient and
// its transpose of a chunk within 6 GiB. Wider chunks keep the products
// wide: at 4096 x 4096 x 128256 on MI355X a step takes 10.9 ms with one
// 4096-row chunk, 11.8 ms with 2048-row chunks (2.1 GB of chunk buffers
// instead of 4.2 GB) and 16.1 ms with 1024-row chunks.
constexpr int64_t kDefaultChunkRows = 2048;
constexpr size_t kDefaultChunkBytes = size_t{6} << 30;
constexpr int kNarrowBlock = 256;
constexpr int kNarrowUnroll = 4;
constexpr int kEpilogueBlock = 1024;

// G (fp32 rows of ldl) times grad_output, rounded to bf16 (nearest even)
// into rows of ldg. One 16-byte vector of G -> one 8-byte vector of bf16;
// the padding columns past V are converted too and never read.
__global__ __launch_bounds__(kNarrowBlock) void grad_narrow_kernel(
    const float* __restrict__ g, int64_t ldl, uint32_t* __restrict__ out, int64_t ldg,
    int64_t nv4, const float* go, int per_row) {
  const int64_t r = blockIdx.y;
  const float s = go ? (per_row ? go[r] : go[0]) : 1.0f;
  const cedev::f4* src = reinterpret_cast<const cedev::f4*>(g + r * ldl);
  uint32_t* dst = out + r * (ldg / 2);
  const int64_t j0 = (static_cast<int64_t>(blockIdx.x) * kNarrowUnroll) * kNarrowBlock + threadIdx.x;
  cedev::f4 v[kNarrowUnroll];
#pragma unroll
  for (int u = 0; u < kNarrowUnroll; ++u) {
    const int64_t j = j0 + u * kNarrowBlock;
    v[u] = j < nv4 ? __builtin_nontemporal_load(src + j) : cedev::f4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int u = 0; u < kNarrowUnroll; ++u) {
    const int64_t j = j0 + u * kNarrowBlock;
    if (j < nv4) {
      dst[2 * j] = cedev::pack_bf16x2(v[u][0] * s, v[u][1] * s);
      dst[2 * j + 1] = cedev::pack_bf16x2(v[u][2] * s, v[u][3] * s);
    }
  }
}

// The same narrowing written transposed: G^T (V rows of ldt bf16) for the
// weight gradient, whose product then reads both operands without a
// transpose (NN; the NT form with G measured 4.16 against 3.49 ms at
// 4096 x 4096 x 128256 on MI355X). If gout is not null the rows of G are
// also written as grad_narrow_kernel does. A tile of 64 chunk rows x 128
// vocabulary entries goes through LDS, so the reads are row runs of 512
// (fp32) or 256 (bf16) bytes and each G^T row segment is one 128-byte line.
// ldt is a multiple of 64; entries of chunk rows past cr are written as
// zeros and never read. BF16IN: g holds G already in bf16 (rows of ldin
// elements, no scale, no gout); else fp32 rows of ldin elements.
constexpr int kTileRows = 64;
constexpr int kTileCols = 128;
constexpr int kTilePitch = kTileCols / 2 + 1;  // dwords per tile row
constexpr int kTBlock = 256;

template <bool BF16IN>
__global__ __launch_bounds__(kTBlock) void grad_narrow_t_kernel(
    const void* __restrict__ g, int64_t ldin, int64_t ncols, int64_t cr, int64_t V,
    uint32_t* __restrict__ gout, int64_t ldg, uint16_t* __restrict__ gt, int64_t ldt,
    const float* go, int per_row) {
  // The tile is kept as it was read (row r, entries 4 c4 ... 4 c4 + 3 in one
  // 8-byte piece), rows kTilePitch dwords apart: an odd pitch puts the two
  // dwords each lane stores, and the column entries each lane reads back, on
  // distinct banks across a wave.
  __shared__ uint32_t tile[kTileRows * kTilePitch];
  const int t = threadIdx.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.y) * kTileRows;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * kTileCols;
  const int c4 = t % (kTileCols / 4);  // 16-byte column of the tile
  const int rsub = t / (kTileCols / 4);
  constexpr int kRowStep = kTBlock / (kTileCols / 4);
  const int64_t v = v0 + 4 * c4;
#pragma unroll
  for (int u = 0; u < kTileRows / kRowStep; ++u) {
    const int r = u * kRowStep + rsub;
    const int64_t i = i0 + r;
    const bool in = i < cr && v < ncols;
    uint32_t lo = 0u, hi = 0u;
    if constexpr (BF16IN) {
      if (in) {
        const cedev::u2 w = __builtin_nontemporal_load(
            reinterpret_cast<const cedev::u2*>(static_cast<const uint16_t*>(g) + i * ldin + v));
        lo = w[0];
        hi = w[1];
      }
    } else {
      cedev::f4 x = {0.0f, 0.0f, 0.0f, 0.0f};
      float s = 0.0f;
      if (in) {
        x = __builtin_nontemporal_load(
            reinterpret_cast<const cedev::f4*>(static_cast<const float*>(g) + i * ldin + v));
        s = go ? (per_row ? go[i] : go[0]) : 1.0f;
      }
      lo = cedev::pack_bf16x2(x[0] * s, x[1] * s);
      hi = cedev::pack_bf16x2(x[2] * s, x[3] * s);
    }
    if (!BF16IN && gout && in) {
      uint32_t* dst = gout + i * (ldg / 2) + v / 2;
      dst[0] = lo;
      dst[1] = hi;
    }
    tile[r * kTilePitch + 2 * c4] = lo;
    tile[r * kTilePitch + 2 * c4 + 1] = hi;
  }
  __syncthreads();
  constexpr int kSegs = kTileRows / 8;  // 16-byte pieces of a G^T row segment
#pragma unroll
  for (int u = 0; u < kTileCols / (kTBlock / kSegs); ++u) {
    const int vr = u * (kTBlock / kSegs) + t / kSegs;
    const int seg = t % kSegs;
    const int64_t vv = v0 + vr;
    if (vv < V) {
      // entries (seg * 8 + j, vr) of the tile: G^T row vr, chunk rows seg * 8 + j
      const uint16_t* col = reinterpret_cast<const uint16_t*>(tile) + vr;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r0 = seg * 8 + 2 * q;
        w[q] = static_cast<uint32_t>(col[r0 * 2 * kTilePitch]) |
               (static_cast<uint32_t>(col[(r0 + 1) * 2 * kTilePitch]) << 16);
      }
      *reinterpret_cast<uint4*>(gt + vv * ldt + i0 + seg * 8) = uint4{w[0], w[1], w[2], w[3]};
    }
  }
}

// grad_weight = 0 for an empty batch (no chunk runs the weight product).
__global__ __launch_bounds__(256) void zero_rows_kernel(float* a, int64_t rows, int64_t cols,
                                                        int64_t ld) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t k = blockIdx.x * 256ll + threadIdx.x; k < cols; k += gridDim.x * 256ll)
      a[r * ld + k] = 0.0f;
}

// The reductions over every row of every chunk, after the last chunk.
__global__ __launch_bounds__(kEpilogueBlock) void linear_epilogue_kernel(cedev::Params p) {
  cedev::epilogue_reduce<kEpilogueBlock>(p);
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct LinLayout {
  int64_t C;        // rows per chunk
  int64_t ldl;      // fp32 logits row stride (16-byte rows)
  int64_t ldg;      // bf16 gradient row stride (16-byte rows)
  int64_t ldt;      // bf16 transposed gradient row stride (chunk rows, 128-byte rows)
  size_t row_ce, row_z, row_ok, part, logits, gbuf, gtbuf, total;
};

// Workspace: the cross-entropy header and per-row arrays for every row,
// partials for one chunk (the larger of a full and the last chunk's plan),
// then one chunk of fp32 logits, one of bf16 gradient and its transpose.
LinLayout lin_layout(int64_t rows, int64_t V, int64_t chunk_rows, uint32_t flags) {
  LinLayout L;
  L.ldl = round_up(V, 4);
  L.ldg = round_up(V, 8);
  const int64_t per_row = L.ldl * 4 + L.ldg * 2 + V * 2;
  int64_t C = chunk_rows;
  if (C <= 0) {
    C = static_cast<int64_t>(kDefaultChunkBytes / static_cast<size_t>(per_row));
    if (C > kDefaultChunkRows) C = kDefaultChunkRows;
  }
  if (C < 1) C = 1;
  if (C > rows) C = rows;
  L.C = C;
  L.ldt = round_up(C > 0 ? C : 1, kTileRows);
  int64_t parts = 0;
  if (rows > 0) {
    const int64_t sizes[2] = {C, rows % C};
    for (int64_t c : sizes) {
      if (c <= 0) continue;
      Plan pl;
      plan_aligned(c, V, CE_F32, flags, &pl);
      const int64_t q = c * plan_partials(pl);
      parts = q > parts ? q : parts;
    }
  }
  size_t off = kAlign;  // header
  L.row_ce = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  L.row_z = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  L.row_ok = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  L.part = off;
  off += align_up(static_cast<size_t>(parts) * sizeof(cedev::Partial));
  L.logits = off;
  off += align_up(static_cast<size_t>(C) * static_cast<size_t>(L.ldl) * 4);
  L.gbuf = off;
  off += align_up(static_cast<size_t>(C) * static_cast<size_t>(L.ldg) * 2);
  L.gtbuf = off;
  off += align_up(static_cast<size_t>(rows > 0 ? V : 0) * static_cast<size_t>(L.ldt) * 2);
  L.total = off;
  return L;
}

// The forward without gradients on the matrix-core kernel
// (ce_linear_mfma.hpp): the header, the row arrays and the (class block, row)
// partials; no logits.
struct FusedLayout {
  int64_t ncb, nrb, cpx, npc, npr, grid;
  size_t row_ce, row_z, row_ok, part, total;
};

FusedLayout fused_layout(int64_t rows, int64_t V) {
  FusedLayout F;
  F.ncb = (V + cedev::kLinTileV - 1) / cedev::kLinTileV;
  F.nrb = (rows + cedev::kLinTileR - 1) / cedev::kLinTileR;
  F.cpx = (F.ncb + 7) / 8;
  F.npc = (F.cpx + 3) / 4;
  F.npr = (F.nrb + 7) / 8;
  F.grid = 8 * F.npc * F.npr * 32;
  size_t off = kAlign;
  F.row_ce = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  F.row_z = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  F.row_ok = off;
  off += align_up(static_cast<size_t>(rows) * 4);
  F.part = off;
  off += align_up(static_cast<size_t>(F.ncb) * static_cast<size_t>(rows) * sizeof(cedev::Partial));
  F.total = off;
  return F;
}

// Calls the matrix-core forward takes: asked for with CE_F_LINEAR_ON_CHIP
// (the library GEMM path is faster at 4096 x 4096 x 128256: 4.1 against
// 4.5-4.9 ms per call on MI355X), H a multiple of the stage width, 16-byte
// rows of hidden and weight, a grid within range.
bool fused_forward_ok(const void* hidden, int64_t ld_hidden, const void* weight,
                      int64_t ld_weight, int64_t rows, int64_t H, int64_t V, uint32_t flags) {
  if (!(flags & CE_F_LINEAR_ON_CHIP)) return false;
  if (H % cedev::kLinTileK || ld_hidden % 8 || ld_weight % 8) return false;
  if (reinterpret_cast<uintptr_t>(hidden) % 16 || reinterpret_cast<uintptr_t>(weight) % 16)
    return false;
  const FusedLayout F = fused_layout(rows, V);
  return F.grid <= kMaxInt && rows <= kMaxInt;
}

template <int SC, int SM>
hipError_t launch_linear_partials_t(const cedev::Params& p, const cedev::LinArgs& g, int64_t grid,
                                    hipStream_t st) {
  cedev::linear_partials_kernel<SC, SM>
      <<<dim3(static_cast<unsigned>(grid)), cedev::kLinThreads, 0, st>>>(p, g);
  return hipGetLastError();
}

hipError_t launch_linear_partials(const cedev::Params& p, const cedev::LinArgs& g, int64_t grid,
                                  hipStream_t st) {
  const bool sc = p.softcap > 0.0f, sm = p.eps > 0.0f;
  if (sc) return sm ? launch_linear_partials_t<1, 1>(p, g, grid, st)
                    : launch_linear_partials_t<1, 0>(p, g, grid, st);
  return sm ? launch_linear_partials_t<0, 1>(p, g, grid, st)
            : launch_linear_partials_t<0, 0>(p, g, grid, st);
}

// One rocBLAS handle per device, created on first use; calls that share it
// set its stream and enqueue their products under the lock.
constexpr int kMaxDevices = 64;
std::mutex g_blas_mu;
rocblas_handle g_blas[kMaxDevices] = {};

rocblas_handle blas_handle(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  if (g_blas[dev] == nullptr) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
    g_blas[dev] = h;
  }
  return g_blas[dev];
}

// Column-major GEMM D = op(A) op(B) + beta D, bf16 inputs, fp32 output and
// accumulation (the row-major products are written as their transposes).
bool gemm_bf16_f32(rocblas_handle h, rocblas_operation ta, rocblas_operation tb, int64_t m,
                   int64_t n, int64_t k, const void* A, int64_t lda, const void* B, int64_t ldb,
                   float beta, float* D, int64_t ldd) {
  const float alpha = 1.0f;
  const rocblas_status st = rocblas_gemm_ex(
      h, ta, tb, static_cast<rocblas_int>(m), static_cast<rocblas_int>(n),
      static_cast<rocblas_int>(k), &alpha, A, rocblas_datatype_bf16_r,
      static_cast<rocblas_int>(lda), B, rocblas_datatype_bf16_r, static_cast<rocblas_int>(ldb),
      &beta, D, rocblas_datatype_f32_r, static_cast<rocblas_int>(ldd), D,
      rocblas_datatype_f32_r, static_cast<rocblas_int>(ldd), rocblas_datatype_f32_r,
      rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success;
}

}  // namespace

namespace {

// The forward without gradients: the prologue when the reduction needs it,
// the matrix-core kernel writing the partials of every (class block, row),
// then the shard finish folding each row's blocks in class order into the
// outputs (no gradient).
ce_status fused_forward(const void* hidden, int64_t ld_hidden, const void* weight,
                        int64_t ld_weight, int64_t rows, int64_t H, int64_t V,
                        const int64_t* target, const float* class_weight, int64_t ignore_index,
                        float label_smoothing, float lse_square_scale, float softcap,
                        int reduction, uint32_t flags, float* loss, float* z_loss,
                        float* token_accuracy, int64_t* argmax, int64_t* counts, char* ws,
                        const FusedLayout& F, hipStream_t st) {
  {  // header and row arrays start each call cleared (a kernel, as on the library path)
    const int64_t nf = static_cast<int64_t>(F.part / 4);
    const int64_t blocks = (nf + 255) / 256;
    const dim3 zg(static_cast<unsigned>(blocks < 1024 ? blocks : 1024), 1);
    zero_rows_kernel<<<zg, 256, 0, st>>>(reinterpret_cast<float*>(ws), 1, nf, nf);
    if (hipGetLastError() != hipSuccess) return CE_E_HIP;
  }
  cedev::Params p;
  fill_options(p, nullptr, rows, V, V, target, class_weight, ignore_index, label_smoothing,
               lse_square_scale, softcap, reduction);
  p.grad = 0;
  p.epilogue = (reduction != CE_RED_NONE || counts != nullptr) ? 1 : 0;
  p.has_hdr = (reduction == CE_RED_MEAN || (class_weight != nullptr && label_smoothing > 0.0f) ||
               (flags & CE_F_CHECK_TARGETS) || rows == 0)
                  ? 1
                  : 0;
  p.loss = loss;
  p.z_loss = z_loss;
  p.acc = token_accuracy;
  p.argmax = argmax;
  p.counts = counts;
  p.hdr = reinterpret_cast<cedev::Header*>(ws);
  p.row_ce = reinterpret_cast<float*>(ws + F.row_ce);
  p.row_z = reinterpret_cast<float*>(ws + F.row_z);
  p.row_ok = reinterpret_cast<int32_t*>(ws + F.row_ok);
  p.xstamp = next_epoch();
  if (p.has_hdr && cehost::launch_prologue(p, st) != hipSuccess) return CE_E_HIP;
  if (rows > 0) {
    cedev::LinArgs g;
    g.hidden = static_cast<const uint16_t*>(hidden);
    g.weight = static_cast<const uint16_t*>(weight);
    g.ldh = ld_hidden;
    g.ldw = ld_weight;
    g.H = static_cast<int>(H);
    g.ncb = static_cast<int>(F.ncb);
    g.nrb = static_cast<int>(F.nrb);
    g.cpx = static_cast<int>(F.cpx);
    g.npr = static_cast<int>(F.npr);
    g.parts = reinterpret_cast<cedev::Partial*>(ws + F.part);
    if (launch_linear_partials(p, g, F.grid, st) != hipSuccess) return CE_E_HIP;
    cedev::ShardArgs sa{};
    sa.v_offset = 0;
    sa.V_total = V;
    sa.weight_g = class_weight;
    sa.parts = g.parts;
    sa.G = static_cast<int>(F.ncb);
    if (cehost::launch_shard_finish(CE_F32, p, sa, false, st) != hipSuccess) return CE_E_HIP;
  }
  if (flags & CE_F_CHECK_TARGETS) return check_status(p.hdr, next_epoch(), st);
  return CE_OK;
}

}  // namespace

CE_API size_t ce_linear_workspace_bytes(int64_t rows, int64_t H, int64_t V, int64_t chunk_rows,
                                        uint32_t flags) {
  if (!valid_shape(rows, V, V) || H < 1 || H > kMaxInt || chunk_rows < 0) return 0;
  // the larger of the two paths' layouts: the gradient calls take the
  // chunked library path, the others the matrix-core forward
  const size_t a = lin_layout(rows, V, chunk_rows, flags).total;
  const size_t b = fused_layout(rows, V).total;
  return a > b ? a : b;
}

CE_API ce_status ce_linear_forward(const void* hidden, int64_t ld_hidden, const void* weight,
                                   int64_t ld_weight, int dtype, int64_t rows, int64_t H,
                                   int64_t V, const int64_t* target, const float* class_weight,
                                   int64_t ignore_index, float label_smoothing,
                                   float lse_square_scale, float softcap, int reduction,
                                   uint32_t flags, const float* grad_output, int per_row,
                                   int64_t chunk_rows, float* loss, float* z_loss,
                                   float* token_accuracy, int64_t* argmax, int64_t* counts,
                                   float* grad_hidden, int64_t ld_grad_hidden,
                                   float* grad_weight, int64_t ld_grad_weight, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (dtype != CE_BF16) return CE_E_DTYPE;
  const ce_status bad = check_options(CE_F32, rows, V, V, label_smoothing, lse_square_scale,
                                      softcap, reduction);
  if (bad != CE_OK) return bad;
  if (H < 1 || H > kMaxInt || chunk_rows < 0) return CE_E_SHAPE;
  if (ld_hidden < H || ld_weight < H || ld_hidden > kMaxInt || ld_weight > kMaxInt)
    return CE_E_SHAPE;
  if (grad_hidden && (ld_grad_hidden < H || ld_grad_hidden > kMaxInt)) return CE_E_SHAPE;
  if (grad_weight && (ld_grad_weight < H || ld_grad_weight > kMaxInt)) return CE_E_SHAPE;
  if (round_up(V, 8) > kMaxInt) return CE_E_SHAPE;
  if (loss == nullptr) return CE_E_NULL;
  if (rows > 0 && (hidden == nullptr || target == nullptr || weight == nullptr)) return CE_E_NULL;
  if (per_row && reduction != CE_RED_NONE) return CE_E_PARAM;
  const bool want_grad = grad_hidden != nullptr || grad_weight != nullptr;
  const LinLayout L = lin_layout(rows, V, chunk_rows, flags);
  const bool fused =
      !want_grad && fused_forward_ok(hidden, ld_hidden, weight, ld_weight, rows, H, V, flags);
  const FusedLayout F = fused_layout(rows, V);
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return CE_E_WORKSPACE;
  if (workspace_bytes < (fused ? F.total : L.total)) return CE_E_WORKSPACE;
  if (fused)
    return fused_forward(hidden, ld_hidden, weight, ld_weight, rows, H, V, target, class_weight,
                         ignore_index, label_smoothing, lse_square_scale, softcap, reduction,
                         flags, loss, z_loss, token_accuracy, argmax, counts,
                         static_cast<char*>(workspace), F, static_cast<hipStream_t>(stream));

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CE_E_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle blas = blas_handle(dev);
  if (blas == nullptr || rocblas_set_stream(blas, st) != rocblas_status_success) return CE_E_HIP;

  char* ws = static_cast<char*>(workspace);
  // The header, per-row arrays and partials start each call cleared (a
  // kernel, so the call may be captured in a graph): the caller need not
  // zero the workspace, and the chunk buffers after them are written
  // before they are read.
  {
    const int64_t nf = static_cast<int64_t>(L.logits / 4);
    const int64_t blocks = (nf + 255) / 256;
    const dim3 zg(static_cast<unsigned>(blocks < 1024 ? blocks : 1024), 1);
    zero_rows_kernel<<<zg, 256, 0, st>>>(reinterpret_cast<float*>(ws), 1, nf, nf);
    if (hipGetLastError() != hipSuccess) return CE_E_HIP;
  }
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  uint32_t* gbuf = reinterpret_cast<uint32_t*>(ws + L.gbuf);
  uint16_t* gtbuf = reinterpret_cast<uint16_t*>(ws + L.gtbuf);
  cedev::Params base;
  fill_options(base, logits, rows, V, L.ldl, target, class_weight, ignore_index,
               label_smoothing, lse_square_scale, softcap, reduction);
  base.grad = want_grad ? 1 : 0;
  base.epilogue = (reduction != CE_RED_NONE || counts != nullptr) ? 1 : 0;
  base.has_hdr = (reduction == CE_RED_MEAN || (class_weight != nullptr && label_smoothing > 0.0f) ||
                  (flags & CE_F_CHECK_TARGETS) || rows == 0)
                     ? 1
                     : 0;
  base.loss = loss;
  base.z_loss = z_loss;
  base.acc = token_accuracy;
  base.argmax = argmax;
  base.counts = counts;
  base.hdr = reinterpret_cast<cedev::Header*>(ws);
  base.row_ce = reinterpret_cast<float*>(ws + L.row_ce);
  base.row_z = reinterpret_cast<float*>(ws + L.row_z);
  base.row_ok = reinterpret_cast<int32_t*>(ws + L.row_ok);
  base.part = reinterpret_cast<cedev::Partial*>(ws + L.part);
  base.xstamp = next_epoch();  // one stamp for the call; each chunk has its own epoch
  base.spin_limit = (flags & CE_F_EXCHANGE_ONE_POLL) ? 1 : 0;

  // n, D and the mean scales over the whole batch, before any gradient.
  if (base.has_hdr && cehost::launch_prologue(base, st) != hipSuccess) return CE_E_HIP;

  const uint32_t path_flags =
      flags & (CE_F_FORCE_FUSED | CE_F_FORCE_SPLITV | CE_F_FORCE_SCALAR | CE_F_SHAPE_ALT);
  const char* hid = static_cast<const char*>(hidden);
  for (int64_t c0 = 0; c0 < rows; c0 += L.C) {
    const int64_t cr = rows - c0 < L.C ? rows - c0 : L.C;
    const void* xc = hid + c0 * ld_hidden * 2;
    // logits (cr x V, row-major) = hidden_chunk @ weight^T
    if (!gemm_bf16_f32(blas, rocblas_operation_transpose, rocblas_operation_none, V, cr, H, weight,
                       ld_weight, xc, ld_hidden, 0.0f, logits, L.ldl))
      return CE_E_HIP;
    cedev::Params pc = base;
    pc.rows = cr;
    pc.target = target + c0;
    pc.row_ce = base.row_ce + c0;
    pc.row_z = base.row_z + c0;
    pc.row_ok = base.row_ok + c0;
    if (reduction == CE_RED_NONE) {
      pc.loss = loss + c0;
      if (z_loss) pc.z_loss = z_loss + c0;
      if (token_accuracy) pc.acc = token_accuracy + c0;
    }
    if (argmax) pc.argmax = argmax + c0;
    pc.counts = nullptr;
    pc.no_reduce = 1;  // per-row values only; one reduction after the last chunk
    Plan pl;
    make_plan(logits, CE_F32, cr, V, L.ldl, class_weight, label_smoothing, path_flags, &pl);
    pc.S = pl.S;
    pc.chunk_vec = pl.chunk_vec;
    pc.epoch = next_epoch();
    const float* go = grad_output ? grad_output + (per_row ? c0 : 0) : nullptr;
    // Split-row plans write G x grad_output as bf16 straight from the
    // cross-entropy kernel, compacted into the first half of each logits row
    // (rows of 2 ldl bf16); other plans write fp32 G, narrowed below.
    const bool gb = want_grad && pl.path == CE_PATH_FUSED && cehost::gbf16_shape(pl.shape);
    if (gb) {
      if (cehost::launch_wide_gbf16(pl.shape, pc, go, per_row, st) != hipSuccess) return CE_E_HIP;
    } else if (cehost::launch_forward_f32(pl, pc, st) != hipSuccess) {
      return CE_E_HIP;
    }
    if (!want_grad) continue;
    const dim3 tgrid(static_cast<unsigned>((L.ldl + kTileCols - 1) / kTileCols),
                     static_cast<unsigned>((cr + kTileRows - 1) / kTileRows));
    const void* gsrc = gbuf;  // G (bf16) for the d hidden product
    int64_t ldgs = L.ldg;
    if (gb) {
      gsrc = logits;
      ldgs = 2 * L.ldl;
      if (grad_weight)
        grad_narrow_t_kernel<true><<<tgrid, kTBlock, 0, st>>>(logits, ldgs, L.ldl, cr, V, nullptr,
                                                              0, gtbuf, L.ldt, nullptr, 0);
    } else if (grad_weight) {
      grad_narrow_t_kernel<false><<<tgrid, kTBlock, 0, st>>>(logits, L.ldl, L.ldl, cr, V,
                                                             grad_hidden ? gbuf : nullptr, L.ldg,
                                                             gtbuf, L.ldt, go, per_row);
    } else {
      const int64_t nv4 = L.ldl / 4;
      const dim3 ngrid(static_cast<unsigned>((nv4 + kNarrowBlock * kNarrowUnroll - 1) /
                                             (kNarrowBlock * kNarrowUnroll)),
                       static_cast<unsigned>(cr));
      grad_narrow_kernel<<<ngrid, kNarrowBlock, 0, st>>>(logits, L.ldl, gbuf, L.ldg, nv4, go,
                                                         per_row);
    }
    if (hipGetLastError() != hipSuccess) return CE_E_HIP;
    // d hidden_chunk (cr x H) = G_chunk @ weight
    if (grad_hidden &&
        !gemm_bf16_f32(blas, rocblas_operation_none, rocblas_operation_none, H, cr, V, weight,
                       ld_weight, gsrc, ldgs, 0.0f, grad_hidden + c0 * ld_grad_hidden,
                       ld_grad_hidden))
      return CE_E_HIP;
    // d weight (V x H) (+)= G_chunk^T @ hidden_chunk, from the stored G^T
    if (grad_weight &&
        !gemm_bf16_f32(blas, rocblas_operation_none, rocblas_operation_none, H, V, cr, xc,
                       ld_hidden, gtbuf, L.ldt, c0 == 0 ? 0.0f : 1.0f, grad_weight, ld_grad_weight))
      return CE_E_HIP;
  }
  if (rows == 0 && grad_weight) {
    const dim3 zg(static_cast<unsigned>((H + 255) / 256),
                  static_cast<unsigned>(V < 65535 ? V : 65535));
    zero_rows_kernel<<<zg, 256, 0, st>>>(grad_weight, V, H, ld_grad_weight);
    if (hipGetLastError() != hipSuccess) return CE_E_HIP;
  }
  if (base.epilogue && rows > 0) {
    linear_epilogue_kernel<<<1, kEpilogueBlock, 0, st>>>(base);
    if (hipGetLastError() != hipSuccess) return CE_E_HIP;
  }
  if (flags & CE_F_CHECK_TARGETS) return check_status(base.hdr, base.xstamp, st);
  return CE_OK;
}
