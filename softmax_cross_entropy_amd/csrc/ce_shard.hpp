// Vocabulary-parallel cross-entropy: the part one device runs when the
// classes of a (rows, V_total) logits matrix are split over G devices, each
// holding the columns [v_offset, v_offset + V) of every row.
//
// The loss and gradient of a row need its log-sum-exp over all V_total
// classes, so each device first reduces its columns to one partial per row
// (stage 1: max, sum of exponentials under it, smoothing sum, largest raw
// logit and its first global index, the target logit when the target is
// one of its classes); the G partial arrays are gathered (the all-gather of
// a multi-device run); every device then combines the G partials of a row in
// shard order, so all compute bitwise identical row scalars, and writes its
// columns' gradient in place (stage 2, which reads its columns again). This
// is the split-V method of the Liger-Kernel page "Kernel Profile:
// CrossEntropy (Tier 3 - Fused/Complex)" (Tiling Strategy: a row of any
// length in chunks) with the chunks on different devices; the tt-mlir PR
// #9324 page's commit list moves the composites towards multi-chip sharding.
#pragma once

#include "ce_kernels.hpp"

namespace cedev {

struct ShardArgs {
  int64_t v_offset;        // global class index of this slice's first column
  int64_t V_total;         // classes over all shards
  const float* weight_g;   // class weights indexed globally (V_total), or null
  Partial* out;            // stage 1: (rows) partials of this slice
  const Partial* parts;    // stage 2: (G, rows) partials, shards by increasing v_offset
  int G;
};

constexpr int kShardBlock = 256;
constexpr int kShardUnroll = 16;  // vectors per thread in flight (4096 per workgroup)

// W = sum of all class weights (the prologue's, over V_total) or V_total,
// and the mean's scales from the prologue when it ran.
__device__ __forceinline__ void shard_scales(const Params& p, const ShardArgs& sa, double& W,
                                             double& alpha, double& beta) {
  W = (p.has_hdr && sa.weight_g) ? p.hdr->W : static_cast<double>(sa.V_total);
  alpha = p.has_hdr ? p.hdr->alpha : 1.0;
  beta = p.has_hdr ? p.hdr->beta : 1.0;
}

// Stage 1: one workgroup per row over the slice (p.V columns; p.weight
// points at this slice's first class weight). VEC: 16-byte rows (vector
// loads, the V mod EPV tail as elements); else every column as an element.
template <class E, int SC, int SM, bool VEC>
__global__ __launch_bounds__(kShardBlock) void shard_partial_kernel(Params p, ShardArgs sa) {
  constexpr int EPV = E::EPV;
  constexpr int BLOCK = kShardBlock;
  constexpr int NW = BLOCK / 64;
  constexpr int U = kShardUnroll;
  __shared__ Acc s_acc[NW];
  __shared__ int s_cand[NW];
  __shared__ int s_nan[NW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t y = p.target[row];
  const char* rp = row_ptr(p, row, E::BYTES);
  if (y == p.ignore_index || y < 0 || y >= sa.V_total) {
    // not counted: stage 2 writes its outputs; a defined partial all the same
    if (tid == 0) {
      Partial q = {kLowest, 0.0f, 0.0f, -__builtin_inff(), kNoIndex, 0.0f, 0, 0};
      sa.out[row] = q;
    }
    return;
  }
  const int nv = VEC ? static_cast<int>(p.V / EPV) : 0;
  const int64_t e_from = static_cast<int64_t>(nv) * EPV;  // first element past the vectors
  Acc a;
  acc_init(a);
  if constexpr (VEC) {
    const u4* vp = reinterpret_cast<const u4*>(rp);
    for (int j0 = 0; j0 < nv; j0 += BLOCK * U) {
      u4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * BLOCK + tid;
        v[u] = j < nv ? __builtin_nontemporal_load(vp + j) : u4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * BLOCK + tid;
        if (j < nv) {
          float f[EPV];
          E::unpack(v[u], f);
          pass1_vec<E, SC, SM>(p, a, f, j, j);
        }
      }
    }
  }
  // elements past the vectors: slots nv + (k - e_from), after every vector slot
  for (int64_t k = e_from + tid; k < p.V; k += BLOCK)
    pass1_one<SC, SM>(p, a, E::ld(rp, k), nv + static_cast<int>(k - e_from), k);
  wave_reduce(a);
  if (lane == 0) s_acc[wave] = a;
  __syncthreads();
  const Acc t = block_combine<NW>(s_acc);
  // first position of the largest raw logit: a vector slot is read again
  // (by one thread) to find its first element equal to the maximum
  if (tid == 0) {
    int arg = kNoIndex;
    if (t.bi != kNoIndex) {
      if (t.bi >= nv) {
        arg = static_cast<int>(e_from) + (t.bi - nv);
      } else {
        float f[EPV];
        E::unpack(reinterpret_cast<const u4*>(rp)[t.bi], f);
        int pos = 0;
#pragma unroll
        for (int i = EPV - 1; i >= 0; --i) pos = (f[i] == t.bv) ? i : pos;
        arg = t.bi * EPV + pos;
      }
    }
    s_cand[0] = arg;
  }
  // a slice holding a NaN (its sum is NaN): its first NaN is the argmax
  const bool has_nan = t.s != t.s;  // uniform
  if (has_nan) {
    int nc = kNoIndex;
    for (int64_t k = p.V - 1 - tid; k >= 0; k -= BLOCK) {
      const float x = E::ld(rp, k);
      nc = (x != x) ? static_cast<int>(k) : nc;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) nc = min(nc, __shfl_xor(nc, off, 64));
    if (lane == 0) s_nan[wave] = nc;
  }
  __syncthreads();
  if (tid == 0) {
    int arg = s_cand[0];
    float bv = t.bv;
    if (has_nan) {
      int na = kNoIndex;
      for (int w = 0; w < NW; ++w) na = min(na, s_nan[w]);
      if (na != kNoIndex) {
        arg = na;
        bv = __builtin_nanf("");
      }
    }
    const int64_t yl = y - sa.v_offset;
    const bool here = yl >= 0 && yl < p.V;
    Partial q;
    q.m = t.m;
    q.s = t.s;
    q.sz = t.sz;
    q.bv = bv;
    q.bi = arg == kNoIndex ? kNoIndex : static_cast<int>(sa.v_offset + arg);
    q.xy = here ? E::ld(rp, yl) : 0.0f;
    q.has_y = here ? 1 : 0;
    q.pad = 0;
    sa.out[row] = q;
  }
}

// Wave 0: the row's G partials folded in a fixed tree: lane l folds the
// partials l K .. l K + K - 1 (K = ceil(G / 64)) in shard order, then the
// lanes combine in a butterfly, each pair taking the lower lane's value
// first, so every lane ends with the same bits and every device that folds
// the same partials gets them too. Returns (m, s, sz, largest raw logit, its
// index, target logit).
__device__ __forceinline__ void fold_shards(const Params& p, const ShardArgs& sa, int64_t row,
                                            float& m, float& s, float& sz, float& bv, int& bi,
                                            float& xy) {
  const int lane = threadIdx.x & 63;
  const int K = (sa.G + 63) / 64;
  m = kLowest;
  s = 0.0f;
  sz = 0.0f;
  bv = -__builtin_inff();
  bi = kNoIndex;
  xy = 0.0f;
  int hy = 0;
  for (int k = 0; k < K; ++k) {
    const int gi = lane * K + k;
    if (gi < sa.G) {
      const Partial q = sa.parts[static_cast<int64_t>(gi) * p.rows + row];
      ms_combine(m, s, q.m, q.s);
      sz += q.sz;
      arg_combine(bv, bi, q.bv, q.bi);  // equal values: the lower index
      if (q.has_y) {
        xy = q.xy;
        hy = 1;
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
    const float z2 = __shfl_xor(sz, off, 64), b2 = __shfl_xor(bv, off, 64);
    const int i2 = __shfl_xor(bi, off, 64), h2 = __shfl_xor(hy, off, 64);
    const float y2 = __shfl_xor(xy, off, 64);
    const bool low = (lane & off) == 0;
    float ma = low ? m : m2, sa_ = low ? s : s2;
    const float mb = low ? m2 : m, sb = low ? s2 : s;
    ms_combine(ma, sa_, mb, sb);
    m = ma;
    s = sa_;
    sz = low ? sz + z2 : z2 + sz;
    arg_combine(bv, bi, b2, i2);  // symmetric: the same result in both lanes
    if (h2) {
      xy = y2;
      hy = 1;
    }
  }
}

// Stage 2: one workgroup per row (one arrival per row at the epilogue's
// counter). The loads of the row's first span (kShardBlock x U vectors, the
// whole slice up to 4096 vectors) go out first, as they do not depend on the
// row scalars; wave 0 folds the row's G partials in shard order and thread 0
// computes the row scalars and writes the row's outputs; then each span's
// gradient is written over the logits, the next span loaded after it.
template <class E, int SC, int SM, bool VEC>
__global__ __launch_bounds__(kShardBlock) void shard_finish_kernel(Params p, ShardArgs sa) {
  constexpr int EPV = E::EPV;
  constexpr int BLOCK = kShardBlock;
  constexpr int U = kShardUnroll;
  __shared__ RowScalars s_rs;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t y = p.target[row];
  const bool ignored = y == p.ignore_index;
  const bool bad = !ignored && (y < 0 || y >= sa.V_total);
  const bool skip = ignored || bad;
  char* rp = row_ptr(p, row, E::BYTES);
  const int64_t yl = y - sa.v_offset;  // the target's column in this slice, if any
  const int nvec = VEC ? static_cast<int>(p.V / EPV) : 0;
  const int64_t tail0 = static_cast<int64_t>(nvec) * EPV;
  const bool owns_y = VEC && p.grad && !skip && yl >= 0 && yl < tail0 &&
                      static_cast<int>(yl / EPV) % BLOCK == tid;
  const float xy_own = owns_y ? E::ld(rp, yl) : 0.0f;  // read before any store
  u4 v[VEC ? U : 1];
  const u4* vp = reinterpret_cast<const u4*>(rp);
  if constexpr (VEC) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = u * BLOCK + tid;
      v[u] = (p.grad && !skip && j < nvec) ? __builtin_nontemporal_load(vp + j)
                                           : u4{0u, 0u, 0u, 0u};
    }
  }
  if (tid < 64) {
    float m = 0.0f, s = 0.0f, sz = 0.0f, bv = 0.0f, xy = 0.0f;
    int bi = kNoIndex;
    if (!skip) fold_shards(p, sa, row, m, s, sz, bv, bi, xy);
    if (tid == 0) {
      RowScalars rs{};
      if (skip) {
        const float q = bad ? __builtin_nanf("") : 0.0f;
        rs.ce = rs.zl = q;
        rs.arg = -1;
        rs.ok = 0;
      } else {
        if (bi == kNoIndex) bi = 0;
        double W, alpha, beta;
        shard_scales(p, sa, W, alpha, beta);
        const float wy = sa.weight_g ? sa.weight_g[y] : 1.0f;
        row_scalars(rs, m, s, sz, zval<SC>(p, xy), wy, W, p, alpha, beta);
        rs.arg = bi;
        rs.ok = (bi == y);
      }
      s_rs = rs;
      write_row_outputs(p, row, rs.ce, rs.zl, rs.ok, rs.arg);
      if (p.epilogue)
        s_last = epilogue_publish(p, row, true, rs.ce, rs.zl, rs.ok, skip ? 0 : 1, gridDim.x);
    }
  }
  __syncthreads();
  const RowScalars rs = s_rs;
  if (p.grad) {
    if constexpr (VEC) {
      u4* wp = reinterpret_cast<u4*>(rp);
      for (int j0 = 0; j0 < nvec; j0 += BLOCK * U) {
        if (j0 > 0) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int j = j0 + u * BLOCK + tid;
            v[u] = (!skip && j < nvec) ? __builtin_nontemporal_load(vp + j) : u4{0u, 0u, 0u, 0u};
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + u * BLOCK + tid;
          if (j < nvec) {
            const u4 g = skip ? u4{0u, 0u, 0u, 0u} : grad_vec<E, SC, SM, true>(p, rs, v[u], j, -1);
            __builtin_nontemporal_store(g, wp + j);
          }
        }
      }
      if (tail0 + tid < p.V) {
        const int64_t k = tail0 + tid;
        float gk = 0.0f;
        if (!skip) {
          const float wk = (SM && p.weight) ? p.weight[k] : 1.0f;
          gk = grad_one<SC, SM>(p, rs, E::ld(rp, k), wk, k == yl);
        }
        E::st_nt(rp, k, gk);
      }
      // the one-hot term, rewritten by the thread that stored the target's vector
      if (owns_y) {
        const float wy = (SM && p.weight) ? p.weight[yl] : 1.0f;
        E::st_nt(rp, yl, grad_one<SC, SM>(p, rs, xy_own, wy, true));
      }
    } else {
      for (int64_t k = tid; k < p.V; k += BLOCK) {
        float gk = 0.0f;
        if (!skip) {
          const float wk = (SM && p.weight) ? p.weight[k] : 1.0f;
          gk = grad_one<SC, SM>(p, rs, E::ld(rp, k), wk, k == yl);
        }
        E::st(rp, k, gk);
      }
    }
  }
  if (p.epilogue) {
    __syncthreads();
    if (s_last) epilogue_finish<BLOCK>(p);
  }
}

}  // namespace cedev
