// The forward without the gradient on long rows: each row streamed through
// one workgroup's registers in chunks, nothing written back to the logits.
#pragma once

#include "ce_kernels.hpp"

namespace cedev {

// ---------------------------------------------------------------------------
// nograd_rows_kernel: rows of the split-row shapes (4 K to 32 K vectors) when
// no gradient is asked for: the evaluation forward of the PR #9324 page's
// cross_entropy, and the forward that keeps the logits for a gradient
// recomputed later. The logits are only read, so a row need not stay on chip
// while a group of workgroups exchanges partials: one persistent workgroup
// streams it in chunks of NREG x BLOCK vectors, the next chunk's loads in
// flight while the current one is reduced (Liger CE profile, Tiling
// Strategy: a row of any length taken in chunks). Rows go to workgroups with
// a fixed stride (b, b + grid, ...).
//
// Pass 1 is the fused kernels' grouped pass: slots in groups of GS, first the
// group's raw maximum, then the exponentials relative to its softcapped
// maximum, one (max, sum) combine per group. Each thread keeps the first
// group holding its raw maximum; the threads holding the row maximum read
// that group back (one to two vectors) to find its first position, and the
// block takes the lowest index. The row scalars and outputs come from the
// helpers fused_row uses; the per-thread sums take the slots in chunk order,
// so the losses agree with the fused forward's within the sums' rounding,
// and the argmax and counts exactly.
// ---------------------------------------------------------------------------
template <class E, int BLOCK, int NREG, int SC, int SM>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) void nograd_rows_kernel(
    Params p) {
  constexpr int EPV = E::EPV;
  constexpr int NW = BLOCK / 64;
  constexpr int GS = (EPV == 4) ? 4 : 2;  // slots per pass-1 group
  constexpr int NG = NREG / GS;           // groups per chunk
  constexpr int CH = NREG * BLOCK;        // vectors per chunk
  static_assert(NREG % GS == 0, "whole groups per chunk");
  __shared__ RowShared<BLOCK> sh;
  __shared__ int s_last;
  if (p.self_scales) compute_self_scales<BLOCK>(p);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nv = static_cast<int>(p.V / EPV);
  const int tail = static_cast<int>(p.V - static_cast<int64_t>(nv) * EPV);
  const int64_t tail0 = static_cast<int64_t>(nv) * EPV;
  const int nch = (nv + CH - 1) / CH;
  const int tail_group = nch * NG;  // tg of the row tail: after every group
  const int voff = tid * 16;

  for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
    __syncthreads();  // every thread is done with the previous row's shared state
    const int64_t y = p.target[row];
    const bool ignored = (y == p.ignore_index);
    const bool bad = !ignored && (y < 0 || y >= p.V);
    char* rp = row_ptr(p, row, E::BYTES);
    if (ignored || bad) {
      skipped_row<E, BLOCK>(p, row, bad, rp, nv, tail);  // p.grad is 0: outputs only
      continue;
    }
    float xy = 0.0f;
    if (tid == 0) xy = E::ld(rp, y);
    float xt = 0.0f;
    if (tid < tail) xt = E::ld(rp, tail0 + tid);
    // One descriptor over the row's vectors: slots past the row read 0 and
    // are masked below, so every chunk's loads are unconditional.
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rp, nv);
    const WSlot wsl = {make_rsrc_bytes(p.weight, static_cast<int>(p.V) * 4), tid * (EPV * 4), 0};

    float tm = kLowest, ts = 0.0f, tsz = 0.0f, tb = -__builtin_inff();
    int tg = -1;
    auto load_chunk = [&](u4 (&r)[NREG], int c) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < NREG; ++k)
        r[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, (c * NREG + k) * BLOCK * 16,
                                                     kLoadNT);
    };
    auto reduce_chunk = [&](const u4 (&r)[NREG], int c) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if ((c * NREG + g * GS) * BLOCK < nv) {  // uniform: skip groups past the row
          float gx = -__builtin_inff();
#pragma unroll
          for (int q = 0; q < GS; ++q) {
            const int k = c * NREG + g * GS + q;  // slot of the row
            if (k * BLOCK < nv) {
              float f[EPV];
              E::unpack(r[g * GS + q], f);
              if ((k + 1) * BLOCK > nv) {  // the row's last, partial slot
                const bool ok = k * BLOCK + tid < nv;
#pragma unroll
                for (int i = 0; i < EPV; ++i) f[i] = ok ? f[i] : -__builtin_inff();
              }
#pragma unroll
              for (int i = 0; i < EPV; ++i) gx = __builtin_fmaxf(gx, f[i]);
            }
          }
          const bool take = gx > tb;  // strict: the first group holding the max stays
          tg = take ? c * NG + g : tg;
          tb = take ? gx : tb;
          const float zg = zval<SC>(p, __builtin_fmaxf(gx, kLowest));
          // softcap rows: the exponent t (c log2 e) - zg log2 e as one fma
          const float zgl = zg * kLog2e;
          const float cl = p.softcap * kLog2e;
          float gsum = 0.0f;
#pragma unroll
          for (int q = 0; q < GS; ++q) {
            const int k = c * NREG + g * GS + q;
            if (k * BLOCK < nv) {
              float f[EPV];
              E::unpack(r[g * GS + q], f);
              float z[EPV];
              if constexpr (SC) {
                float u[EPV];
#pragma unroll
                for (int i = 0; i < EPV; ++i) u[i] = f[i] * p.inv_softcap;
                tanh_vec<EPV>(u, z);  // t = tanh(x / c); z = c t is folded below
              } else {
#pragma unroll
                for (int i = 0; i < EPV; ++i) z[i] = f[i];
              }
              float es = 0.0f;
#pragma unroll
              for (int i = 0; i < EPV; ++i)
                es += ex2(SC ? __builtin_fmaf(z[i], cl, -zgl) : (z[i] - zg) * kLog2e);
              float zs = 0.0f;
              if constexpr (SM) {
                if (p.weight) {
                  float wk[EPV];
                  load_w<E>(p.weight, WSlot{wsl.rs, wsl.voff, k * BLOCK * EPV * 4}, wk);
#pragma unroll
                  for (int i = 0; i < EPV; ++i) zs = __builtin_fmaf(wk[i], z[i], zs);
                } else {
#pragma unroll
                  for (int i = 0; i < EPV; ++i) zs += z[i];
                }
              }
              if constexpr (SC && SM) zs *= p.softcap;  // sum of w t, times c
              if ((k + 1) * BLOCK > nv) {  // lanes past the row add nothing
                const bool ok = k * BLOCK + tid < nv;
                es = ok ? es : 0.0f;
                zs = ok ? zs : 0.0f;
              }
              gsum += es;
              if constexpr (SM) tsz += zs;
            }
          }
          ms_combine(tm, ts, zg, gsum);
        }
      }
    };
    // Two register sets: chunk c + 1 loads while chunk c is reduced. The loads
    // are unconditional (past the row they read 0 without touching memory),
    // so the compiler waits for exactly the chunk it reduces.
    u4 ra[NREG], rb[NREG];
    load_chunk(ra, 0);
    for (int c = 0; c < nch; c += 2) {
      load_chunk(rb, c + 1);
      reduce_chunk(ra, c);
      load_chunk(ra, c + 2);
      if (c + 1 < nch) reduce_chunk(rb, c + 1);
    }
    if (tid < tail) {
      // the row tail: one element per thread, after every vector in index order
      const bool take = xt > tb;
      tg = take ? tail_group : tg;
      tb = take ? xt : tb;
      const float z = zval<SC>(p, xt);
      ms_combine(tm, ts, z, 1.0f);
      if constexpr (SM) tsz = p.weight ? __builtin_fmaf(p.weight[tail0 + tid], z, tsz) : tsz + z;
    }

    Acc a;
    a.m = tm;
    a.s = ts;
    a.sz = tsz;
    a.bv = tb;
    a.bi = 0;
    wave_reduce(a);
    if (lane == 0) sh.acc[wave] = a;
    __syncthreads();
    const Acc t = block_combine_p<NW>(sh.acc);

    // ---- argmax: the threads holding the row maximum read their first group
    // holding it back and take its first position; the block takes the lowest.
    int cand = kNoIndex;
    if (tg >= 0 && tb == t.bv) {
      if (tg == tail_group) {
        cand = static_cast<int>(tail0) + tid;
      } else {
        const int k0 = (tg / NG) * NREG + (tg % NG) * GS;  // the group's first slot
#pragma unroll
        for (int q = GS - 1; q >= 0; --q) {
          const int k = k0 + q;
          if (k * BLOCK + tid < nv) {
            const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + k * BLOCK * 16, 0, 0);
            float f[EPV];
            E::unpack(v, f);
#pragma unroll
            for (int i = EPV - 1; i >= 0; --i)
              cand = (f[i] == t.bv) ? (k * BLOCK + tid) * EPV + i : cand;
          }
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cand = min(cand, __shfl_xor(cand, off, 64));
    if (lane == 0) sh.cand[wave] = cand;
    // A row holding a NaN (or +inf: its sum is NaN too): the first NaN ranks
    // above every number; the row is read again, each thread its vectors in
    // increasing order (rows like this are rare).
    const bool row_nan = t.s != t.s;  // uniform
    if (row_nan) {
      int nc = kNoIndex;
      for (int j = tid; j < nv; j += BLOCK) {
        const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, j * 16, 0, 0);
        float f[EPV];
        E::unpack(v, f);
        int vn = kNoIndex;  // the vector's first NaN
#pragma unroll
        for (int i = EPV - 1; i >= 0; --i) vn = (f[i] != f[i]) ? j * EPV + i : vn;
        nc = min(nc, vn);
      }
      if (tid < tail && xt != xt) nc = min(nc, static_cast<int>(tail0) + tid);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) nc = min(nc, __shfl_xor(nc, off, 64));
      if (lane == 0) sh.nanc[wave] = nc;
    }
    __syncthreads();

    if (tid == 0) {
      int arg = sh.cand[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) arg = min(arg, sh.cand[w]);
      if (row_nan) {
        int na = kNoIndex;
#pragma unroll
        for (int w = 0; w < NW; ++w) na = min(na, sh.nanc[w]);
        if (na != kNoIndex) arg = na;
      }
      if (arg == kNoIndex) arg = 0;  // no value above -inf: index 0
      double W, alpha, beta;
      load_scales(p, W, alpha, beta);
      const float wy = p.weight ? p.weight[y] : 1.0f;
      RowScalars rs;
      row_scalars(rs, t.m, t.s, t.sz, zval<SC>(p, xy), wy, W, p, alpha, beta);
      rs.arg = arg;
      rs.ok = (arg == y);
      write_row_outputs(p, row, rs.ce, rs.zl, rs.ok, arg);
      write_row_stats(p, row, rs.m, rs.l2s);
      if (p.epilogue) publish_row(p, row, rs.ce, rs.zl, rs.ok, 1);
    }
  }
  if (p.epilogue) {
    if (threadIdx.x == 0) s_last = arrive(p, gridDim.x);
    __syncthreads();
    if (s_last) epilogue_finish<BLOCK>(p);
  }
}

}  // namespace cedev
