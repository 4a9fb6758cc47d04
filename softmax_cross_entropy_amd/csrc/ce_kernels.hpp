// Kernel templates of the fused softmax cross-entropy forward + gradient.
//
// The method (Liger-Kernel page "Kernel Profile: CrossEntropy (Tier 3 -
// Fused/Complex)", Key Patterns): per row, an online softmax pass gives the
// max and log-sum-exp, a second pass writes softmax minus the smoothed
// one-hot over the logits in place (gradient-in-forward), and the backward
// only rescales that gradient by grad_output.
//
// MI355X design (not the page's Triton loop):
//  * rows_kernel: persistent workgroups, one row at a time each, rows claimed
//    in the order workgroups finish. The whole row is read from HBM once
//    with non-temporal dwordx4 buffer loads and kept in VGPRs, so the
//    gradient pass reads registers instead of re-reading HBM: 1 read + 1
//    write per logit. fp32 rows keep exp(x - group max) in place of x, so
//    the gradient pass is one multiply per element. Longer rows are split
//    over a group of workgroups (ce_wide.hpp).
//  * splitv_partial_kernel + splitv_finish_kernel: the row is split into S
//    chunks held by different workgroups; stage 1 writes per-chunk partials
//    (max, sum, argmax, target logit), stage 2 combines them in a fixed
//    order and writes its chunk's gradient. For rows that exceed one CU's
//    on-chip storage or for batches with too few rows to fill 256 CUs.
//  * row_scalar_kernel: rows that are not 16-byte aligned (any V, any
//    stride); element loads, same math.
//  * prologue_kernel: n, D = sum w[target], W = sum w, the mean scales and
//    the target range check, needed before any gradient is written.
//  * backward_kernel: grad *= grad_output (scalar or per row), in place.
#pragma once

#include "ce_device.hpp"

namespace cedev {


// Raw buffer descriptor over nvec 16-byte vectors at base (stride 0: byte
// offsets; the fourth word selects 32-bit data on gfx9-family GPUs). Loads
// past the end return 0 and stores past the end are dropped by the hardware.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kStoreNT = 2;  // non-temporal store (streaming gradient)
constexpr int kLoadNT = 2;   // non-temporal load (each logit is read once)
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kWaitVmcnt8 = 0x0F78;  // vmcnt(8), the other counters not waited on

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nvec) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           nvec * 16, kRsrcWord3);
}
// The same over `bytes` bytes (a row's V elements).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_bytes(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kRsrcWord3);
}
// Zero in a VGPR that the compiler cannot see through.
__device__ __forceinline__ uint32_t opaque_zero() {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Softcapped value z = c tanh(x / c) (Liger-Kernel CE profile, Forward Pass:
// softcap; the tanh form is the reading taken for "softcapping").
template <int SC>
__device__ __forceinline__ float zval(const Params& p, float x) {
  if constexpr (SC) {
    return p.softcap * tanh_f(x * p.inv_softcap);
  } else {
    return x;
  }
}

// Weights of the EPV classes of vector jg (weighted smoothing only), for
// paths whose lanes stop at the row's last vector.
template <class E>
__device__ __forceinline__ void load_w(const float* w, int64_t jg, float (&wk)[E::EPV]) {
  const f4* wv = reinterpret_cast<const f4*>(w + jg * E::EPV);
#pragma unroll
  for (int q = 0; q < E::EPV / 4; ++q) {
    const f4 t = wv[q];
    wk[4 * q + 0] = t[0];
    wk[4 * q + 1] = t[1];
    wk[4 * q + 2] = t[2];
    wk[4 * q + 3] = t[3];
  }
}

// A vector's weights in the fused row kernels, whose lanes past the row (or
// part) run the slot's code with their stores dropped: read through a
// descriptor over the V weights (rs), at the lane's byte offset voff plus
// the slot's uniform offset soff, so those lanes get 0 instead of reading
// past the array, and no per-vector address arithmetic is needed.
struct WSlot {
  __amdgpu_buffer_rsrc_t rs;
  int voff;
  int soff;
};
template <class E>
__device__ __forceinline__ void load_w(const float*, const WSlot& ws, float (&wk)[E::EPV]) {
#pragma unroll
  for (int q = 0; q < E::EPV / 4; ++q) {
    const f4 t = __builtin_bit_cast(
        f4, __builtin_amdgcn_raw_buffer_load_b128(ws.rs, ws.voff + 16 * q, ws.soff, 0));
    wk[4 * q + 0] = t[0];
    wk[4 * q + 1] = t[1];
    wk[4 * q + 2] = t[2];
    wk[4 * q + 3] = t[3];
  }
}

// Pass 1 over one vector: raw max and its first slot (argmax), online
// (max, sum exp) of the softcapped values, and the smoothing sum.
template <class E, int SC, int SM>
__device__ __forceinline__ void pass1_vec(const Params& p, Acc& a, const float (&f)[E::EPV],
                                          int slot, int64_t jg) {
  constexpr int EPV = E::EPV;
  float vm = f[0];
#pragma unroll
  for (int i = 1; i < EPV; ++i) vm = __builtin_fmaxf(vm, f[i]);
  // Slots may be visited out of index order (a wave reduction combines
  // them), so the tie-break compares indices. vm ignores NaN; a chunk
  // holding one is found by first_nan.
  const bool take = (vm > a.bv) || (vm == a.bv && slot < a.bi);
  a.bv = take ? vm : a.bv;
  a.bi = take ? slot : a.bi;

  float z[EPV];
  if constexpr (SC) {
    float u[EPV], t[EPV];
#pragma unroll
    for (int i = 0; i < EPV; ++i) u[i] = f[i] * p.inv_softcap;
    tanh_vec<EPV>(u, t);
#pragma unroll
    for (int i = 0; i < EPV; ++i) z[i] = p.softcap * t[i];
  } else {
#pragma unroll
    for (int i = 0; i < EPV; ++i) z[i] = f[i];
  }
  float zm = vm;
  if constexpr (SC) {
    zm = z[0];
#pragma unroll
    for (int i = 1; i < EPV; ++i) zm = __builtin_fmaxf(zm, z[i]);
  }
  const float mn = __builtin_fmaxf(a.m, zm);
  float e[EPV];
#pragma unroll
  for (int i = 0; i < EPV; ++i) e[i] = ex2((z[i] - mn) * kLog2e);
#pragma unroll
  for (int h = EPV / 2; h >= 1; h >>= 1) {
#pragma unroll
    for (int i = 0; i < h; ++i) e[i] += e[i + h];
  }
  a.s = a.s * ex2((a.m - mn) * kLog2e) + e[0];
  a.m = mn;
  if constexpr (SM) {
    if (p.weight) {
      float wk[EPV];
      load_w<E>(p.weight, jg, wk);
#pragma unroll
      for (int i = 0; i < EPV; ++i) a.sz = __builtin_fmaf(wk[i], z[i], a.sz);
    } else {
      float t = 0.0f;
#pragma unroll
      for (int i = 0; i < EPV; ++i) t += z[i];
      a.sz += t;
    }
  }
}

// Pass 1 over one scalar element (row tails and the unaligned path).
template <int SC, int SM>
__device__ __forceinline__ void pass1_one(const Params& p, Acc& a, float x, int slot, int64_t k) {
  arg_combine(a.bv, a.bi, x, slot);
  const float z = zval<SC>(p, x);
  const float mn = __builtin_fmaxf(a.m, z);
  a.s = a.s * ex2((a.m - mn) * kLog2e) + ex2((z - mn) * kLog2e);
  a.m = mn;
  if constexpr (SM) {
    a.sz = p.weight ? __builtin_fmaf(p.weight[k], z, a.sz) : a.sz + z;
  }
}

// Gradient of one element: ((p_k A - B w_k - C [k = y]) * dz/dx), with t the
// tanh of x / c (softcap only).
template <int SC, int SM>
__device__ __forceinline__ float grad_elem(const Params& p, const RowScalars& rs, float x, float t,
                                           float wk, bool is_y) {
  float z = x;
  if constexpr (SC) z = p.softcap * t;
  const float pk = ex2(__builtin_fmaf(z - rs.m, kLog2e, -rs.l2s));
  float g;
  if constexpr (SM) {
    g = __builtin_fmaf(pk, rs.A, -(rs.B * wk));
  } else {
    g = pk * rs.A;
  }
  g = is_y ? g - rs.C : g;
  if constexpr (SC) g = g * __builtin_fmaf(-t, t, 1.0f);
  return g;
}

template <int SC, int SM>
__device__ __forceinline__ float grad_one(const Params& p, const RowScalars& rs, float x, float wk,
                                          bool is_y) {
  const float t = SC ? tanh_f(x * p.inv_softcap) : 0.0f;
  return grad_elem<SC, SM>(p, rs, x, t, wk, is_y);
}

// FOLD (bf16 results without smoothing, where it is taken): A p_k as one
// exponential when A > 0.
// jg: the vector's index into the weights, or its WSlot.
template <class E, int SC, int SM, bool FOLD = false, class J = int64_t>
__device__ __forceinline__ u4 grad_vec(const Params& p, const RowScalars& rs, const u4 v,
                                       const J& jg, int yi) {
  constexpr int EPV = E::EPV;
  float f[EPV], wk[EPV];
  E::unpack(v, f);
  if constexpr (SM) {
    if (p.weight) {
      load_w<E>(p.weight, jg, wk);
    } else {
#pragma unroll
      for (int i = 0; i < EPV; ++i) wk[i] = 1.0f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPV; ++i) wk[i] = 1.0f;
  }
  float t[EPV];
  if constexpr (SC) {
    float u[EPV];
#pragma unroll
    for (int i = 0; i < EPV; ++i) u[i] = f[i] * p.inv_softcap;
    tanh_vec<EPV>(u, t);
  } else {
#pragma unroll
    for (int i = 0; i < EPV; ++i) t[i] = 0.0f;
  }
  float g[EPV];
  if constexpr (FOLD && E::EPV == 8 && !SM) {
    // bf16 result without smoothing: A p_k as one exponential, 2^(z log2 e +
    // cA), two operations fewer per element. Its relative error (about
    // |z| 2^-23) is far below the bf16 rounding that follows; fp32 results
    // keep the exact (z - m) form. (Taken by the row kernel: the split-row
    // kernel measured slower with it, its registers being fuller.)
    if (rs.cA == rs.cA && yi < 0) {  // uniform: A > 0
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        const float z = SC ? p.softcap * t[i] : f[i];
        g[i] = ex2(__builtin_fmaf(z, kLog2e, rs.cA));
        if constexpr (SC) g[i] = g[i] * __builtin_fmaf(-t[i], t[i], 1.0f);
      }
      return E::pack(g);
    }
  }
  if constexpr (E::EPV == 8 && SC) {
    // bf16 results with a softcap: the exponent as one fma with the cap
    // folded in, 2^(t (c log2 e) - (m log2 e + log2 s)), two operations fewer
    // per element than forming z, then z - m. Its relative error (about
    // |z| 2^-23) is far below the bf16 rounding that follows; the target's
    // element below keeps the exact form.
    const float c0 = __builtin_fmaf(-rs.m, kLog2e, -rs.l2s);
    const float cl = p.softcap * kLog2e;
#pragma unroll
    for (int i = 0; i < EPV; ++i) {
      const float pk = ex2(__builtin_fmaf(t[i], cl, c0));
      float gi;
      if constexpr (SM) {
        gi = __builtin_fmaf(pk, rs.A, -(rs.B * wk[i]));
      } else {
        gi = pk * rs.A;
      }
      g[i] = gi * __builtin_fmaf(-t[i], t[i], 1.0f);
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPV; ++i) g[i] = grad_elem<SC, SM>(p, rs, f[i], t[i], wk[i], false);
  }
  if (yi >= 0) {
    // The one element of the row at the target class: recompute it with the
    // one-hot term (same arithmetic as grad_one on that element).
#pragma unroll
    for (int i = 0; i < EPV; ++i)
      if (i == yi) g[i] = grad_elem<SC, SM>(p, rs, f[i], t[i], wk[i], true);
  }
  return E::pack(g);
}

// Combine the per-wave Acc records in wave order (fixed, deterministic).
template <int NW>
__device__ __forceinline__ Acc block_combine_p(const Acc* s) {
  Acc t = s[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    ms_combine(t.m, t.s, s[w].m, s[w].s);
    t.sz += s[w].sz;
    arg_combine(t.bv, t.bi, s[w].bv, s[w].bi);
  }
  return t;
}

template <int NW>
__device__ __forceinline__ Acc block_combine(const Acc (&s)[NW]) {
  Acc t = s[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    ms_combine(t.m, t.s, s[w].m, s[w].s);
    t.sz += s[w].sz;
    arg_combine(t.bv, t.bi, s[w].bv, s[w].bi);
  }
  return t;
}

// The mean's scales computed by the workgroup itself (self_scales):
// {D, alpha = 1/D, beta = 1/n}.
__shared__ double s_self_scales[3];

// Every workgroup of a fused launch with self_scales counts the counted rows
// n and D = sum of w[target] over them (the prologue's sums, in the same
// fixed order in every workgroup, so all get the same bits) and keeps the
// mean scales in LDS; workgroup 0 also stores D, n and the scales in the
// header for the epilogue (device-scope stores, complete before its arrival).
// UNROLL targets per thread are in flight at once: 16 where the kernel has
// registers to spare (the order of the sums does not depend on it).
template <int BLOCK, int UNROLL = 8>
__device__ __forceinline__ void compute_self_scales(const Params& p) {
  constexpr int NW = BLOCK / 64;
  constexpr int kU = UNROLL;
  __shared__ double s_D[NW];
  __shared__ int64_t s_n[NW];
  const int tid = threadIdx.x;
  double D = 0.0;
  int64_t n = 0;
  for (int64_t r0 = tid; r0 < p.rows; r0 += static_cast<int64_t>(BLOCK) * kU) {
    int64_t yv[kU];
    if constexpr (UNROLL > 8) {
      // one round of loads for 16 rows per thread (4096 rows on 256 threads
      // at once), indexes clamped instead of branched on; rows past the end
      // count as ignored
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t r = r0 + static_cast<int64_t>(u) * BLOCK;
        yv[u] = p.target[r < p.rows - 1 ? r : p.rows - 1];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t r = r0 + static_cast<int64_t>(u) * BLOCK;
        yv[u] = r < p.rows ? yv[u] : p.ignore_index;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t r = r0 + static_cast<int64_t>(u) * BLOCK;
        yv[u] = r < p.rows ? p.target[r] : p.ignore_index;
      }
    }
    float wv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool ok = yv[u] != p.ignore_index && yv[u] >= 0 && yv[u] < p.V;
      wv[u] = ok ? (p.weight ? p.weight[yv[u]] : 1.0f) : 0.0f;
      n += ok ? 1 : 0;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) D += static_cast<double>(wv[u]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    D += __shfl_xor(D, off, 64);
    n += __shfl_xor(n, off, 64);
  }
  if ((tid & 63) == 0) {
    s_D[tid >> 6] = D;
    s_n[tid >> 6] = n;
  }
  __syncthreads();
  if (tid == 0) {
    double tD = 0.0;
    int64_t tn = 0;
    for (int w = 0; w < NW; ++w) {
      tD += s_D[w];
      tn += s_n[w];
    }
    const double alpha = (tD != 0.0) ? static_cast<double>(static_cast<float>(1.0 / tD)) : 0.0;
    const double beta =
        (tn != 0) ? static_cast<double>(static_cast<float>(1.0 / static_cast<double>(tn))) : 0.0;
    s_self_scales[0] = tD;
    s_self_scales[1] = alpha;
    s_self_scales[2] = beta;
    if (blockIdx.x == 0) {
      __hip_atomic_store(&p.hdr->D, tD, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.hdr->n, tn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
}

// Scales of the row formulas: from the prologue when it ran (mean, weighted
// smoothing), from the workgroup's own count (self_scales), else the
// sum/none values alpha = beta = 1 and W = V.
__device__ __forceinline__ void load_scales(const Params& p, double& W, double& alpha,
                                            double& beta) {
  if (p.self_scales) {
    W = static_cast<double>(p.V);
    alpha = s_self_scales[1];
    beta = s_self_scales[2];
  } else if (p.has_hdr) {
    W = p.hdr->W;
    alpha = p.hdr->alpha;
    beta = p.hdr->beta;
  } else {
    W = static_cast<double>(p.V);
    alpha = 1.0;
    beta = 1.0;
  }
}

// Register slot k of a thread (k is a compile-time constant once the slot
// loops are unrolled; slots past NREG only appear in branches that are not
// taken).
template <int NREG>
__device__ __forceinline__ u4& slot(u4 (&r)[NREG], int k) {
  return r[k < NREG ? k : 0];
}

template <int EPV>
__device__ __forceinline__ float vec_max(const float (&f)[EPV]) {
  float m = f[0];
#pragma unroll
  for (int i = 1; i < EPV; ++i) m = __builtin_fmaxf(m, f[i]);
  return m;
}

// Gradient of one fp32 vector from its stored exponentials e = 2^((x - m_g) log2 e):
// p_k = e sc / A with sc = A 2^((m_g - m) log2 e - log2 s), so
// g = e sc - B w_k - C [k = y].
template <int SM, class J = int64_t>
__device__ __forceinline__ u4 grad_vec_e(const Params& p, const RowScalars& rs, const u4 v,
                                         float sc, const J& jg, int yi) {
  float e[4], g[4];
  F32::unpack(v, e);
  if constexpr (SM) {
    if (p.weight) {
      float wk[4];
      load_w<F32>(p.weight, jg, wk);
#pragma unroll
      for (int i = 0; i < 4; ++i) g[i] = __builtin_fmaf(e[i], sc, -(rs.B * wk[i]));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) g[i] = __builtin_fmaf(e[i], sc, -rs.B);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) g[i] = e[i] * sc;
  }
  if (yi >= 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i == yi) g[i] -= rs.C;
  }
  return F32::pack(g);
}

// Argmax of a row (or part) holding a NaN: the lowest element index holding
// a NaN, the order numpy and torch give argmax. Such a row's sum of
// exponentials is NaN (so is one holding +inf, which this finds no NaN in),
// so the search runs only then. Over a thread's slots k (vectors
// k * BLOCK + tid < nv, the first at element e0) and its row-tail element
// xt; REREAD: the slots hold exponentials, so the raw logits are loaded
// again (before any gradient store). Reduced over the wave; kNoIndex if none.
template <class E, int BLOCK, int NREG, bool REREAD>
__device__ __forceinline__ int first_nan(const u4 (&r)[NREG], __amdgpu_buffer_rsrc_t rsrc,
                                         int voff, int nv, int tid, int64_t e0, float xt,
                                         bool has_tail, int64_t tail_idx) {
  constexpr int EPV = E::EPV;
  // the row tail comes after every vector, so any vector NaN replaces it
  int nc = (has_tail && xt != xt) ? static_cast<int>(tail_idx) : kNoIndex;
  if constexpr (REREAD) {
    // one vector in flight at a time (a rolled loop): the slots stay live
    // for the gradient pass, so this path must not add registers
#pragma nounroll
    for (int k = NREG - 1; k >= 0; --k) {
      if (k * BLOCK < nv) {  // uniform
        const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, k * BLOCK * 16, 0);
        float f[EPV];
        E::unpack(v, f);
        const bool in = k * BLOCK + tid < nv;
#pragma unroll
        for (int i = EPV - 1; i >= 0; --i)
          nc = (in && f[i] != f[i])
                   ? static_cast<int>(e0 + static_cast<int64_t>(k * BLOCK + tid) * EPV + i)
                   : nc;
      }
    }
  } else {
#pragma unroll
    for (int k = NREG - 1; k >= 0; --k) {
      if (k * BLOCK < nv) {  // uniform
        float f[EPV];
        E::unpack(r[k], f);
        const bool in = k * BLOCK + tid < nv;
#pragma unroll
        for (int i = EPV - 1; i >= 0; --i)
          nc = (in && f[i] != f[i])
                   ? static_cast<int>(e0 + static_cast<int64_t>(k * BLOCK + tid) * EPV + i)
                   : nc;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) nc = min(nc, __shfl_xor(nc, off, 64));
  return nc;
}

// Outputs of a row that is ignored (gradient exactly +0.0, never read) or
// whose target is out of range (NaN loss).
template <class E, int BLOCK>
__device__ __forceinline__ void skipped_row(const Params& p, int64_t row, bool bad, char* rp,
                                            int nv, int tail) {
  const int tid = threadIdx.x;
  if (p.grad) {
    u4* vp = reinterpret_cast<u4*>(rp);
    for (int j = tid; j < nv; j += BLOCK) __builtin_nontemporal_store(u4{0u, 0u, 0u, 0u}, vp + j);
    if (tid < tail) E::st(rp, static_cast<int64_t>(nv) * E::EPV + tid, 0.0f);
  }
  if (tid == 0) {
    const float q = bad ? __builtin_nanf("") : 0.0f;
    write_row_outputs(p, row, q, q, 0, -1);
    write_row_stats(p, row, 0.0f, 0.0f);
    if (p.epilogue) publish_row(p, row, q, q, 0, 0);
  }
}

// Block-shared state of one row in flight.
template <int BLOCK>
struct RowShared {
  Acc acc[BLOCK / 64];
  int cand[BLOCK / 64];
  int nanc[BLOCK / 64];      // per wave: first NaN index (rows holding one)
  RowScalars rs;
  float xy;
  int64_t next_row, next_y;  // persistent kernel: the row claimed next and its target
};

// ---------------------------------------------------------------------------
// fused_row: one row in one workgroup; the row is read from HBM once and kept
// on chip. Slots: thread tid owns vectors j = k * BLOCK + tid, k < NREG, in
// VGPRs; the row tail (V % EPV elements) is held by threads tid < tail.
//
// Pass 1 takes the slots in groups of GS: first the group's raw maximum,
// then the exponentials relative to the group's softcapped maximum and their
// sum, folded into the thread's (max, sum) once per group. Each thread also
// keeps the first group that holds its raw maximum; once the row maximum is
// known, only threads holding it look for its first position (no
// per-element argmax work). Rows of fp32 logits without softcap keep the
// exponentials on chip in place of the logits, so the gradient pass is one
// multiply (or fma) per element by a per-group scale; other rows keep the
// logits and the gradient pass recomputes the exponential.
// ---------------------------------------------------------------------------
// Row claims of the persistent kernel: workgroup b starts with row b; once
// a row's pass 1 is done, thread 0 claims the next one (gridDim.x + the
// claim counter), so rows go to workgroups in the order they finish. Every
// row processed takes exactly one claim, so the claim that returns rows - 1
// is the launch's last: it resets the counter for the next launch.
struct RowClaim {
  uint32_t c;
  __device__ __forceinline__ void issue(const Params& p) {
    c = __hip_atomic_fetch_add(&p.hdr->next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Thread 0, once the claim has returned: the next row (>= rows: none), the
  // load of its target, and the counter reset by the last claim.
  __device__ __forceinline__ int64_t row(const Params& p) const {
    if (c == static_cast<uint32_t>(p.rows - 1))
      __hip_atomic_store(&p.hdr->next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return static_cast<int64_t>(gridDim.x) + c;
  }
};

template <class E, int BLOCK, int NREG, int SC, int SM, bool DYN>
__device__ __forceinline__ void fused_row(const Params& p, int64_t row, int64_t y,
                                          RowShared<BLOCK>& sh, uint32_t* arrival = nullptr,
                                          int64_t* pf_row = nullptr) {
  constexpr int EPV = E::EPV;
  // Claimed fp32 rows: PF slots of the next row are loaded into LDS while
  // this row's gradient is computed and stored (see before pass 2). (bf16
  // rows measured faster with it only when every launch starts from caches
  // flushed of the previous launch's writes, and slower back to back, so
  // they keep loading every slot from HBM.)
  constexpr int PF = (DYN && EPV == 4) ? 4 : 0;
  __shared__ u4 s_pfr[PF > 0 ? PF * BLOCK : 1];
  constexpr int NS = NREG;
  constexpr int NW = BLOCK / 64;
  constexpr bool KEEP_E = (EPV == 4) && !SC;
  constexpr int GS = (EPV == 4) ? 8 : 2;
  constexpr int NG = (NS + GS - 1) / GS;
  Acc* s_acc = sh.acc;
  int* s_cand = sh.cand;

  // Opaque per call: in the persistent loop, values derived from the thread
  // index and the row length are recomputed per row instead of being
  // hoisted out of the loop into registers (which would spill).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool ignored = (y == p.ignore_index);
  const bool bad = !ignored && (y < 0 || y >= p.V);
  char* rp = row_ptr(p, row, E::BYTES);
  int nv = __builtin_amdgcn_readfirstlane(static_cast<int>(p.V / EPV));
  asm volatile("" : "+s"(nv));
  const int tail = static_cast<int>(p.V - static_cast<int64_t>(nv) * EPV);
  const int64_t tail0 = static_cast<int64_t>(nv) * EPV;

  if (ignored || bad) {
    // Ignored rows are never read; their gradient is exactly +0.0
    // (tt-mlir PR #9324 page: ignored rows, also with non-finite logits).
    if constexpr (DYN) {
      // Every wave has read the previous row's next_row before it is
      // overwritten (this path has no other barrier before the write).
      __syncthreads();
      if (tid == 0) {
        RowClaim cl;
        cl.issue(p);
        const int64_t nr = cl.row(p);
        sh.next_row = nr;
        sh.next_y = nr < p.rows ? p.target[nr] : 0;
      }
      __syncthreads();
    }
    skipped_row<E, BLOCK>(p, row, bad, rp, nv, tail);
    return;
  }
  RowClaim claim;

  // ---- issue every load of the row up front ----
  // Raw buffer loads over a descriptor that spans exactly the row's vectors:
  // one VGPR offset for every slot (the slot offset is scalar) and hardware
  // bounds checking (lanes past the row read 0 and their stores are
  // dropped), so the loads are unconditional and the compiler waits, for
  // each slot, only for that slot's data. Order: the target logit and the
  // row tail, then the slots. The slot loads are non-temporal (each logit
  // is read once, and the class weights of weighted rows stay in L2).
  float xy = 0.0f;
  if (tid == 0) xy = E::ld(rp, y);
  float xt = 0.0f;
  if (tid < tail) xt = E::ld(rp, tail0 + tid);
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rp, nv);
  const int voff = tid * 16;
  // the class weights of the thread's vectors (weighted smoothing)
  const WSlot wsl = {make_rsrc_bytes(p.weight, static_cast<int>(p.V) * 4), tid * (EPV * 4), 0};
  u4 r[NREG];
  bool from_lds = false;
  if constexpr (PF > 0) from_lds = pf_row != nullptr && *pf_row == row;
  if (from_lds) {
    // The row's first PF slots are in LDS, each thread's own vectors (loaded
    // by its own lane). The row before stored at least 9 slots after issuing
    // them, so at most 8 operations of this wave in flight means they have
    // landed (without gradient stores: none in flight).
    if (p.grad) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt8);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NREG; ++k)
      r[k] = k < PF ? s_pfr[k * BLOCK + tid]
                    : __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, k * BLOCK * 16, kLoadNT);
  } else {
#pragma unroll
    for (int k = 0; k < NREG; ++k)
      r[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, k * BLOCK * 16, kLoadNT);
  }
  // ---- pass 1 ----
  // Thread state: (tm, ts) = max of z and sum of exp(z - tm), tsz = smoothing
  // sum, tb = raw maximum and tg = first group holding it (NG: the tail).
  float tm = kLowest, ts = 0.0f, tsz = 0.0f, tb = -__builtin_inff();
  int tg = -1;
  float gm[KEEP_E ? NG : 1];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g * GS * BLOCK < nv) {  // uniform: skip groups past the row
      float gx = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < GS; ++q) {
        const int k = g * GS + q;
        if (k < NS && k * BLOCK < nv) {
          float f[EPV];
          E::unpack(slot(r, k), f);
          if ((k + 1) * BLOCK > nv) {  // the row's last, partial slot (a scalar branch)
            asm volatile("");
            const bool ok = k * BLOCK + tid < nv;
#pragma unroll
            for (int i = 0; i < EPV; ++i) f[i] = ok ? f[i] : -__builtin_inff();
          }
#pragma unroll
          for (int i = 0; i < EPV; ++i) gx = __builtin_fmaxf(gx, f[i]);
        }
      }
      const bool take = gx > tb;  // strict: the first group holding the max stays
      tg = take ? g : tg;
      tb = take ? gx : tb;
      const float zg = zval<SC>(p, __builtin_fmaxf(gx, kLowest));
      // softcap rows: the exponent t (c log2 e) - zg log2 e as one fma
      const float zgl = zg * kLog2e;
      const float cl = p.softcap * kLog2e;
      float gsum = 0.0f;
#pragma unroll
      for (int q = 0; q < GS; ++q) {
        const int k = g * GS + q;
        if (k < NS && k * BLOCK < nv) {
          float f[EPV];
          E::unpack(slot(r, k), f);
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
          float e[EPV];
#pragma unroll
          for (int i = 0; i < EPV; ++i)
            e[i] = ex2(SC ? __builtin_fmaf(z[i], cl, -zgl) : (z[i] - zg) * kLog2e);
          if constexpr (KEEP_E) slot(r, k) = F32::pack(e);
          float es = e[0];
#pragma unroll
          for (int i = 1; i < EPV; ++i) es += e[i];
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
            asm volatile("");
            const bool ok = k * BLOCK + tid < nv;
            es = ok ? es : 0.0f;
            zs = ok ? zs : 0.0f;
          }
          gsum += es;
          if constexpr (SM) tsz += zs;
        }
      }
      ms_combine(tm, ts, zg, gsum);
      if constexpr (KEEP_E) gm[g] = zg;
    }
  }
  if (tid < tail) {
    // the row tail: one element per thread, after every vector in index order
    const bool take = xt > tb;
    tg = take ? NG : tg;
    tb = take ? xt : tb;
    const float z = zval<SC>(p, xt);
    ms_combine(tm, ts, z, 1.0f);
    if constexpr (SM) tsz = p.weight ? __builtin_fmaf(p.weight[tail0 + tid], z, tsz) : tsz + z;
  }

  // Claim the next row now that this one is almost done (claiming earlier
  // would hold rows back from workgroups that finish first); thread 0 reads
  // the claim back while it computes the row scalars.
  int64_t next_row = 0, next_y = 0;
  if (DYN && tid == 0) claim.issue(p);

  Acc a;
  a.m = tm;
  a.s = ts;
  a.sz = tsz;
  a.bv = tb;
  a.bi = 0;
  wave_reduce(a);
  if (lane == 0) s_acc[wave] = a;
  __syncthreads();
  const Acc t = block_combine_p<NW>(s_acc);

  // ---- argmax: threads holding the row maximum find its first position in
  // their first group holding it; the block takes the lowest index. With
  // exponentials kept on chip the maximum sits at e == 1 exactly, and for
  // 2 <= |max| < inf no other value can round to 1 (neighbouring floats
  // there differ by at least 2^-22); otherwise the group's raw logits are
  // read back (before any gradient store).
  int cand = kNoIndex;
  if (tg >= 0 && tb == t.bv) {
    if (tg == NG) {
      cand = static_cast<int>(tail0) + tid;
    } else {
      const bool by_e = !KEEP_E || (__builtin_fabsf(t.bv) >= 2.0f && t.bv < __builtin_inff());
      const float want = KEEP_E && by_e ? 1.0f : t.bv;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g == tg) {
#pragma unroll
          for (int q = GS - 1; q >= 0; --q) {
            const int k = g * GS + q;
            if (k < NS && k * BLOCK + tid < nv) {
              u4 v;
              if (KEEP_E && !by_e) {
                v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, k * BLOCK * 16, 0);
              } else {
                v = slot(r, k);
              }
              float f[EPV];
              E::unpack(v, f);
#pragma unroll
              for (int i = EPV - 1; i >= 0; --i)
                cand = (f[i] == want) ? (k * BLOCK + tid) * EPV + i : cand;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cand = min(cand, __shfl_xor(cand, off, 64));
  if (lane == 0) s_cand[wave] = cand;
  const bool row_nan = t.s != t.s;  // uniform: a NaN (or +inf) in the row
  if (row_nan) {
    const int nc = first_nan<E, BLOCK, NS, KEEP_E>(r, rsrc, voff, nv, tid, 0, xt, tid < tail,
                                                   tail0 + tid);
    if (lane == 0) sh.nanc[wave] = nc;
  }
  __syncthreads();

  if (tid == 0) {
    if constexpr (DYN) {
      next_row = claim.row(p);
      if (next_row < p.rows) next_y = p.target[next_row];
    }
    int arg = s_cand[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) arg = min(arg, s_cand[w]);
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
    sh.rs = rs;
    sh.xy = xy;
    if constexpr (DYN) {
      sh.next_row = next_row;
      sh.next_y = next_y;
    }
    write_row_outputs(p, row, rs.ce, rs.zl, rs.ok, arg);
    write_row_stats(p, row, rs.m, rs.l2s);
  }
  __syncthreads();
  if (tid == 0 && p.epilogue) {
    const RowScalars& rs = sh.rs;
    publish_row(p, row, rs.ce, rs.zl, rs.ok, 1);
    if constexpr (DYN) {
      // The workgroup's last row: it arrives once this row's values are
      // stored, and the arrival's round trip overlaps the gradient stores
      // below (the result is read after them). The address carries an
      // opaque per-lane zero, so the atomic stays a one-lane one whose
      // result is not waited for here.
      if (sh.next_row >= p.rows) {
        __builtin_amdgcn_s_waitcnt(0);
        int zero = 0;
        asm volatile("" : "+v"(zero));
        *arrival = __hip_atomic_fetch_add(&p.hdr->done + zero, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // The next row is claimed and its target known: the first PF slots of it
  // go to LDS now (buffer loads that write LDS directly, so no registers),
  // and HBM keeps reading while this row's gradient is computed and stored.
  // Counted rows only (an ignored row is never read), of more than 8 slots
  // (the wait above counts on at least 9 gradient stores after these loads).
  if constexpr (PF > 0) {
    if (pf_row != nullptr) {
      *pf_row = -1;
      const int64_t nrow = sh.next_row;
      const int64_t nyv = sh.next_y;
      if (nrow < p.rows && nyv != p.ignore_index && nyv >= 0 && nyv < p.V && nv > 8 * BLOCK) {
        const __amdgpu_buffer_rsrc_t rn = make_rsrc(row_ptr(p, nrow, E::BYTES), nv);
#pragma unroll
        for (int k = 0; k < PF; ++k)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rn, (__attribute__((address_space(3))) void*)(&s_pfr[k * BLOCK + wave * 64]), 16,
              voff, k * BLOCK * 16, 0, 0);
        *pf_row = nrow;
      }
    }
  }

  // ---- pass 2: gradient from on-chip data, written over the logits ----
  if (p.grad) {
    const RowScalars rs = sh.rs;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g * GS * BLOCK < nv) {
        float sc = 0.0f;
        if constexpr (KEEP_E) sc = rs.A * ex2(__builtin_fmaf(gm[g] - rs.m, kLog2e, -rs.l2s));
#pragma unroll
        for (int q = 0; q < GS; ++q) {
          const int k = g * GS + q;
          if (k < NS && k * BLOCK < nv) {
            const u4 v = slot(r, k);
            u4 gv;
            if constexpr (KEEP_E) {
              gv = grad_vec_e<SM>(p, rs, v, sc, WSlot{wsl.rs, wsl.voff, k * BLOCK * 16}, -1);
            } else {
              gv = grad_vec<E, SC, SM, true>(p, rs, v,
                                             WSlot{wsl.rs, wsl.voff, k * BLOCK * EPV * 4}, -1);
            }
            // lanes past the row are outside the descriptor: the store is dropped
            __builtin_amdgcn_raw_buffer_store_b128(gv, rsrc, voff, k * BLOCK * 16, kStoreNT);
          }
        }
      }
    }
    if (tid < tail) {
      const int64_t k = tail0 + tid;
      const float wk = (SM && p.weight) ? p.weight[k] : 1.0f;
      E::st(rp, k, grad_one<SC, SM>(p, rs, xt, wk, k == y));
    }
    // The one-hot term: the vectors above were written without it; the
    // thread that wrote the target's vector rewrites that one element (its
    // own later store to the same address, same path and policy, so it
    // lands last). No per-element test for the target in the loop above.
    if (y < tail0 && tid == static_cast<int>((y / EPV) % BLOCK)) {
      const float wy = (SM && p.weight) ? p.weight[y] : 1.0f;
      E::template st_buf<kStoreNT>(rsrc, static_cast<int>(y), grad_one<SC, SM>(p, rs, sh.xy, wy, true));
    }
  }
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32));
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<int>(v));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Persistent variant: gridDim.x resident workgroups. With 16 or more slots
// per thread (DYN: rows of 64 KiB and up) workgroups take rows in the order
// they finish (RowClaim; at 4096 x 32768 bf16 3 % faster than a fixed
// stride); for shorter rows workgroup b takes rows b, b + gridDim.x, ... (a
// claim's latency would be a large share of a short row), with the targets
// staged in LDS. Either way
// the loads of a workgroup's next row are issued as soon as the gradient
// stores of its current one are (they drain while the next row arrives).
// Each row's values for the epilogue are stored as the row completes; the
// workgroup arrives once, at its end.
constexpr int kRowsStaged = 256;
// bf16 rows of 256 x 16 slots: three workgroups per CU (at most 168 VGPRs);
// four (128 VGPRs) measured 2-3 % slower at 4096 x 32768 on MI355X.
template <class E, int BLOCK, int NREG, int SC, int SM>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(
    1, (E::EPV == 8 && BLOCK == 256 && NREG == 16) ? 3 : 8))) void rows_kernel(Params p) {
  constexpr bool DYN = NREG >= 16;
  __shared__ RowShared<BLOCK> sh;
  __shared__ int64_t s_y[DYN ? 1 : kRowsStaged];
  __shared__ int s_last;
  const int64_t G = gridDim.x;
  // self_scales: every workgroup counts n and D once, before its rows (kept
  // out of the row loop, whose registers it would otherwise crowd)
  if (p.self_scales) compute_self_scales<BLOCK, DYN ? 16 : 8>(p);
  // thread 0: the arrival count returned when the workgroup arrived with its
  // last row (claimed rows), else ~0
  uint32_t arrival = ~0u;
  int64_t pf_row = -1;  // the row whose first slots the LDS prefetch holds, or -1
  if constexpr (DYN) {
    int64_t row = blockIdx.x;
    int64_t y = p.target[row];
    while (true) {
      fused_row<E, BLOCK, NREG, SC, SM, true>(p, row, y, sh, &arrival, &pf_row);
      row = uniform_i64(sh.next_row);
      y = uniform_i64(sh.next_y);
      if (row >= p.rows) break;
    }
  } else {
    int64_t i = 0;
    for (int64_t row = blockIdx.x; row < p.rows; row += G, ++i) {
      const int q = static_cast<int>(i % kRowsStaged);
      if (q == 0) {
        __syncthreads();  // every thread is done with the previous batch
        for (int t = threadIdx.x; t < kRowsStaged; t += BLOCK) {
          const int64_t r = row + static_cast<int64_t>(t) * G;
          if (r < p.rows) s_y[t] = p.target[r];
        }
        __syncthreads();
      }
      fused_row<E, BLOCK, NREG, SC, SM, false>(p, row, uniform_i64(s_y[q]), sh);
    }
  }
  if (p.epilogue) {
    if (threadIdx.x == 0)
      s_last = arrival != ~0u ? arrival == static_cast<uint32_t>(G) - 1u
                              : arrive(p, static_cast<uint32_t>(G));
    __syncthreads();
    // 16 rows per thread in flight where the row loop's registers leave room
    // (4096 rows on 256 threads in one round of loads)
    if (s_last) epilogue_finish<BLOCK, DYN ? 16 : 8>(p);
  }
}

// ---------------------------------------------------------------------------
// Split-V stage 1: workgroup (row, c) reads chunk c of the row once and
// writes its partial (max, sum, smoothing sum, argmax, target logit). Slots
// as in fused_row, over the chunk's vectors.
// ---------------------------------------------------------------------------
template <class E, int BLOCK, int NREG, int SC, int SM>
__global__ __launch_bounds__(BLOCK) void splitv_partial_kernel(Params p) {
  constexpr int EPV = E::EPV;
  constexpr int NW = BLOCK / 64;
  __shared__ Acc s_acc[NW];
  __shared__ int s_arg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = blockIdx.x / p.S;
  const int c = blockIdx.x - static_cast<int>(row) * p.S;
  const int64_t y = p.target[row];
  const bool ignored = (y == p.ignore_index);
  const bool bad = !ignored && (y < 0 || y >= p.V);
  if (ignored || bad) return;  // stage 2 writes the outputs of skipped rows
  char* rp = row_ptr(p, row, E::BYTES);
  const int nvec_row = static_cast<int>(p.V / EPV);
  const int tail = static_cast<int>(p.V - static_cast<int64_t>(nvec_row) * EPV);
  const int v0 = c * p.chunk_vec;
  const int v1 = min(v0 + p.chunk_vec, nvec_row);
  const bool has_tail = (c == p.S - 1) && tail > 0;
  const int nv = v1 - v0;
  u4* vp = reinterpret_cast<u4*>(rp) + v0;
  const int64_t tail0 = static_cast<int64_t>(nvec_row) * EPV;

  const bool y_here = (y >= static_cast<int64_t>(v0) * EPV && y < static_cast<int64_t>(v1) * EPV) ||
                      (has_tail && y >= tail0);
  float xy = 0.0f;
  if (tid == 0 && y_here) xy = E::ld(rp, y);
  float xt = 0.0f;
  if (has_tail && tid < tail) xt = E::ld(rp, tail0 + tid);
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(vp, nv);
  const int voff = tid * 16;
  u4 r[NREG];
#pragma unroll
  for (int k = 0; k < NREG; ++k)
    r[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, k * BLOCK * 16, 0);

  Acc a;
  acc_init(a);
#pragma unroll
  for (int k = 0; k < NREG; ++k) {
    const int j = k * BLOCK + tid;
    if (k * BLOCK < nv && j < nv) {
      float f[EPV];
      E::unpack(r[k], f);
      pass1_vec<E, SC, SM>(p, a, f, v0 + j, static_cast<int64_t>(v0) + j);
    }
  }
  if (has_tail && tid < tail) pass1_one<SC, SM>(p, a, xt, nvec_row + tid, tail0 + tid);

  wave_reduce(a);
  if (lane == 0) s_acc[wave] = a;
  __syncthreads();
  const Acc t = block_combine<NW>(s_acc);

  // argmax: the owner of the winning slot finds the first position
  if (t.bi >= nvec_row) {
    if (tid == 0) s_arg = (t.bi == kNoIndex) ? 0 : static_cast<int>(tail0) + (t.bi - nvec_row);
  } else {
    const int jl = t.bi - v0;
    if (jl % BLOCK == tid) {
      const int kk = jl / BLOCK;
      int pos = 0;
#pragma unroll
      for (int k = 0; k < NREG; ++k) {
        if (k == kk) {
          float f[EPV];
          E::unpack(r[k], f);
#pragma unroll
          for (int i = EPV - 1; i >= 0; --i) pos = (f[i] == t.bv) ? i : pos;
        }
      }
      s_arg = t.bi * EPV + pos;
    }
  }
  // a chunk holding a NaN: its first NaN is the chunk's argmax
  __shared__ int s_nan[NW];
  const bool chunk_nan = t.s != t.s;  // uniform
  if (chunk_nan) {
    const int nc = first_nan<E, BLOCK, NREG, false>(r, rsrc, voff, nv, tid,
                                                    static_cast<int64_t>(v0) * EPV, xt,
                                                    has_tail && tid < tail, tail0 + tid);
    if (lane == 0) s_nan[wave] = nc;
  }
  __syncthreads();
  if (tid == 0) {
    Partial q;
    q.m = t.m;
    q.s = t.s;
    q.sz = t.sz;
    q.bv = t.bv;
    q.bi = s_arg;
    if (chunk_nan) {
      int na = kNoIndex;
      for (int w = 0; w < NW; ++w) na = min(na, s_nan[w]);
      if (na != kNoIndex) {
        q.bv = __builtin_nanf("");
        q.bi = na;
      }
    }
    q.xy = xy;
    q.has_y = y_here ? 1 : 0;
    q.pad = 0;
    p.part[row * p.S + c] = q;
  }
}

// ---------------------------------------------------------------------------
// Split-V stage 2: combine the S partials of the row (same order in every
// chunk's workgroup, so every chunk sees identical row scalars), then
// re-read this chunk and write its gradient.
// ---------------------------------------------------------------------------
template <class E, int BLOCK, int SC, int SM>
__global__ __launch_bounds__(BLOCK) void splitv_finish_kernel(Params p) {
  constexpr int EPV = E::EPV;
  constexpr int U = 4;
  __shared__ RowScalars s_rs;
  __shared__ float s_xy;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / p.S;
  const int c = blockIdx.x - static_cast<int>(row) * p.S;
  const int64_t y = p.target[row];
  const bool ignored = (y == p.ignore_index);
  const bool bad = !ignored && (y < 0 || y >= p.V);
  char* rp = row_ptr(p, row, E::BYTES);
  const int nvec_row = static_cast<int>(p.V / EPV);
  const int tail = static_cast<int>(p.V - static_cast<int64_t>(nvec_row) * EPV);
  const int v0 = c * p.chunk_vec;
  const int v1 = min(v0 + p.chunk_vec, nvec_row);
  const bool has_tail = (c == p.S - 1) && tail > 0;
  const int nv = v1 - v0;
  u4* vp = reinterpret_cast<u4*>(rp) + v0;
  const int64_t tail0 = static_cast<int64_t>(nvec_row) * EPV;

  if (ignored || bad) {
    if (p.grad) {
      for (int j = tid; j < nv; j += BLOCK) __builtin_nontemporal_store(u4{0u, 0u, 0u, 0u}, vp + j);
      if (has_tail && tid < tail) E::st(rp, tail0 + tid, 0.0f);
    }
    __shared__ int s_last0;
    if (tid == 0) {
      const float q = bad ? __builtin_nanf("") : 0.0f;
      if (c == 0) {
        write_row_outputs(p, row, q, q, 0, -1);
        write_row_stats(p, row, 0.0f, 0.0f);
      }
      if (p.epilogue) s_last0 = epilogue_publish(p, row, c == 0, q, q, 0, 0, gridDim.x);
    }
    if (p.epilogue) {
      __syncthreads();
      if (s_last0) epilogue_finish<BLOCK>(p);
    }
    return;
  }

  if (tid == 0) {
    const Partial* q = p.part + row * p.S;
    float m = q[0].m, s = q[0].s, sz = q[0].sz, bv = q[0].bv, xy = q[0].xy;
    int bi = q[0].bi;
    for (int i = 1; i < p.S; ++i) {
      ms_combine(m, s, q[i].m, q[i].s);
      sz += q[i].sz;
      arg_combine(bv, bi, q[i].bv, q[i].bi);
      if (q[i].has_y) xy = q[i].xy;
    }
    double W, alpha, beta;
    load_scales(p, W, alpha, beta);
    const float wy = p.weight ? p.weight[y] : 1.0f;
    RowScalars rs;
    row_scalars(rs, m, s, sz, zval<SC>(p, xy), wy, W, p, alpha, beta);
    rs.arg = bi;
    rs.ok = (bi == y);
    s_rs = rs;
    s_xy = xy;
    if (c == 0) {
      write_row_outputs(p, row, rs.ce, rs.zl, rs.ok, bi);
      write_row_stats(p, row, rs.m, rs.l2s);
    }
  }
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0 && p.epilogue) {
    const RowScalars& rs = s_rs;
    s_last = epilogue_publish(p, row, c == 0, rs.ce, rs.zl, rs.ok, 1, gridDim.x);
  }
  if (p.grad) {
    const RowScalars rs = s_rs;
    for (int j0 = 0; j0 < nv; j0 += BLOCK * U) {
      u4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * BLOCK + tid;
        v[u] = (j < nv) ? vp[j] : u4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * BLOCK + tid;
        if (j < nv) {
          const int64_t jg = static_cast<int64_t>(v0) + j;
          const u4 g = grad_vec<E, SC, SM>(p, rs, v[u], jg, -1);
          __builtin_nontemporal_store(g, vp + j);
        }
      }
    }
    if (has_tail && tid < tail) {
      const int64_t k = tail0 + tid;
      const float xk = E::ld(rp, k);
      const float wk = (SM && p.weight) ? p.weight[k] : 1.0f;
      E::st(rp, k, grad_one<SC, SM>(p, rs, xk, wk, k == y));
    }
    // The one-hot term, rewritten by the thread that stored the target's
    // vector (its own later store to the same address).
    const int64_t jy = y / EPV - v0;
    if (y < tail0 && jy >= 0 && jy < nv && tid == static_cast<int>(jy % BLOCK)) {
      const float wy = (SM && p.weight) ? p.weight[y] : 1.0f;
      E::st_nt(rp, y, grad_one<SC, SM>(p, rs, s_xy, wy, true));
    }
  }
  if (p.epilogue) {
    __syncthreads();
    if (s_last) epilogue_finish<BLOCK>(p);
  }
}

// ---------------------------------------------------------------------------
// Unaligned rows: one workgroup per row, element loads, two passes (the
// second re-reads the row).
// ---------------------------------------------------------------------------
template <class E, int BLOCK, int SC, int SM>
__global__ __launch_bounds__(BLOCK) void row_scalar_kernel(Params p) {
  constexpr int NW = BLOCK / 64;
  __shared__ Acc s_acc[NW];
  __shared__ RowScalars s_rs;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t y = p.target[row];
  const bool ignored = (y == p.ignore_index);
  const bool bad = !ignored && (y < 0 || y >= p.V);
  char* rp = row_ptr(p, row, E::BYTES);
  if (ignored || bad) {
    if (p.grad)
      for (int64_t k = tid; k < p.V; k += BLOCK) E::st(rp, k, 0.0f);
    __shared__ int s_last0;
    if (tid == 0) {
      const float q = bad ? __builtin_nanf("") : 0.0f;
      write_row_outputs(p, row, q, q, 0, -1);
      write_row_stats(p, row, 0.0f, 0.0f);
      if (p.epilogue) s_last0 = epilogue_publish(p, row, true, q, q, 0, 0, gridDim.x);
    }
    if (p.epilogue) {
      __syncthreads();
      if (s_last0) epilogue_finish<BLOCK>(p);
    }
    return;
  }
  Acc a;
  acc_init(a);
  for (int64_t k = tid; k < p.V; k += BLOCK) pass1_one<SC, SM>(p, a, E::ld(rp, k), static_cast<int>(k), k);
  wave_reduce(a);
  if (lane == 0) s_acc[wave] = a;
  __syncthreads();
  if (tid == 0) {
    const Acc t = block_combine<NW>(s_acc);
    double W, alpha, beta;
    load_scales(p, W, alpha, beta);
    const float wy = p.weight ? p.weight[y] : 1.0f;
    RowScalars rs;
    row_scalars(rs, t.m, t.s, t.sz, zval<SC>(p, E::ld(rp, y)), wy, W, p, alpha, beta);
    rs.arg = t.bi;
    rs.ok = (t.bi == y);
    s_rs = rs;
    write_row_outputs(p, row, rs.ce, rs.zl, rs.ok, t.bi);
    write_row_stats(p, row, rs.m, rs.l2s);
  }
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0 && p.epilogue) {
    const RowScalars& rs = s_rs;
    s_last = epilogue_publish(p, row, true, rs.ce, rs.zl, rs.ok, 1, gridDim.x);
  }
  if (p.grad) {
    const RowScalars rs = s_rs;
    for (int64_t k = tid; k < p.V; k += BLOCK) {
      const float wk = (SM && p.weight) ? p.weight[k] : 1.0f;
      E::st(rp, k, grad_one<SC, SM>(p, rs, E::ld(rp, k), wk, k == y));
    }
  }
  if (p.epilogue) {
    __syncthreads();
    if (s_last) epilogue_finish<BLOCK>(p);
  }
}

// ---------------------------------------------------------------------------
// Prologue (one workgroup): counted rows n, D = sum of w[target] over them,
// W = sum of w, the target-range error bit, the mean scales
// alpha = 1/D, beta = 1/n (0 when the denominator is 0: zero gradients for
// an all-ignored mean, tt-mlir PR #9324 page, Copilot comments on the mean
// reduction), and a reset arrival counter. Fixed-order sums: deterministic.
// ---------------------------------------------------------------------------
template <int kPrologueBlock>
__global__ __launch_bounds__(kPrologueBlock) void prologue_kernel(Params p) {
  constexpr int NW = kPrologueBlock / 64;
  __shared__ double s_D[NW], s_W[NW];
  __shared__ int64_t s_n[NW];
  __shared__ uint32_t s_e[NW];
  const int tid = threadIdx.x;
  double D = 0.0, W = 0.0;
  int64_t n = 0;
  uint32_t err = 0;
  // kU independent loads in flight per thread (one workgroup has to cover
  // every target and, with weighted smoothing, every class weight); the
  // sums still run in a fixed order.
  constexpr int kU = 8;
  for (int64_t r0 = tid; r0 < p.rows; r0 += static_cast<int64_t>(kPrologueBlock) * kU) {
    int64_t yv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t r = r0 + static_cast<int64_t>(u) * kPrologueBlock;
      yv[u] = r < p.rows ? p.target[r] : p.ignore_index;
    }
    float wv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool ok = yv[u] != p.ignore_index && yv[u] >= 0 && yv[u] < p.V;
      wv[u] = (ok && p.weight) ? p.weight[yv[u]] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (yv[u] != p.ignore_index) {
        if (yv[u] >= 0 && yv[u] < p.V) {
          n += 1;
          D += static_cast<double>(wv[u]);
        } else {
          err = 1u;
        }
      }
    }
  }
  if (p.weight) {
    const bool vec = (reinterpret_cast<uintptr_t>(p.weight) & 15) == 0;
    const int64_t nv4 = vec ? p.V / 4 : 0;
    const f4* w4 = reinterpret_cast<const f4*>(p.weight);
    for (int64_t j0 = tid; j0 < nv4; j0 += static_cast<int64_t>(kPrologueBlock) * kU) {
      f4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t j = j0 + static_cast<int64_t>(u) * kPrologueBlock;
        v[u] = j < nv4 ? w4[j] : f4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        W += static_cast<double>(v[u][0]);
        W += static_cast<double>(v[u][1]);
        W += static_cast<double>(v[u][2]);
        W += static_cast<double>(v[u][3]);
      }
    }
    for (int64_t k = nv4 * 4 + tid; k < p.V; k += kPrologueBlock) W += static_cast<double>(p.weight[k]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    D += __shfl_xor(D, off, 64);
    W += __shfl_xor(W, off, 64);
    n += __shfl_xor(n, off, 64);
    err |= __shfl_xor(err, off, 64);
  }
  if ((tid & 63) == 0) {
    s_D[tid >> 6] = D;
    s_W[tid >> 6] = W;
    s_n[tid >> 6] = n;
    s_e[tid >> 6] = err;
  }
  __syncthreads();
  if (tid == 0) {
    double tD = 0.0, tW = 0.0;
    int64_t tn = 0;
    uint32_t te = 0;
    for (int w = 0; w < NW; ++w) {
      tD += s_D[w];
      tW += s_W[w];
      tn += s_n[w];
      te |= s_e[w];
    }
    Header* h = p.hdr;
    h->D = tD;
    h->W = p.weight ? tW : static_cast<double>(p.V);
    h->n = tn;
    if (p.reduction == 1) {
      h->alpha = (tD != 0.0) ? static_cast<float>(1.0 / tD) : 0.0f;
      h->beta = (tn != 0) ? static_cast<float>(1.0 / static_cast<double>(tn)) : 0.0f;
    } else {
      h->alpha = 1.0f;
      h->beta = 1.0f;
    }
    h->err = te;
    h->done = 0u;
    if (p.rows == 0 && p.epilogue) {
      // No row blocks will run: the reductions of an empty batch.
      const double nan = __builtin_nan("");
      if (p.reduction == 1) {
        if (p.loss) p.loss[0] = static_cast<float>(nan);
        if (p.z_loss) p.z_loss[0] = static_cast<float>(nan);
      } else if (p.reduction == 2) {
        if (p.loss) p.loss[0] = 0.0f;
        if (p.z_loss) p.z_loss[0] = 0.0f;
      }
      if (p.reduction != 0 && p.acc) p.acc[0] = static_cast<float>(nan);
      if (p.counts) {
        p.counts[0] = 0;
        p.counts[1] = 0;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gradient recomputed from kept logits (the backward of a forward that did
// not overwrite them; PR #9324 page, the cross_entropy_bw composite takes
// the saved logits and target): grad = grad_output * d loss / d logits, from
// the logits, the target and the row's (m, log2 s) that the forward saved.
// Grid: rows x blocks_per_row, each block kBwdBlock x kBwdUnroll vectors (or
// elements) of its row. grad may be the logits themselves (same stride).
// ---------------------------------------------------------------------------
template <class E, int SC, int SM, bool VEC>
__global__ __launch_bounds__(kBwdBlock) void recompute_kernel(Params p, void* grad,
                                                              int64_t grad_stride, const float* go,
                                                              int per_row, int blocks_per_row) {
  constexpr int EPV = E::EPV;
  constexpr int U = kBwdUnroll;
  __shared__ RowScalars s_rs;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / blocks_per_row;
  const int b = blockIdx.x - static_cast<int>(row) * blocks_per_row;
  const int64_t y = p.target[row];
  const bool skip = (y == p.ignore_index) || y < 0 || y >= p.V;
  const char* xp = row_ptr(p, row, E::BYTES);
  char* gp = static_cast<char*>(grad) + row * grad_stride * E::BYTES;
  const float scale = per_row ? go[row] : go[0];
  // The block's logit loads go out first (they do not depend on the row
  // scalars), so their latency overlaps thread 0's read of the row's
  // statistics and the barrier.
  const int nvec = static_cast<int>(p.V / EPV);
  const u4* xv = reinterpret_cast<const u4*>(xp);
  const int j0 = b * kBwdBlock * U;
  const int64_t tail0 = static_cast<int64_t>(nvec) * EPV;
  // The owner of the target's vector reads the target logit before any
  // store (grad may be the logits).
  const int jy = static_cast<int>(y / EPV);
  const bool owns_y = VEC && !skip && y < tail0 && jy >= j0 && jy < j0 + kBwdBlock * U &&
                      (jy - j0) % kBwdBlock == tid;
  const float xy = owns_y ? E::ld(xp, y) : 0.0f;
  u4 v[U];
  if constexpr (VEC) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kBwdBlock + tid;
      v[u] = (!skip && j < nvec) ? __builtin_nontemporal_load(xv + j) : u4{0u, 0u, 0u, 0u};
    }
  }
  if (!skip && tid == 0) {
    double W, alpha, beta;
    load_scales(p, W, alpha, beta);
    const float wy = p.weight ? p.weight[y] : 1.0f;
    RowScalars rs;
    grad_scalars(rs, p.row_stats[2 * row], p.row_stats[2 * row + 1], wy, W, p, alpha, beta);
    s_rs = rs;
  }
  __syncthreads();
  const RowScalars rs = s_rs;
  if constexpr (VEC) {
    u4* gv = reinterpret_cast<u4*>(gp);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kBwdBlock + tid;
      if (j < nvec) {
        u4 g = u4{0u, 0u, 0u, 0u};
        if (!skip) {
          float f[EPV], wk[EPV], t[EPV], out[EPV];
          E::unpack(v[u], f);
#pragma unroll
          for (int i = 0; i < EPV; ++i) wk[i] = 1.0f;
          if (SM && p.weight) load_w<E>(p.weight, j, wk);
          if constexpr (SC) {
            float uu[EPV];
#pragma unroll
            for (int i = 0; i < EPV; ++i) uu[i] = f[i] * p.inv_softcap;
            tanh_vec<EPV>(uu, t);
          } else {
#pragma unroll
            for (int i = 0; i < EPV; ++i) t[i] = 0.0f;
          }
#pragma unroll
          for (int i = 0; i < EPV; ++i)
            out[i] = grad_elem<SC, SM>(p, rs, f[i], t[i], wk[i], false) * scale;
          g = E::pack(out);
        }
        __builtin_nontemporal_store(g, gv + j);
      }
    }
    if (b == blocks_per_row - 1 && tail0 + tid < p.V) {
      const int64_t k = tail0 + tid;
      float gk = 0.0f;
      if (!skip) {
        const float wk = (SM && p.weight) ? p.weight[k] : 1.0f;
        gk = grad_one<SC, SM>(p, rs, E::ld(xp, k), wk, k == y) * scale;
      }
      E::st_nt(gp, k, gk);
    }
    // The one-hot term, rewritten by the thread that stored the target's
    // vector (its own later store to the same address).
    if (owns_y) {
      const float wy = (SM && p.weight) ? p.weight[y] : 1.0f;
      E::st_nt(gp, y, grad_one<SC, SM>(p, rs, xy, wy, true) * scale);
    }
  } else {
    const int64_t span = static_cast<int64_t>(kBwdBlock) * U;
    const int64_t k0 = static_cast<int64_t>(b) * span;
    for (int64_t k = k0 + tid; k < p.V && k < k0 + span; k += kBwdBlock) {
      float gk = 0.0f;
      if (!skip) {
        const float wk = (SM && p.weight) ? p.weight[k] : 1.0f;
        gk = grad_one<SC, SM>(p, rs, E::ld(xp, k), wk, k == y) * scale;
      }
      E::st(gp, k, gk);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward: the stored gradient times grad_output, in place (Liger-Kernel CE
// profile, Backward Pass). Work units are (row, span of kBwdBlock x
// kBwdUnroll vectors); a bounded grid strides over them. A scalar
// grad_output of exactly 1 ends every block at once (the common
// loss.backward() call costs one small launch); with per-row scales a unit
// whose row scale is exactly 1 is skipped.
// ---------------------------------------------------------------------------
template <class E, bool VEC>
__global__ __launch_bounds__(kBwdBlock) void backward_kernel(void* grad, int64_t rows, int64_t V,
                                                             int64_t stride, const float* go,
                                                             int per_row, int blocks_per_row) {
  constexpr int EPV = E::EPV;
  if (!per_row && go[0] == 1.0f) return;
  const int64_t units = rows * blocks_per_row;
  const int tid = threadIdx.x;
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int64_t row = unit / blocks_per_row;
    const int b = static_cast<int>(unit - row * blocks_per_row);
    const float g = per_row ? go[row] : go[0];
    if (g == 1.0f) continue;
    char* rp = static_cast<char*>(grad) + row * stride * E::BYTES;
    if constexpr (VEC) {
      const int nvec = static_cast<int>(V / EPV);
      u4* vp = reinterpret_cast<u4*>(rp);
      const int j0 = b * kBwdBlock * kBwdUnroll;
      u4 v[kBwdUnroll];
#pragma unroll
      for (int u = 0; u < kBwdUnroll; ++u) {
        const int j = j0 + u * kBwdBlock + tid;
        v[u] = (j < nvec) ? vp[j] : u4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kBwdUnroll; ++u) {
        const int j = j0 + u * kBwdBlock + tid;
        if (j < nvec) {
          float f[EPV];
          E::unpack(v[u], f);
#pragma unroll
          for (int i = 0; i < EPV; ++i) f[i] *= g;
          __builtin_nontemporal_store(E::pack(f), vp + j);
        }
      }
      if (b == blocks_per_row - 1) {
        const int64_t tail0 = static_cast<int64_t>(nvec) * EPV;
        if (tail0 + tid < V) E::st(rp, tail0 + tid, E::ld(rp, tail0 + tid) * g);
      }
    } else {
      const int64_t span = static_cast<int64_t>(kBwdBlock) * kBwdUnroll;
      const int64_t k0 = static_cast<int64_t>(b) * span;
      for (int64_t k = k0 + tid; k < V && k < k0 + span; k += kBwdBlock)
        E::st(rp, k, E::ld(rp, k) * g);
    }
  }
}

}  // namespace cedev
