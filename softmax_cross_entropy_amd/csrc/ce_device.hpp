// Device-side building blocks for the fused softmax cross-entropy kernels
// (gfx950 / CDNA4, wave64).
//
// Everything here is per-element or per-row arithmetic shared by the kernel
// templates in ce_kernels.hpp. Numerics follow the Liger-Kernel page
// "Kernel Profile: CrossEntropy (Tier 3 - Fused/Complex)": fp32 for exp and
// log (Forward Pass, precision_sensitive_ops), a max-shifted log-sum-exp as
// the aten fallback lowering of tt-mlir PR #9339 (quoted on the PR #9324
// page) requires, and the loss/gradient components of its Key Patterns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cedev {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLowest = -3.402823466e+38f;  // -FLT_MAX: identity of the running max
constexpr int kNoIndex = 0x7fffffff;
constexpr int kPrologueBlock = 1024;  // threads of the single-workgroup prologue
constexpr int kBwdBlock = 256;        // backward: threads per block
constexpr int kBwdUnroll = 4;         // backward: vectors per thread
constexpr int kBwdMaxGrid = 4096;     // backward: blocks (grid-stride over the rest)

// ---------------------------------------------------------------------------
// Hardware transcendentals (v_exp_f32 = 2^x, v_log_f32 = log2 x, v_rcp_f32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ex2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float lg2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// tanh for the softcap z = c tanh(x / c). The softcapped value is scaled by c,
// so tanh needs a small *relative* error near 0 (where 1 - 2/(e^{2u}+1)
// cancels) as well as exact saturation:
//  * |u| < 0.55: u + u^3 Q(u^2), Q of degree 4, coefficients fitted here by
//    Lawson-weighted least squares to tanh(u)/u on [0, 0.55] (the polynomial
//    with these fp32 coefficients is within 3.5e-9 relative of tanh in exact
//    arithmetic; within 1e-7 relative once evaluated in fp32).
//  * |u| >= 0.55: sign(u) (1 - 2 / (e^{2|u|} + 1)) with one Newton step on the
//    reciprocal; |u| is clamped to 15, where tanh rounds to 1 in fp32 (a
//    NaN is not clamped: it reaches the exponential and stays NaN, as it
//    does on the polynomial branch).
constexpr float kTanhSplit = 0.55f;
constexpr float kTanhQ1 = -0.3333331048488617f;
constexpr float kTanhQ2 = 0.13332460820674896f;
constexpr float kTanhQ3 = -0.053842708468437195f;
constexpr float kTanhQ4 = 0.021039674058556557f;
constexpr float kTanhQ5 = -0.006235557142645121f;

__device__ __forceinline__ float tanh_poly(float u) {
  const float s = u * u;
  float q = kTanhQ5;
  q = __builtin_fmaf(q, s, kTanhQ4);
  q = __builtin_fmaf(q, s, kTanhQ3);
  q = __builtin_fmaf(q, s, kTanhQ2);
  q = __builtin_fmaf(q, s, kTanhQ1);
  return __builtin_fmaf(u * s, q, u);
}

__device__ __forceinline__ float tanh_exp(float u) {
  const float au = __builtin_fabsf(u);
  const float a = au > 15.0f ? 15.0f : au;  // false for NaN: NaN propagates
  const float d = ex2(a * (2.0f * kLog2e)) + 1.0f;
  float r = rcp(d);
  r = __builtin_fmaf(r, __builtin_fmaf(-d, r, 1.0f), r);
  return __builtin_copysignf(__builtin_fmaf(-2.0f, r, 1.0f), u);
}

__device__ __forceinline__ float tanh_f(float u) {
  return (__builtin_fabsf(u) < kTanhSplit) ? tanh_poly(u) : tanh_exp(u);
}

// Vector form: when no element of the vector in any lane of the wave reaches
// the split, every lane takes the polynomial alone (wave-uniform branch).
// Either way each element gets exactly tanh_f's value.
template <int N>
__device__ __forceinline__ void tanh_vec(const float (&u)[N], float (&t)[N]) {
  float amax = __builtin_fabsf(u[0]);
#pragma unroll
  for (int i = 1; i < N; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(u[i]));
  if (__ballot(!(amax < kTanhSplit)) != 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = tanh_f(u[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = tanh_poly(u[i]);
  }
}

// ---------------------------------------------------------------------------
// Storage types. A row is read and written as 16-byte vectors (dwordx4);
// elements are widened exactly to fp32 and bf16 results are rounded to
// nearest even (v_cvt_pk_bf16_f32).
// ---------------------------------------------------------------------------
struct F32 {
  static constexpr int EPV = 4;
  static constexpr int BYTES = 4;
  // Whole-vector reinterpretation only: this compiler mistranslates a bit
  // cast applied to one component of an ext_vector (it always reads .x).
  __device__ static __forceinline__ void unpack(const u4 v, float (&f)[4]) {
    const f4 t = __builtin_bit_cast(f4, v);
    f[0] = t[0];
    f[1] = t[1];
    f[2] = t[2];
    f[3] = t[3];
  }
  __device__ static __forceinline__ u4 pack(const float (&f)[4]) {
    const f4 t = {f[0], f[1], f[2], f[3]};
    return __builtin_bit_cast(u4, t);
  }
  __device__ static __forceinline__ float ld(const void* row, int64_t i) {
    return static_cast<const float*>(row)[i];
  }
  // The fp32 value of an element's bits (loaded early, widened where used).
  __device__ static __forceinline__ float widen(uint32_t r) { return __builtin_bit_cast(float, r); }
  // Element i (bits) through a buffer descriptor: 0 outside it.
  __device__ static __forceinline__ uint32_t ld_buf(__amdgpu_buffer_rsrc_t r, int i) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0);
  }
  __device__ static __forceinline__ void st(void* row, int64_t i, float v) {
    static_cast<float*>(row)[i] = v;
  }
  __device__ static __forceinline__ void st_nt(void* row, int64_t i, float v) {
    __builtin_nontemporal_store(v, static_cast<float*>(row) + i);
  }
  // Store element i through a buffer descriptor with cache policy AUX.
  template <int AUX>
  __device__ static __forceinline__ void st_buf(__amdgpu_buffer_rsrc_t r, int i, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, i * 4, 0, AUX);
  }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const b2 r = __builtin_convertvector((f2{lo, hi}), b2);
  return __builtin_bit_cast(uint32_t, r);
}

// One fp32 value rounded to bf16 (nearest even), as pack_bf16x2 rounds it.
__device__ __forceinline__ uint16_t to_bf16(float v) {
  return static_cast<uint16_t>(pack_bf16x2(v, 0.0f));
}

struct BF16 {
  static constexpr int EPV = 8;
  static constexpr int BYTES = 2;
  __device__ static __forceinline__ void unpack(const u4 v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      const uint32_t lo = w << 16, hi = w & 0xffff0000u;
      f[2 * i] = __builtin_bit_cast(float, lo);
      f[2 * i + 1] = __builtin_bit_cast(float, hi);
    }
  }
  __device__ static __forceinline__ u4 pack(const float (&f)[8]) {
    return u4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
              pack_bf16x2(f[6], f[7])};
  }
  __device__ static __forceinline__ float ld(const void* row, int64_t i) {
    const uint32_t h = static_cast<const uint16_t*>(row)[i];
    return __builtin_bit_cast(float, h << 16);
  }
  __device__ static __forceinline__ float widen(uint32_t r) {
    return __builtin_bit_cast(float, r << 16);
  }
  __device__ static __forceinline__ uint32_t ld_buf(__amdgpu_buffer_rsrc_t r, int i) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, i * 2, 0, 0);
  }
  __device__ static __forceinline__ void st(void* row, int64_t i, float v) {
    static_cast<uint16_t*>(row)[i] = static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
  __device__ static __forceinline__ void st_nt(void* row, int64_t i, float v) {
    __builtin_nontemporal_store(static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xffffu),
                                static_cast<uint16_t*>(row) + i);
  }
  template <int AUX>
  __device__ static __forceinline__ void st_buf(__amdgpu_buffer_rsrc_t r, int i, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(pack_bf16x2(v, 0.0f) & 0xffffu),
                                          r, i * 2, 0, AUX);
  }
};

// ---------------------------------------------------------------------------
// Launch-wide parameters (kernel argument, passed by value).
// ---------------------------------------------------------------------------
// First 256 bytes of the workspace. The fields the prologue writes (read by
// every row block) and the arrival counter (an atomic per row block) sit on
// different 128-byte lines, so the counter's traffic does not evict or
// serialize the reads of the scales.
struct Header {
  double D;              // sum of w[target] over counted rows
  double W;              // sum of all class weights (V when unweighted)
  int64_t n;             // counted rows
  float alpha;           // gradient scale of the cross-entropy part
  float beta;            // gradient scale of the z-loss part
  uint32_t err;          // bit 0: a target outside [0, V) that is not ignore_index
  uint32_t xerr_epoch;   // stamp of the last call in which a split row's exchange
                         // gave up waiting for a part (never reset: stamps are unique)
  uint32_t pad0[22];
  uint32_t done;         // arrival counter of the last-block epilogue (byte 128)
  uint32_t pad1[15];
  uint32_t next;         // row claims of the persistent row kernel (byte 192)
  uint32_t pad2[15];
};
static_assert(sizeof(Header) == 256, "the header fills the workspace's first 256 bytes");

struct Partial {         // one (row, chunk) of the split-V first stage: 32 bytes
  float m;               // running max of softcapped logits over the chunk
  float s;               // sum exp(z - m) over the chunk
  float sz;              // sum z (or sum w z) over the chunk
  float bv;              // largest raw logit in the chunk
  int32_t bi;            // lowest element index holding bv
  float xy;              // raw logit at the target (valid when has_y)
  int32_t has_y;
  int32_t pad;
};

struct Params {
  void* logits;
  int64_t rows, V, row_stride;         // row_stride in elements
  const int64_t* target;
  const float* weight;                 // (V) or null
  int64_t ignore_index;
  float eps, lam, softcap, inv_softcap;
  double one_minus_eps, eps_over_v, lam_d;  // host-computed row-invariant terms
  int reduction;                       // 0 none, 1 mean, 2 sum
  int grad;                            // write d loss / d logits in place
  int epilogue;                        // publish per-row values, run the last-block reduction
  int no_reduce;                       // epilogue: publish and arrive only (a later launch
                                       // reduces, e.g. over several row chunks)
  int self_scales;                     // mean without the prologue: every workgroup counts n
                                       // and D itself (workgroup 0 also fills the header)
  int has_hdr;                         // the prologue ran: scales, W and D are in hdr
  float* loss;
  float* z_loss;
  float* acc;
  int64_t* argmax;
  int64_t* counts;
  Header* hdr;
  float* row_ce;                       // (rows) cross-entropy term per row
  float* row_z;                        // (rows) z-loss term per row
  int32_t* row_ok;                     // (rows) bit 0: argmax == target, bit 1: counted
  float* row_stats;                    // (rows, 2) shift m and log2 s per row, or null
  Partial* part;                       // (rows, S) split-V partials; 128 bytes per row for row pairs
  uint32_t epoch;                      // unique per forward call: row-pair exchange stamp
  int spin_limit;                      // polls before a split row's exchange gives up (0: default)
  uint32_t xstamp;                     // unique per call (non-zero): stamped into hdr->xerr_epoch
                                       // when an exchange gives up, checked by the epilogue
  int S;                               // chunks per row (split-V)
  int chunk_vec;                       // vectors per chunk (split-V)
};

__device__ __forceinline__ char* row_ptr(const Params& p, int64_t row, int bytes) {
  return static_cast<char*>(p.logits) + row * p.row_stride * bytes;
}

// ---------------------------------------------------------------------------
// Online (max, sum) and argmax combination.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void ms_combine(float& m, float& s, float m2, float s2) {
  const float mn = __builtin_fmaxf(m, m2);
  s = s * ex2((m - mn) * kLog2e) + s2 * ex2((m2 - mn) * kLog2e);
  m = mn;
}

// Larger value wins, a NaN ranking above every number (the order numpy and
// torch give argmax); on equal values, or two NaNs, the lower index wins.
__device__ __forceinline__ void arg_combine(float& v, int& i, float v2, int i2) {
  const bool n1 = v != v, n2 = v2 != v2;
  const bool take = n2 ? (!n1 || i2 < i) : (!n1 && ((v2 > v) || (v2 == v && i2 < i)));
  v = take ? v2 : v;
  i = take ? i2 : i;
}

struct Acc {
  float m, s, sz;  // running max of z, sum exp(z - m), sum z or sum w z
  float bv;        // largest raw logit seen
  int bi;          // vector (or element) index where bv was first seen
};

__device__ __forceinline__ void acc_init(Acc& a) {
  a.m = kLowest;
  a.s = 0.0f;
  a.sz = 0.0f;
  a.bv = -__builtin_inff();
  a.bi = kNoIndex;
}

// Wave64 reduction of Acc (butterfly over all 64 lanes; result in every lane).
__device__ __forceinline__ void wave_reduce(Acc& a) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(a.m, off, 64);
    const float s2 = __shfl_xor(a.s, off, 64);
    const float z2 = __shfl_xor(a.sz, off, 64);
    const float v2 = __shfl_xor(a.bv, off, 64);
    const int i2 = __shfl_xor(a.bi, off, 64);
    ms_combine(a.m, a.s, m2, s2);
    a.sz += z2;
    arg_combine(a.bv, a.bi, v2, i2);
  }
}

// Per-row scalars that drive the loss and the gradient.
struct RowScalars {
  float m;      // shift (max of softcapped logits)
  float l2s;    // log2 of the shifted sum
  float A;      // coefficient of p_k
  float B;      // constant term (times w_k when weighted smoothing)
  float C;      // extra term subtracted at the target class
  float cA;     // log2 A - m log2 e - log2 s when A > 0, else NaN: A p_k as the single
                // exponential 2^(z_k log2 e + cA) (bf16 gradients without smoothing)
  float ce;     // cross-entropy + smoothing loss of the row
  float zl;     // z-loss of the row
  int arg;      // argmax element index
  int ok;       // argmax == target
};

// Loss and gradient coefficients of one counted row, from the reduced
// (m, s, sum z) and the raw target logit. With z = softcapped logits,
// lse = m + ln s, eps = label smoothing, w = class weights, W = sum w:
//   l    = w_y (1 - eps) (lse - z_y) + (eps / V) (W lse - sum_k w_k z_k)
//   zeta = lam lse^2
//   dL/dz_k = alpha [w_y (1 - eps)(p_k - [k = y]) + (eps / V)(W p_k - w_k)]
//             + beta 2 lam lse p_k
// (Liger-Kernel CE profile, Key Patterns: cross entropy, label smoothing and
// z-loss each contribute to loss and gradient; PyTorch's convention for how
// smoothing mass and class weights combine.)
// The gradient coefficients A, B, C of a row from its shift m and the log2 of
// its shifted sum; returns lse. Shared by the forward (row_scalars) and the
// gradient recomputed from kept logits, so both use identical coefficients.
__device__ __forceinline__ double grad_scalars(RowScalars& r, float m, float l2s, float wy,
                                               double W, const Params& p, double alpha,
                                               double beta) {
  const double lns = static_cast<double>(l2s) * static_cast<double>(kLn2);
  const double lse = static_cast<double>(m) + lns;
  const double wyd = wy;
  const double ome = p.one_minus_eps, epv = p.eps_over_v, lam = p.lam_d;
  r.m = m;
  r.l2s = l2s;
  const double A = alpha * (wyd * ome + epv * W) + beta * 2.0 * lam * lse;
  r.A = static_cast<float>(A);
  r.B = static_cast<float>(alpha * epv);
  r.C = static_cast<float>(alpha * wyd * ome);
  // (the hardware log2: a double-precision one is a library call, which this
  // code keeps out of the kernels)
  r.cA = A > 0.0 ? static_cast<float>(static_cast<double>(lg2(static_cast<float>(A))) -
                                      static_cast<double>(m) * 1.4426950408889634 -
                                      static_cast<double>(l2s))
                 : __builtin_nanf("");
  return lse;
}

__device__ __forceinline__ void row_scalars(RowScalars& r, float m, float s, float sz, float zy,
                                            float wy, double W, const Params& p, double alpha,
                                            double beta) {
  const float l2s = lg2(s);
  const double lse = grad_scalars(r, m, l2s, wy, W, p, alpha, beta);
  const double lns = static_cast<double>(l2s) * static_cast<double>(kLn2);
  const double wyd = wy;
  const double ce = wyd * p.one_minus_eps * ((static_cast<double>(m) - zy) + lns) +
                    p.eps_over_v * (W * lse - static_cast<double>(sz));
  r.ce = static_cast<float>(ce);
  r.zl = static_cast<float>(p.lam_d * lse * lse);
}

// ---------------------------------------------------------------------------
// Last-block epilogue: every participating block publishes its per-row
// values and bumps an arrival counter; the block that arrives last reduces
// the per-row arrays in a fixed order (bitwise deterministic) in fp64.
// Reductions: Liger-Kernel CE profile, forward_outputs (scalar loss, or per
// row for "none"); the PR #9324 page's fallback lowering (none returns rows,
// sum and mean reduce); IEEE 0/0 = NaN keeps the all-ignored mean NaN.
//
// Publication without an L2 write-back: the per-row values are written with
// device-scope atomic stores (they write through the per-XCD L2 to the
// device-coherent level), the writer waits for those stores to complete
// (s_waitcnt 0) before its arrival atomic, and the last block reads them
// back with device-scope atomic loads. An agent-scope release fence would
// instead write back the whole L2 of the XCD once per block. The single
// publishing thread does this right after the row scalars are known, so
// the wait covers only its loads and these three stores (not the row's
// gradient stores) and the other waves go on with the gradient meanwhile.
// ---------------------------------------------------------------------------

// The row's values for the epilogue (device-scope atomic stores, no wait).
__device__ __forceinline__ void publish_row(const Params& p, int64_t row, float ce, float zl,
                                            int ok, int counted) {
  __hip_atomic_store(p.row_ce + row, ce, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p.row_z + row, zl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p.row_ok + row, (ok ? 1 : 0) | (counted ? 2 : 0), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// The calling thread's stores are complete, then it bumps the arrival
// counter. Returns true in the block that arrives last of total_blocks.
__device__ __forceinline__ bool arrive(const Params& p, uint32_t total_blocks) {
  __builtin_amdgcn_s_waitcnt(0);
  const uint32_t prev =
      __hip_atomic_fetch_add(&p.hdr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return prev == total_blocks - 1u;
}

// One thread per block. has_row: the block owns the row's values (a split-V
// row is owned by its chunk 0). Returns true in the block that arrives last.
__device__ __forceinline__ bool epilogue_publish(const Params& p, int64_t row, bool has_row,
                                                 float ce, float zl, int ok, int counted,
                                                 uint32_t total_blocks) {
  if (has_row) publish_row(p, row, ce, zl, ok, counted);
  return arrive(p, total_blocks);
}

// Whole block, in the block that arrived last only. UNROLL: rows per thread
// in flight (the VGPRs this takes are the kernel's peak in the lighter
// kernels, so it is 8 unless a kernel has registers to spare).
template <int BLOCK, int UNROLL = 8>
__device__ __forceinline__ void epilogue_reduce(const Params& p) {
  __shared__ double s_red[2][BLOCK / 64];
  __shared__ int64_t s_cnt[2][BLOCK / 64];
  const int tid = threadIdx.x;
  // Every load here is device-coherent and takes a full memory latency at
  // the end of a launch, when the last gradient stores are draining: thread
  // 0 issues its two header words together with its first rows, and each
  // thread has UNROLL rows in flight at once, with indexes clamped into the
  // arrays so no load sits behind a per-lane branch. The sums still run in
  // row order and skip the rows past the end, so the result does not depend
  // on UNROLL.
  uint32_t xe = 0u;
  double D_hdr = 0.0;
  if (tid == 0) {
    if (p.xstamp != 0u)
      xe = __hip_atomic_load(&p.hdr->xerr_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.has_hdr || p.self_scales)
      D_hdr = __hip_atomic_load(&p.hdr->D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  double ce = 0.0, zl = 0.0;
  int64_t ok = 0, cnt = 0;
  constexpr int kEpiUnroll = UNROLL;
  constexpr int64_t kRound = static_cast<int64_t>(BLOCK) * kEpiUnroll;
  for (int64_t rb = 0; rb < p.rows; rb += kRound) {
    // a uniform base per round and one 32-bit index per row, shared by the
    // three arrays (a scalar base plus a vector offset per load)
    const int nr = static_cast<int>(p.rows - rb < kRound ? p.rows - rb : kRound);
    const float* bce = p.row_ce + rb;
    const float* bz = p.row_z + rb;
    const int32_t* bok = p.row_ok + rb;
    float vce[kEpiUnroll], vz[kEpiUnroll];
    int32_t vf[kEpiUnroll];
#pragma unroll
    for (int u = 0; u < kEpiUnroll; ++u) {
      const int i = tid + u * BLOCK;
      const uint32_t ic = static_cast<uint32_t>(i < nr ? i : nr - 1);
      vce[u] = __hip_atomic_load(bce + ic, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      vz[u] = __hip_atomic_load(bz + ic, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      vf[u] = __hip_atomic_load(bok + ic, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < kEpiUnroll; ++u) {
      const bool in = tid + u * BLOCK < nr;
      ce = in ? ce + static_cast<double>(vce[u]) : ce;
      zl = in ? zl + static_cast<double>(vz[u]) : zl;
      ok += in ? (vf[u] & 1) : 0;
      cnt += in ? ((vf[u] >> 1) & 1) : 0;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ce += __shfl_xor(ce, off, 64);
    zl += __shfl_xor(zl, off, 64);
    ok += __shfl_xor(ok, off, 64);
    cnt += __shfl_xor(cnt, off, 64);
  }
  const int lane = tid & 63, wv = tid >> 6;
  if (lane == 0) {
    s_red[0][wv] = ce;
    s_red[1][wv] = zl;
    s_cnt[0][wv] = ok;
    s_cnt[1][wv] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    double tce = 0.0, tz = 0.0;
    int64_t nc = 0, ncount = 0;
    for (int w = 0; w < BLOCK / 64; ++w) {
      tce += s_red[0][w];
      tz += s_red[1][w];
      nc += s_cnt[0][w];
      ncount += s_cnt[1][w];
    }
    // A split row whose exchange gave up in this call poisons the reduced
    // outputs (its own values are NaN already when its part 0 gave up).
    const bool xfail = p.xstamp != 0u && xe == p.xstamp;
    if (xfail) tce = tz = __builtin_nan("");
    const double n = static_cast<double>(ncount);
    const double D = (p.has_hdr || p.self_scales) ? D_hdr : n;
    if (p.reduction == 1) {
      if (p.loss) p.loss[0] = static_cast<float>(tce / D + tz / n);
      if (p.z_loss) p.z_loss[0] = static_cast<float>(tz / n);
    } else if (p.reduction == 2) {
      if (p.loss) p.loss[0] = static_cast<float>(tce + tz);
      if (p.z_loss) p.z_loss[0] = static_cast<float>(tz);
    }
    if (p.reduction != 0 && p.acc)
      p.acc[0] = xfail ? __builtin_nanf("") : static_cast<float>(static_cast<double>(nc) / n);
    if (p.counts) {
      p.counts[0] = ncount;
      p.counts[1] = nc;
    }
    p.hdr->done = 0u;
  }
}

// The last block's work: the reduction, or with no_reduce only the reset of
// the arrival counter (the per-row values stay for a later reduction).
template <int BLOCK, int UNROLL = 8>
__device__ __forceinline__ void epilogue_finish(const Params& p) {
  if (p.no_reduce) {
    if (threadIdx.x == 0) p.hdr->done = 0u;
  } else {
    epilogue_reduce<BLOCK, UNROLL>(p);
  }
}

// Per-row outputs of one row (thread 0 of the row's block); the reduced
// outputs go through epilogue_publish.
// The row's (m, log2 s), kept for a later gradient recomputed from the logits.
__device__ __forceinline__ void write_row_stats(const Params& p, int64_t row, float m, float l2s) {
  if (p.row_stats) {
    p.row_stats[2 * row] = m;
    p.row_stats[2 * row + 1] = l2s;
  }
}

__device__ __forceinline__ void write_row_outputs(const Params& p, int64_t row, float ce, float zl,
                                                  int ok, int64_t arg) {
  if (p.reduction == 0) {
    if (p.loss) p.loss[row] = ce + zl;
    if (p.z_loss) p.z_loss[row] = zl;
    if (p.acc) p.acc[row] = ok ? 1.0f : 0.0f;
  }
  if (p.argmax) p.argmax[row] = arg;
}

}  // namespace cedev
