// Wide row kernel: rows of up to 16 K 16-byte vectors (256 KiB) per
// workgroup of 1024 threads, or rows of up to 32 K vectors (512 KiB) split
// into two halves held by a pair of workgroups. Each workgroup reads its
// part of the row from HBM once, keeps it in VGPRs (NREG vectors per thread)
// and writes the gradient over it.
//
// Same method as fused_row (Liger-Kernel page "Kernel Profile: CrossEntropy
// (Tier 3 - Fused/Complex)", Key Patterns: online softmax pass, then the
// gradient written in place of the logits), laid out for the largest rows:
//  * 16 waves per CU with 16 dwordx4 loads in flight per wave. On MI355X the
//    in-place read-then-write of a 1023 x 128256 fp32 batch runs at about
//    5.9 TB/s in this layout (a half row per CU) against 5.2 TB/s with
//    8 waves of 63 loads holding a whole row per CU (VGPRs + LDS).
//  * A row of two halves: each workgroup reduces its half to a partial
//    (max, sum, smoothing sum, argmax), publishes it, and takes the other
//    half's partial; both combine the two in the same order (half 0 first),
//    so both get bitwise identical row scalars. Pairs are fixed: workgroups
//    2j and 2j + 1 take the two halves of one row after another, so a
//    workgroup only ever waits for its neighbour, which the hardware starts
//    right after it. Pair j starts with row j; the even workgroup claims the
//    pair's next row when it starts a row and hands it over with its
//    partial.
//  * Pass 1 works in groups of 4 slots (fp32; 2 for bf16) with one shift per
//    group; rows of fp32 logits without softcap keep exp(z - group shift)
//    in place of the logits, so the gradient pass is one multiply per
//    element.
#pragma once

#include "ce_kernels.hpp"

namespace cedev {

constexpr int kWideBlock = 1024;
constexpr int kWideSlots = 16;  // VGPR slots per thread of the largest wide shapes
// Polls of the partner's words before a pair gives up and flags the row
// (each poll is one device-coherent load, about a microsecond); a partner
// that never arrives would otherwise hold the workgroup forever. After one
// such failure the workgroup polls once per row: the error bit is set and
// the launch ends in bounded time.
constexpr int kPairSpinLimit = 1 << 22;

// Row-pair exchange through the row's two 64-byte slots (one per half).
// Words 0-4 are a half's partial (max, sum, smoothing sum, largest raw
// logit, its index); words 5-7, written by half 0 only, are the pair's next
// row and that row's target (low, high). Each word travels as a 64-bit
// atomic store of (word, epoch), where the epoch is a number the host makes
// unique per call: a reader that sees this call's epoch in a pair has that
// pair's word, with no wait between data and flag on the writer's side.
// Nothing has to be reset between calls: a slot left by an earlier call
// carries an older epoch.
constexpr int kPairWords = 5;
constexpr int kSlotWords = 8;

// Thread 0: publishes words [A, B) of `mine`, then polls words [C, D) of
// the partner's slot until all carry this call's epoch; returns false if
// the partner did not publish within `limit` polls.
template <int A, int B, int C, int D>
__device__ __forceinline__ bool pair_exchange(const Params& p, int64_t row, int h,
                                              const uint32_t (&mine)[kSlotWords],
                                              uint32_t (&other)[kSlotWords], int limit) {
  uint64_t* slot = reinterpret_cast<uint64_t*>(p.part + row * 4);  // 2 x 64 bytes
  const uint64_t ep = static_cast<uint64_t>(p.epoch) << 32;
#pragma unroll
  for (int i = A; i < B; ++i)
    __hip_atomic_store(slot + kSlotWords * h + i, ep | mine[i], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if constexpr (C == D) return true;
  const uint64_t* osrc = slot + kSlotWords * (1 - h);
  int it = 0;
  while (true) {
    bool all = true;
#pragma unroll
    for (int i = C; i < D; ++i) {
      const uint64_t v = __hip_atomic_load(osrc + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      other[i] = static_cast<uint32_t>(v);
      all = all && (static_cast<uint32_t>(v >> 32) == p.epoch);
    }
    if (all) return true;
    if (++it >= limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Block-shared state of the part in flight.
struct WideShared {
  Acc acc[kWideBlock / 64];
  int cand[kWideBlock / 64];
  RowScalars rs;
  float xy;
  int64_t next_t, next_y;  // the part (whole rows) or row (pairs) next, and its target
  int limit;               // poll limit of the pair exchange (thread 0 only)
};

// Whole-row parts are claimed: workgroup b starts with part b; thread 0
// claims the next one (gridDim.x + the claim counter) once the current
// part's pass 1 is done, so parts go to workgroups in the order they finish.
// Every part processed takes exactly one claim, so the claim that returns
// parts - 1 is the launch's last and resets the counter for the next launch.
// Half rows are not claimed one by one (a workgroup that claimed before
// waiting for its partner could be handed that partner's half and wait on
// itself): half 0 of a fixed pair claims whole rows (pairs + the counter)
// when it starts a row, so it holds its next row before it can wait; the
// launch makes one claim per row, and the claim that returns rows - 1
// resets the counter.
__device__ __forceinline__ uint32_t claim_issue(const Params& p) {
  return __hip_atomic_fetch_add(&p.hdr->next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same for a claim issued before the part's loads: the address carries
// an opaque per-lane zero, so the compiler keeps it a one-lane atomic instead
// of a wave-wide one whose result it would wait for (and with it for every
// store still in flight) right after issuing it.
__device__ __forceinline__ uint32_t claim_issue_early(const Params& p) {
  int zero = 0;
  asm volatile("" : "+v"(zero));
  return __hip_atomic_fetch_add(&p.hdr->next + zero, 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
template <int HALVES>
__device__ __forceinline__ void claim_finish(const Params& p, uint32_t c, WideShared& sh) {
  const int64_t parts = p.rows * HALVES;
  if (c == static_cast<uint32_t>(parts - 1))
    __hip_atomic_store(&p.hdr->next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int64_t nt = static_cast<int64_t>(gridDim.x) + c;
  sh.next_t = nt;
  sh.next_y = nt < parts ? p.target[nt / HALVES] : 0;
}

// Half 0 of a pair (thread 0): the row a claim `c` stands for (issued when
// the current row started, so its target is read while the row is in
// flight); the launch's last claim resets the counter.
__device__ __forceinline__ int64_t pair_row(const Params& p, uint32_t c) {
  return static_cast<int64_t>(gridDim.x >> 1) + c;
}
__device__ __forceinline__ int64_t pair_target(const Params& p, uint32_t c) {
  const int64_t nr = pair_row(p, c);
  return nr < p.rows ? p.target[nr] : 0;
}
__device__ __forceinline__ void pair_reset(const Params& p, uint32_t c) {
  if (c == static_cast<uint32_t>(p.rows - 1))
    __hip_atomic_store(&p.hdr->next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0: the pair's next row and its target into the block-shared state
// (half 1 takes them from half 0's words 5-7; if they never came, the
// workgroup stops).
__device__ __forceinline__ void pair_next(const Params& p, int h, bool ok, uint32_t c,
                                          int64_t ny, const uint32_t (&other)[kSlotWords],
                                          WideShared& sh) {
  if (h == 0) {
    sh.next_t = pair_row(p, c);
    sh.next_y = ny;
  } else {
    sh.next_t = ok ? static_cast<int64_t>(other[5]) : p.rows;
    sh.next_y = static_cast<int64_t>((static_cast<uint64_t>(other[7]) << 32) | other[6]);
  }
  if (!ok) {
    atomicOr(&p.hdr->err, 2u);
    sh.limit = 1;
  }
}

// Half 0's words 5-7: the pair's next row and its target.
__device__ __forceinline__ void next_words(const Params& p, uint32_t c, int64_t ny,
                                           uint32_t (&w)[kSlotWords]) {
  w[5] = static_cast<uint32_t>(pair_row(p, c));
  w[6] = static_cast<uint32_t>(ny);
  w[7] = static_cast<uint32_t>(static_cast<uint64_t>(ny) >> 32);
}

// One part (a whole row, or half of one) of the persistent wide kernel.
template <class E, int NREG, int HALVES, int SC, int SM>
__device__ __forceinline__ void wide_part(const Params& p, int64_t t, int64_t y,
                                          WideShared& sh, int64_t& next_t, int64_t& next_y) {
  constexpr int BLOCK = kWideBlock;
  constexpr int NW = BLOCK / 64;
  constexpr int EPV = E::EPV;
  constexpr int GS = (EPV == 4) ? 4 : 2;  // slots per pass-1 group
  constexpr int NG = NREG / GS;
  constexpr bool KEEP_E = (EPV == 4) && !SC;
  Acc* s_acc = sh.acc;
  int* s_cand = sh.cand;

  const int64_t row = t / HALVES;
  const int h = HALVES == 1 ? 0 : static_cast<int>(t % HALVES);
  // Opaque per part: values derived from the thread index are recomputed per
  // part instead of being kept live across the loop.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool ignored = (y == p.ignore_index);
  const bool bad = !ignored && (y < 0 || y >= p.V);
  char* rp = row_ptr(p, row, E::BYTES);
  const int nv_row = static_cast<int>(p.V / EPV);
  const int half = (nv_row + HALVES - 1) / HALVES;
  const int v0 = h * half;
  const int nv = max(0, min(half, nv_row - v0));  // vectors of this part
  const bool last = (h == HALVES - 1);
  const int tail = last ? static_cast<int>(p.V - static_cast<int64_t>(nv_row) * EPV) : 0;
  const int64_t tail0 = static_cast<int64_t>(nv_row) * EPV;
  char* hp = rp + static_cast<int64_t>(v0) * 16;  // this part's first vector
  const int64_t e0 = static_cast<int64_t>(v0) * EPV;  // its first element

  if (ignored || bad) {
    // Ignored rows are never read; their gradient is exactly +0.0
    // (tt-mlir PR #9324 page: ignored rows, also with non-finite logits).
    if constexpr (HALVES == 1) {
      __syncthreads();  // every thread has read the previous part's next_t
      if (tid == 0) claim_finish<HALVES>(p, claim_issue(p), sh);
      __syncthreads();
      next_t = uniform_i64(sh.next_t);
      next_y = uniform_i64(sh.next_y);
    }
    uint32_t claim = 0;
    if constexpr (HALVES == 2) {
      if (tid == 0 && h == 0) claim = claim_issue(p);
    }
    if (p.grad) {
      u4* vp = reinterpret_cast<u4*>(hp);
      for (int j = tid; j < nv; j += BLOCK) __builtin_nontemporal_store(u4{0u, 0u, 0u, 0u}, vp + j);
      if (tid < tail) E::st(rp, tail0 + tid, 0.0f);
    }
    if constexpr (HALVES == 2) {
      // no partials to combine: half 0 only hands over the pair's next row
      __syncthreads();  // every thread has read the previous part's next_t
      if (tid == 0) {
        uint32_t mine_w[kSlotWords] = {}, other_w[kSlotWords] = {};
        bool ok = true;
        int64_t ny = 0;
        if (h == 0) {
          pair_reset(p, claim);
          ny = pair_target(p, claim);
          next_words(p, claim, ny, mine_w);
          pair_exchange<5, kSlotWords, 0, 0>(p, row, h, mine_w, other_w, sh.limit);
        } else {
          ok = pair_exchange<0, 0, 5, kSlotWords>(p, row, h, mine_w, other_w, sh.limit);
        }
        pair_next(p, h, ok, claim, ny, other_w, sh);
      }
      __syncthreads();
      next_t = uniform_i64(sh.next_t);
      next_y = uniform_i64(sh.next_y);
    }
    if (tid == 0 && h == 0) {
      const float q = bad ? __builtin_nanf("") : 0.0f;
      write_row_outputs(p, row, q, q, 0, -1);
      write_row_stats(p, row, 0.0f, 0.0f);
      if (p.epilogue) publish_row(p, row, q, q, 0, 0);
    }
  } else {
    // ---- every load of this part, issued up front ----
    // Non-temporal buffer loads (each logit is read once) over a descriptor
    // spanning exactly the part's vectors: lanes past it read 0 and their
    // stores are dropped. Both halves read the target logit before either
    // can write a gradient (each writes only after both have published).
    // Half 0 of a pair claims the pair's next row before its loads go out.
    uint32_t claim = 0;
    if constexpr (HALVES == 2) {
      if (tid == 0 && h == 0) claim = claim_issue_early(p);
    }
    // The target logit and the row tail as stored, read by every lane of wave
    // 0 (the waves that use them) through a descriptor over the row's V
    // elements (lanes past the tail read 0), and widened where used: a load
    // in a per-lane branch, or a bf16 widening right here, would make the
    // wave wait for the previous row's stores before its own loads go out.
    // The other waves' value is an opaque zero, so the compiler cannot fold
    // the widening into the branch.
    uint32_t xy_raw = opaque_zero(), xt_raw = xy_raw;
    if (wave == 0) {
      const __amdgpu_buffer_rsrc_t rrow = make_rsrc_bytes(rp, static_cast<int>(p.V) * E::BYTES);
      xy_raw = E::ld_buf(rrow, static_cast<int>(y));
      xt_raw = E::ld_buf(rrow, static_cast<int>(tail0) + tid);
    }
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(hp, nv);
    const int voff = tid * 16;
    u4 r[NREG];
#pragma unroll
    for (int k = 0; k < NREG; ++k)
      r[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, k * BLOCK * 16, kLoadNT);
    int64_t ny = 0;  // target of the pair's next row (half 0, thread 0)
    if constexpr (HALVES == 2) {
      if (tid == 0 && h == 0) ny = pair_target(p, claim);
    }

    // ---- pass 1, group by group in load order ----
    // (tm, ts): max of z and sum of exp(z - tm); tsz: smoothing sum;
    // tb / tg: the thread's raw maximum and the first group holding it
    // (NG: the row tail).
    float tm = kLowest, ts = 0.0f, tsz = 0.0f, tb = -__builtin_inff();
    int tg = -1;
    float gm[KEEP_E ? NG : 1];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g * GS * BLOCK < nv) {  // uniform: groups past the part are skipped
        float gx = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < GS; ++q) {
          const int k = g * GS + q;
          if (k * BLOCK < nv) {
            float f[EPV];
            E::unpack(r[k], f);
            if ((k + 1) * BLOCK > nv) {  // the part's last, partial slot
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
        float gsum = 0.0f;
#pragma unroll
        for (int q = 0; q < GS; ++q) {
          const int k = g * GS + q;
          if (k * BLOCK < nv) {
            float f[EPV];
            E::unpack(r[k], f);
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
            float e[EPV];
#pragma unroll
            for (int i = 0; i < EPV; ++i) e[i] = ex2((z[i] - zg) * kLog2e);
            if constexpr (KEEP_E) r[k] = F32::pack(e);
            float es = e[0];
#pragma unroll
            for (int i = 1; i < EPV; ++i) es += e[i];
            float zs = 0.0f;
            if constexpr (SM) {
              if (p.weight) {
                float wk[EPV];
                load_w<E>(p.weight, v0 + k * BLOCK + tid, wk);
#pragma unroll
                for (int i = 0; i < EPV; ++i) zs = __builtin_fmaf(wk[i], z[i], zs);
              } else {
#pragma unroll
                for (int i = 0; i < EPV; ++i) zs += z[i];
              }
            }
            if ((k + 1) * BLOCK > nv) {  // lanes past the part add nothing
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
    const float xt = E::widen(xt_raw);
    if (tid < tail) {
      // the row tail (last part): one element per thread, after every vector
      const bool take = xt > tb;
      tg = take ? NG : tg;
      tb = take ? xt : tb;
      const float z = zval<SC>(p, xt);
      ms_combine(tm, ts, z, 1.0f);
      if constexpr (SM) tsz = p.weight ? __builtin_fmaf(p.weight[tail0 + tid], z, tsz) : tsz + z;
    }

    // Every load of the part has been consumed by pass 1 (a part holds data
    // in each group it reads); saying so with an explicit wait keeps the
    // compiler from guarding later writes of those registers with a wait
    // for every store in flight (it cannot see that a skipped group's load
    // is skipped too).
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    Acc a;
    a.m = tm;
    a.s = ts;
    a.sz = tsz;
    a.bv = tb;
    a.bi = 0;
    wave_reduce(a);
    if (lane == 0) s_acc[wave] = a;
    __syncthreads();
    // Every thread needs only the part's largest raw logit here; thread 0
    // combines the full records (in wave order) below.
    float bmax = s_acc[0].bv;
#pragma unroll
    for (int w = 1; w < NW; ++w) bmax = __builtin_fmaxf(bmax, s_acc[w].bv);

    // ---- argmax: threads holding the part's maximum look for its first
    // position in their first group holding it; the block takes the lowest
    // index. With exponentials kept on chip the maximum sits at e == 1
    // exactly, and for 2 <= |max| < inf no other value can round to 1
    // (neighbouring floats there differ by at least 2^-22); otherwise the
    // group's raw logits are read back (before any gradient store).
    int cand = kNoIndex;
    const bool mine = tg >= 0 && tb == bmax;
    if (mine && tg == NG) cand = static_cast<int>(tail0) + tid;
    const bool by_e = !KEEP_E || (__builtin_fabsf(bmax) >= 2.0f && bmax < __builtin_inff());
    const float want = KEEP_E && by_e ? 1.0f : bmax;
    if (__ballot(mine && tg < NG) != 0) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const bool here = mine && tg == g;
        if (__ballot(here) != 0) {
#pragma unroll
          for (int q = GS - 1; q >= 0; --q) {
            const int k = g * GS + q;
            if (k * BLOCK < nv) {
              u4 v;
              if (KEEP_E && !by_e) {  // uniform: the raw logits, read back from HBM
                v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, k * BLOCK * 16, 0);
              } else {
                v = r[k];
              }
              float f[EPV];
              E::unpack(v, f);
              const bool in = here && k * BLOCK + tid < nv;
#pragma unroll
              for (int i = EPV - 1; i >= 0; --i)
                cand = (in && f[i] == want) ? static_cast<int>(e0) + (k * BLOCK + tid) * EPV + i
                                            : cand;
            }
          }
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cand = min(cand, __shfl_xor(cand, off, 64));
    if (lane == 0) s_cand[wave] = cand;
    __syncthreads();

    if (wave == 0) {
      // Wave 0 combines the NW wave records with a fixed butterfly (lane l
      // holds wave l's record; the same tree every time, so bitwise
      // deterministic); lane 0 then owns the part's totals.
      Acc t;
      int arg = kNoIndex;
      if (lane < NW) {
        t = s_acc[lane];
        arg = s_cand[lane];
      } else {
        acc_init(t);
      }
#pragma unroll
      for (int off = NW / 2; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(t.m, off, 64);
        const float s2 = __shfl_xor(t.s, off, 64);
        const float z2 = __shfl_xor(t.sz, off, 64);
        ms_combine(t.m, t.s, m2, s2);
        t.sz += z2;
        arg = min(arg, __shfl_xor(arg, off, 64));
      }
      t.bv = bmax;
      t.bi = arg;
      if (lane == 0) {
        if constexpr (HALVES == 1) claim = claim_issue(p);
        if constexpr (HALVES == 2) {
          // Exchange partials with the other half (half 0 adds the pair's
          // next row); both combine half 0 first.
          uint32_t mine_w[kSlotWords] = {
              __builtin_bit_cast(uint32_t, t.m), __builtin_bit_cast(uint32_t, t.s),
              __builtin_bit_cast(uint32_t, t.sz), __builtin_bit_cast(uint32_t, t.bv),
              static_cast<uint32_t>(t.bi), 0u, 0u, 0u};
          uint32_t other_w[kSlotWords] = {};
          bool ok;
          if (h == 0) {
            pair_reset(p, claim);
            next_words(p, claim, ny, mine_w);
            ok = pair_exchange<0, kSlotWords, 0, kPairWords>(p, row, h, mine_w, other_w,
                                                             sh.limit);
          } else {
            ok = pair_exchange<0, kPairWords, 0, kSlotWords>(p, row, h, mine_w, other_w,
                                                             sh.limit);
          }
          pair_next(p, h, ok, claim, ny, other_w, sh);
          const uint32_t* q0 = h == 0 ? mine_w : other_w;
          const uint32_t* q1 = h == 0 ? other_w : mine_w;
          float m = __builtin_bit_cast(float, q0[0]), sum = __builtin_bit_cast(float, q0[1]);
          ms_combine(m, sum, __builtin_bit_cast(float, q1[0]), __builtin_bit_cast(float, q1[1]));
          t.m = m;
          t.s = sum;
          t.sz = __builtin_bit_cast(float, q0[2]) + __builtin_bit_cast(float, q1[2]);
          const float bv0 = __builtin_bit_cast(float, q0[3]);
          const float bv1 = __builtin_bit_cast(float, q1[3]);
          const bool take1 = bv1 > bv0;  // ties keep half 0 (the lower indices)
          t.bv = take1 ? bv1 : bv0;
          t.bi = static_cast<int>(take1 ? q1[4] : q0[4]);
        }
        if (t.bi == kNoIndex) t.bi = 0;  // no finite or infinite value: index 0
        double W, alpha, beta;
        load_scales(p, W, alpha, beta);
        const float wy = p.weight ? p.weight[y] : 1.0f;
        RowScalars rs;
        row_scalars(rs, t.m, t.s, t.sz, zval<SC>(p, E::widen(xy_raw)), wy, W, p, alpha, beta);
        rs.arg = t.bi;
        rs.ok = (t.bi == y);
        sh.rs = rs;
        sh.xy = E::widen(xy_raw);
        if constexpr (HALVES == 1) claim_finish<HALVES>(p, claim, sh);
        if (h == 0) {
          write_row_outputs(p, row, rs.ce, rs.zl, rs.ok, t.bi);
          write_row_stats(p, row, rs.m, rs.l2s);
          if (p.epilogue) publish_row(p, row, rs.ce, rs.zl, rs.ok, 1);
        }
      }
    }
    __syncthreads();
    // The next part, read here rather than after the gradient stores: an LDS
    // read behind them made the compiler wait for every store to complete
    // before the next part's loads could go out.
    next_t = uniform_i64(sh.next_t);
    next_y = uniform_i64(sh.next_y);

    // ---- pass 2: the gradient from on-chip data, written over the logits ----
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
            if (k * BLOCK < nv) {
              u4 gv;
              if constexpr (KEEP_E) {
                gv = grad_vec_e<SM>(p, rs, r[k], sc, v0 + k * BLOCK + tid, -1);
              } else {
                gv = grad_vec<E, SC, SM>(p, rs, r[k], v0 + k * BLOCK + tid, -1);
              }
              // lanes past the part are outside the descriptor: the store is dropped
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
      // own later store to the same address, same path and policy).
      const int64_t yl = y - e0;  // target position within this part
      if (yl >= 0 && yl < static_cast<int64_t>(nv) * EPV &&
          tid == static_cast<int>((yl / EPV) % BLOCK)) {
        const float wy = (SM && p.weight) ? p.weight[y] : 1.0f;
        E::template st_buf<kStoreNT>(rsrc, static_cast<int>(yl),
                                     grad_one<SC, SM>(p, rs, sh.xy, wy, true));
      }
    }
  }
}

// Persistent: as many workgroups as fit on the device at once (at most one
// per part; an even number for half rows); each processes parts until the
// claims run out, then arrives once at the epilogue. The next part's loads
// are issued as soon as the current part's gradient stores are (they drain
// while the next part arrives).
template <class E, int NREG, int HALVES, int SC, int SM>
__global__ __launch_bounds__(kWideBlock) void wide_kernel(Params p) {
  static_assert(HALVES == 1 || HALVES == 2, "whole rows or half rows");
  __shared__ WideShared sh;
  __shared__ int s_last;
  // self_scales: every workgroup counts n and D once, before its parts
  // (kept out of the part loop, whose registers it would otherwise crowd)
  if (p.self_scales) compute_self_scales<kWideBlock>(p);
  if (threadIdx.x == 0) sh.limit = kPairSpinLimit;
  if constexpr (HALVES == 2) {
    // pair j = workgroups 2j, 2j + 1 starts with row j (the grid holds at
    // most one pair per row)
    const int h = blockIdx.x & 1;
    int64_t row = blockIdx.x >> 1;
    int64_t y = p.target[row];
    while (row < p.rows) {
      int64_t nr, ny;
      wide_part<E, NREG, HALVES, SC, SM>(p, 2 * row + h, y, sh, nr, ny);
      row = nr;
      y = ny;
    }
  } else {
    const int64_t parts = p.rows;
    int64_t t = blockIdx.x;
    int64_t y = p.target[t];
    while (t < parts) {
      int64_t nt, ny;
      wide_part<E, NREG, HALVES, SC, SM>(p, t, y, sh, nt, ny);
      t = nt;
      y = ny;
    }
  }
  if (p.epilogue) {
    if (threadIdx.x == 0) s_last = arrive(p, gridDim.x);
    __syncthreads();
    if (s_last) epilogue_finish<kWideBlock>(p);
  }
}

}  // namespace cedev
