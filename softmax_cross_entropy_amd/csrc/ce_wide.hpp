// Wide row kernel: rows of up to 16 K 16-byte vectors (256 KiB) per
// workgroup of 1024 threads, or rows of up to 32 K vectors (512 KiB) split
// into G parts held by a group of workgroups: four quarters on 512-thread
// workgroups (two per CU), or two halves on 512- or 1024-thread ones. Each
// workgroup reads its part of the row from HBM once, keeps it in VGPRs
// (NREG vectors per thread) and writes the gradient over it.
//
// Same method as fused_row (Liger-Kernel page "Kernel Profile: CrossEntropy
// (Tier 3 - Fused/Complex)", Key Patterns: online softmax pass, then the
// gradient written in place of the logits), laid out for the largest rows:
//  * 16 waves per CU with 16 dwordx4 loads in flight per wave. On MI355X the
//    in-place read-then-write of a 1023 x 128256 fp32 batch runs at about
//    5.9 TB/s with a half row per CU against 5.2 TB/s with 8 waves holding a
//    whole row per CU (VGPRs + LDS); with quarter rows, two workgroups per
//    CU, one streams while the other waits for its group.
//  * A split row: each workgroup reduces its part to a partial (max, sum,
//    smoothing sum, argmax), publishes it, and folds the G partials in part
//    order (part 0 first), so all get bitwise identical row scalars. Groups
//    are fixed: workgroups G j ... G j + G - 1 take the parts of one row
//    after another, so a workgroup only ever waits for its neighbours, which
//    the hardware starts right after it. Group j starts with row j; part 0
//    claims the group's next row when it starts a row and hands it over with
//    its partial.
//  * Pass 1 works in groups of 4 slots (fp32; 2 for bf16) with one shift per
//    group; rows of fp32 logits without softcap keep exp(z - group shift)
//    in place of the logits, so the gradient pass is one multiply per
//    element.
#pragma once

#include "ce_kernels.hpp"

namespace cedev {

// Polls of the other parts' words before a group gives up (each poll is one
// device-coherent load, about a microsecond); a part that never arrives
// would otherwise hold the workgroup forever. A part that gives up on a
// row's partials poisons what it writes of that row: NaN gradient over its
// part, and, in part 0, NaN over the rest of the row and NaN per-row loss
// and z-loss with argmax -1; it stamps the call's epoch into the header
// (hdr->xerr_epoch = xstamp), which turns the reduced outputs NaN and makes
// CE_F_CHECK_TARGETS report CE_E_EXCHANGE. After one such failure the
// workgroup polls once per row, so the launch ends in bounded time. Parts
// other than 0 still wait the full limit for part 0's words 5-7 (their
// next row), so they go on writing their part of every later row.
constexpr int kGroupSpinLimit = 1 << 22;

// Exchange within a row's group of G parts (a pair, or four quarters)
// through the row's G 64-byte slots, one per part. Words 0-4 are a part's
// partial (max, sum, smoothing sum, largest raw logit, its index); words
// 5-7, written by part 0 only, are the group's next row and that row's
// target (low, high). Each word travels as a 64-bit atomic store of
// (word, epoch), where the epoch is a number the host makes unique per call:
// a reader that sees this call's epoch in a pair has that pair's word, with
// no wait between data and flag on the writer's side. Nothing has to be
// reset between calls: a slot left by an earlier call carries an older
// epoch.
constexpr int kPartialWords = 5;
constexpr int kSlotWords = 8;

template <int G>
__device__ __forceinline__ uint64_t* row_slots(const Params& p, int64_t row) {
  return reinterpret_cast<uint64_t*>(p.part) + row * (G * kSlotWords);
}

// Thread 0: words [a, b) of `w` into a slot.
__device__ __forceinline__ void slot_publish(const Params& p, uint64_t* slot,
                                             const uint32_t (&w)[kSlotWords], int a, int b) {
  const uint64_t ep = static_cast<uint64_t>(p.epoch) << 32;
#pragma unroll
  for (int i = 0; i < kSlotWords; ++i)
    if (i >= a && i < b)
      __hip_atomic_store(slot + i, ep | w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0: polls words [a, b) of a slot until all carry this call's epoch;
// false if they did not within `limit` polls.
__device__ __forceinline__ bool slot_poll(const Params& p, const uint64_t* slot,
                                          uint32_t (&w)[kSlotWords], int a, int b, int limit) {
  int it = 0;
  while (true) {
    bool all = true;
#pragma unroll
    for (int i = 0; i < kSlotWords; ++i) {
      if (i >= a && i < b) {
        const uint64_t v = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w[i] = static_cast<uint32_t>(v);
        all = all && (static_cast<uint32_t>(v >> 32) == p.epoch);
      }
    }
    if (all) return true;
    if (++it >= limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Block-shared state of the part in flight.
template <int BLOCK>
struct WideShared {
  Acc acc[BLOCK / 64];
  int cand[BLOCK / 64];
  int nanc[BLOCK / 64];    // per wave: first NaN index (parts holding one)
  RowScalars rs;
  float xy;
  int64_t next_t, next_y;  // the part (whole rows) or row (split rows) next, and its target
  int limit;               // poll limit of the group exchange (thread 0 only)
};

// Whole-row parts are claimed: workgroup b starts with part b; thread 0
// claims the next one (gridDim.x + the claim counter) once the current
// part's pass 1 is done, so parts go to workgroups in the order they finish.
// Every part processed takes exactly one claim, so the claim that returns
// parts - 1 is the launch's last and resets the counter for the next launch.
// Parts of a split row are not claimed one by one (a workgroup that claimed
// before waiting for its partners could be handed a partner's part and wait
// on itself): part 0 of a fixed group claims whole rows (groups + the
// counter) when it starts a row, so it holds its next row before it can
// wait; the launch makes one claim per row, and the claim that returns
// rows - 1 resets the counter.
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
template <int PARTS, class SH>
__device__ __forceinline__ void claim_finish(const Params& p, uint32_t c, SH& sh) {
  const int64_t parts = p.rows * PARTS;
  if (c == static_cast<uint32_t>(parts - 1))
    __hip_atomic_store(&p.hdr->next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int64_t nt = static_cast<int64_t>(gridDim.x) + c;
  sh.next_t = nt;
  sh.next_y = nt < parts ? p.target[nt / PARTS] : 0;
}

// Part 0 of a group (thread 0): the row a claim `c` stands for (issued when
// the current row started, so its target is read while the row is in
// flight); the launch's last claim resets the counter.
template <int G>
__device__ __forceinline__ int64_t group_row(const Params& p, uint32_t c) {
  return static_cast<int64_t>(gridDim.x / G) + c;
}
template <int G>
__device__ __forceinline__ int64_t group_target(const Params& p, uint32_t c) {
  const int64_t nr = group_row<G>(p, c);
  return nr < p.rows ? p.target[nr] : 0;
}
__device__ __forceinline__ void group_reset(const Params& p, uint32_t c) {
  if (c == static_cast<uint32_t>(p.rows - 1))
    __hip_atomic_store(&p.hdr->next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0: the group's next row and its target into the block-shared
// state (the other parts take them from part 0's words 5-7; if they never
// came, the workgroup stops). ok: every part's words arrived in time; else
// the call's epoch is stamped into the header and later exchanges of the
// workgroup poll once.
template <int G, class SH>
__device__ __forceinline__ void group_next(const Params& p, int h, bool ok, bool have_next,
                                          uint32_t c, int64_t ny,
                                          const uint32_t (&w0)[kSlotWords], SH& sh) {
  if (h == 0) {
    sh.next_t = group_row<G>(p, c);
    sh.next_y = ny;
  } else {
    sh.next_t = have_next ? static_cast<int64_t>(w0[5]) : p.rows;
    sh.next_y = static_cast<int64_t>((static_cast<uint64_t>(w0[7]) << 32) | w0[6]);
  }
  if (!ok) {
    __hip_atomic_store(&p.hdr->xerr_epoch, p.xstamp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.limit = 1;
  }
}

// Part 0 of a row whose exchange gave up: NaN over the whole row's gradient
// (its nv_row vectors and the row tail). GB: the compacted bf16 layout
// (element e at byte 2 e).
template <class E, int BLOCK, int GB>
__device__ __forceinline__ void poison_row(char* rp, int nv_row, int64_t tail0, int tail,
                                           int tid) {
  if constexpr (GB) {
    const u2 q = {0x7fc07fc0u, 0x7fc07fc0u};
    for (int j = tid; j < nv_row; j += BLOCK)
      __builtin_nontemporal_store(q, reinterpret_cast<u2*>(rp) + j);
    if (tid < tail) reinterpret_cast<uint16_t*>(rp)[tail0 + tid] = 0x7fc0u;
  } else {
    const uint32_t w = E::EPV == 4 ? 0x7fc00000u : 0x7fc07fc0u;
    const u4 q = {w, w, w, w};
    for (int j = tid; j < nv_row; j += BLOCK)
      __builtin_nontemporal_store(q, reinterpret_cast<u4*>(rp) + j);
    if (tid < tail) E::st(rp, tail0 + tid, __builtin_nanf(""));
  }
}

// Part 0's words 5-7: the group's next row and its target.
template <int G>
__device__ __forceinline__ void next_words(const Params& p, uint32_t c, int64_t ny,
                                           uint32_t (&w)[kSlotWords]) {
  w[5] = static_cast<uint32_t>(group_row<G>(p, c));
  w[6] = static_cast<uint32_t>(ny);
  w[7] = static_cast<uint32_t>(static_cast<uint64_t>(ny) >> 32);
}

// One part (a whole row, or a half or quarter of one) of the persistent
// wide kernel.
// GB = 1 (fp32 logits only): the gradient is written as bf16 (nearest even),
// times gscale (one value, or one per row with gscale_per_row; null = 1),
// compacted in place at the start of the row's bytes (element e at byte
// 2 e), not as fp32 over the logits. A part writes only after every
// part of its row has published its partial, i.e. after every logit of the
// row has been consumed, so the compacted writes never meet a pending read.
template <class E, int BLOCK, int NREG, int PARTS, int SC, int SM, int GB = 0>
__device__ __forceinline__ void wide_part(const Params& p, int64_t t, int64_t y,
                                          WideShared<BLOCK>& sh, int64_t& next_t,
                                          int64_t& next_y, const float* gscale = nullptr,
                                          int gscale_per_row = 0,
                                          uint32_t* arrival = nullptr) {
  constexpr int NW = BLOCK / 64;
  constexpr int EPV = E::EPV;
  constexpr int GS = (EPV == 4) ? 4 : 2;  // slots per pass-1 group
  constexpr int NG = NREG / GS;
  constexpr bool KEEP_E = (EPV == 4) && !SC;
  Acc* s_acc = sh.acc;
  int* s_cand = sh.cand;

  const int64_t row = t / PARTS;
  const int h = PARTS == 1 ? 0 : static_cast<int>(t % PARTS);
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
  const int half = (nv_row + PARTS - 1) / PARTS;
  const int v0 = h * half;
  const int nv = max(0, min(half, nv_row - v0));  // vectors of this part
  const bool last = (h == PARTS - 1);
  const int tail = last ? static_cast<int>(p.V - static_cast<int64_t>(nv_row) * EPV) : 0;
  const int64_t tail0 = static_cast<int64_t>(nv_row) * EPV;
  char* hp = rp + static_cast<int64_t>(v0) * 16;  // this part's first vector
  const int64_t e0 = static_cast<int64_t>(v0) * EPV;  // its first element

  if (ignored || bad) {
    // Ignored rows are never read; their gradient is exactly +0.0
    // (tt-mlir PR #9324 page: ignored rows, also with non-finite logits).
    if constexpr (PARTS == 1) {
      __syncthreads();  // every thread has read the previous part's next_t
      if (tid == 0) claim_finish<PARTS>(p, claim_issue(p), sh);
      __syncthreads();
      next_t = uniform_i64(sh.next_t);
      next_y = uniform_i64(sh.next_y);
    }
    uint32_t claim = 0;
    if constexpr (PARTS > 1) {
      if (tid == 0 && h == 0) claim = claim_issue(p);
    }
    if (p.grad) {
      if constexpr (GB) {
        u2* vp = reinterpret_cast<u2*>(rp + e0 * 2);
        for (int j = tid; j < nv; j += BLOCK) __builtin_nontemporal_store(u2{0u, 0u}, vp + j);
        if (tid < tail) reinterpret_cast<uint16_t*>(rp)[tail0 + tid] = 0;
      } else {
        u4* vp = reinterpret_cast<u4*>(hp);
        for (int j = tid; j < nv; j += BLOCK)
          __builtin_nontemporal_store(u4{0u, 0u, 0u, 0u}, vp + j);
        if (tid < tail) E::st(rp, tail0 + tid, 0.0f);
      }
    }
    if constexpr (PARTS > 1) {
      // no partials to combine: part 0 only hands over the group's next row
      __syncthreads();  // every thread has read the previous part's next_t
      if (tid == 0) {
        uint32_t w[kSlotWords] = {};
        bool ok = true;
        int64_t ny = 0;
        uint64_t* slots = row_slots<PARTS>(p, row);
        if (h == 0) {
          group_reset(p, claim);
          ny = group_target<PARTS>(p, claim);
          next_words<PARTS>(p, claim, ny, w);
          slot_publish(p, slots, w, kPartialWords, kSlotWords);
        } else {
          ok = slot_poll(p, slots, w, kPartialWords, kSlotWords, kGroupSpinLimit);
        }
        group_next<PARTS>(p, h, ok, ok, claim, ny, w, sh);
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
    // stores are dropped. Every part reads the target logit before any
    // can write a gradient (each writes only after all have published).
    // Part 0 of a group claims the group's next row before its loads go out.
    uint32_t claim = 0;
    if constexpr (PARTS > 1) {
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
    // the class weights of the thread's vectors (weighted smoothing)
    const WSlot wsl = {make_rsrc_bytes(p.weight, static_cast<int>(p.V) * 4),
                       (v0 + tid) * (EPV * 4), 0};
    u4 r[NREG];
#pragma unroll
    for (int k = 0; k < NREG; ++k)
      r[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, k * BLOCK * 16, kLoadNT);
    int64_t ny = 0;  // target of the group's next row (part 0, thread 0)
    if constexpr (PARTS > 1) {
      if (tid == 0 && h == 0) ny = group_target<PARTS>(p, claim);
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
        // softcap rows: the exponent t (c log2 e) - zg log2 e as one fma
        const float zgl = zg * kLog2e;
        const float cl = p.softcap * kLog2e;
        float gsum = 0.0f;
#pragma unroll
        for (int q = 0; q < GS; ++q) {
          const int k = g * GS + q;
          if (k * BLOCK < nv) {
            float f[EPV];
            E::unpack(r[k], f);
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
            if constexpr (KEEP_E) r[k] = F32::pack(e);
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
    bool part_nan = s_acc[0].s != s_acc[0].s;  // a NaN (or +inf) in the part
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      bmax = __builtin_fmaxf(bmax, s_acc[w].bv);
      part_nan = part_nan || s_acc[w].s != s_acc[w].s;
    }

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
    if (part_nan) {
      const int nc = first_nan<E, BLOCK, NREG, KEEP_E>(r, rsrc, voff, nv, tid, e0, xt,
                                                       tid < tail, tail0 + tid);
      if (lane == 0) sh.nanc[wave] = nc;
    }
    __syncthreads();

    if (wave == 0) {
      // Wave 0 combines the NW wave records with a fixed butterfly (lane l
      // holds wave l's record; the same tree every time, so bitwise
      // deterministic); lane 0 then owns the part's totals.
      Acc t;
      int arg = kNoIndex, nanarg = kNoIndex;
      if (lane < NW) {
        t = s_acc[lane];
        arg = s_cand[lane];
        if (part_nan) nanarg = sh.nanc[lane];
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
        nanarg = min(nanarg, __shfl_xor(nanarg, off, 64));
      }
      t.bv = bmax;
      t.bi = arg;
      if (nanarg != kNoIndex) {  // the part's first NaN ranks above every number
        t.bv = __builtin_nanf("");
        t.bi = nanarg;
      }
      if constexpr (PARTS > 1) {
        // Lane 0 publishes this part's partial (part 0 adds the group's
        // next row); lanes 0 .. G-1 poll the other parts' slots, one slot
        // per lane, so the group costs one round trip; then every lane folds
        // the G partials in part order, part 0 first, so every part of the
        // row gets bitwise identical row scalars.
        uint64_t* slots = row_slots<PARTS>(p, row);
        if (lane == 0) {
          uint32_t mine_w[kSlotWords] = {
              __builtin_bit_cast(uint32_t, t.m), __builtin_bit_cast(uint32_t, t.s),
              __builtin_bit_cast(uint32_t, t.sz), __builtin_bit_cast(uint32_t, t.bv),
              static_cast<uint32_t>(t.bi), 0u, 0u, 0u};
          if (h == 0) {
            group_reset(p, claim);
            next_words<PARTS>(p, claim, ny, mine_w);
          }
          slot_publish(p, slots + kSlotWords * h, mine_w, 0, h == 0 ? kSlotWords : kPartialWords);
        }
        uint32_t w[kSlotWords] = {};
        const int nwords = lane == 0 ? kSlotWords : kPartialWords;
        bool done = !(lane < PARTS && lane != h);
        // After `limit` polls the exchange has failed; a part other than 0
        // then waits on (the full limit) only for part 0's words 5-7, the
        // group's next row.
        const int limit = sh.limit;
        bool failed = false;
        int it = 0;
        while (true) {
          if (!done) {
            const uint64_t* src = slots + kSlotWords * lane;
            bool all = true;
#pragma unroll
            for (int i = 0; i < kSlotWords; ++i) {
              if (i < nwords) {
                const uint64_t v =
                    __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                w[i] = static_cast<uint32_t>(v);
                all = all && (static_cast<uint32_t>(v >> 32) == p.epoch);
              }
            }
            done = all;
          }
          if (__all(done)) break;
          ++it;  // counts every poll round, so the limits below always end the loop
          failed = failed || it >= limit;
          if (failed && (h == 0 || __shfl(done ? 1 : 0, 0, 64) != 0)) break;
          if (it >= kGroupSpinLimit) break;
          __builtin_amdgcn_s_sleep(1);
        }
        const bool ok = !failed;
        const bool have_next = h == 0 || __shfl(done ? 1 : 0, 0, 64) != 0;
        const float own_m = __shfl(t.m, 0, 64), own_s = __shfl(t.s, 0, 64);
        const float own_z = __shfl(t.sz, 0, 64), own_b = __shfl(t.bv, 0, 64);
        const int own_i = __shfl(t.bi, 0, 64);
        float m = 0.0f, sum = 0.0f, sz = 0.0f, bv = 0.0f;
        int bi = kNoIndex;
#pragma unroll
        for (int q = 0; q < PARTS; ++q) {
          float mq = __builtin_bit_cast(float, __shfl(w[0], q, 64));
          float sq = __builtin_bit_cast(float, __shfl(w[1], q, 64));
          float zq = __builtin_bit_cast(float, __shfl(w[2], q, 64));
          float bq = __builtin_bit_cast(float, __shfl(w[3], q, 64));
          int iq = static_cast<int>(__shfl(w[4], q, 64));
          if (q == h) {
            mq = own_m;
            sq = own_s;
            zq = own_z;
            bq = own_b;
            iq = own_i;
          }
          if (q == 0) {
            m = mq;
            sum = sq;
            sz = zq;
            bv = bq;
            bi = iq;
          } else {
            ms_combine(m, sum, mq, sq);
            sz += zq;
            // ties keep the earlier part (lower indices); a NaN ranks above
            // every number, the earliest part's first
            const bool take = (bq != bq) ? (bv == bv) : (bv == bv && bq > bv);
            bv = take ? bq : bv;
            bi = take ? iq : bi;
          }
        }
        if (!ok) {  // poisoned: NaN row scalars, no argmax
          m = sum = sz = bv = __builtin_nanf("");
          bi = -1;
        }
        uint32_t w0[kSlotWords] = {};  // part 0's words 5-7: the next row (parts 1 .. G-1)
        w0[5] = __shfl(w[5], 0, 64);
        w0[6] = __shfl(w[6], 0, 64);
        w0[7] = __shfl(w[7], 0, 64);
        if (lane == 0) group_next<PARTS>(p, h, ok, have_next, claim, ny, w0, sh);
        t.m = m;
        t.s = sum;
        t.sz = sz;
        t.bv = bv;
        t.bi = bi;
      }
      if (lane == 0) {
        if constexpr (PARTS == 1) claim = claim_issue(p);
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
        if constexpr (PARTS == 1) claim_finish<PARTS>(p, claim, sh);
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
    // fp32: the workgroup's last part arrives at the epilogue's counter now
    // (this part's row values, if any, are stored), and the arrival's round
    // trip overlaps the gradient stores below (the result is read after
    // them). The address carries an opaque per-lane zero, so the atomic
    // stays a one-lane one whose result is not waited for here. (The check
    // in every part measured slower on the bf16 kernels, whose workgroups
    // run many more parts at the benchmarked sizes.)
    if constexpr (E::EPV == 4) {
      if (arrival != nullptr && p.epilogue && tid == 0 &&
          next_t >= (PARTS > 1 ? p.rows : p.rows * PARTS)) {
        __builtin_amdgcn_s_waitcnt(0);
        int zero = 0;
        asm volatile("" : "+v"(zero));
        *arrival = __hip_atomic_fetch_add(&p.hdr->done + zero, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    // ---- pass 2: the gradient from on-chip data, written over the logits ----
    // (part 0 of a row whose exchange gave up, argmax -1, writes NaN over the
    // whole row instead, so no part of it keeps stale logits even if another
    // part stopped)
    if (PARTS > 1 && p.grad && h == 0 && sh.rs.arg < 0) {
      poison_row<E, BLOCK, GB>(rp, nv_row, tail0, static_cast<int>(p.V - tail0), tid);
    } else if (p.grad) {
      const RowScalars rs = sh.rs;
      // GB: this part's bf16 gradient bytes and the scale applied before rounding
      __amdgpu_buffer_rsrc_t rsrc_g = rsrc;
      float gsc = 1.0f;
      if constexpr (GB) {
        rsrc_g = make_rsrc_bytes(rp + e0 * 2, nv * 8);
        if (gscale) gsc = gscale[gscale_per_row ? row : 0];
      }
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
                gv = grad_vec_e<SM>(p, rs, r[k], sc, WSlot{wsl.rs, wsl.voff, k * BLOCK * 16}, -1);
              } else {
                gv = grad_vec<E, SC, SM>(p, rs, r[k], WSlot{wsl.rs, wsl.voff, k * BLOCK * EPV * 4},
                                         -1);
              }
              // lanes past the part are outside the descriptor: the store is dropped
              if constexpr (GB) {
                const f4 gf = __builtin_bit_cast(f4, gv);
                const u2 gb = {pack_bf16x2(gf[0] * gsc, gf[1] * gsc),
                               pack_bf16x2(gf[2] * gsc, gf[3] * gsc)};
                __builtin_amdgcn_raw_buffer_store_b64(gb, rsrc_g, tid * 8, k * BLOCK * 8, kStoreNT);
              } else {
                __builtin_amdgcn_raw_buffer_store_b128(gv, rsrc, voff, k * BLOCK * 16, kStoreNT);
              }
            }
          }
        }
      }
      if (tid < tail) {
        const int64_t k = tail0 + tid;
        const float wk = (SM && p.weight) ? p.weight[k] : 1.0f;
        if constexpr (GB) {
          reinterpret_cast<uint16_t*>(rp)[k] = to_bf16(grad_one<SC, SM>(p, rs, xt, wk, k == y) * gsc);
        } else {
          E::st(rp, k, grad_one<SC, SM>(p, rs, xt, wk, k == y));
        }
      }
      // The one-hot term: the vectors above were written without it; the
      // thread that wrote the target's vector rewrites that one element (its
      // own later store to the same address, same path and policy).
      const int64_t yl = y - e0;  // target position within this part
      if (yl >= 0 && yl < static_cast<int64_t>(nv) * EPV &&
          tid == static_cast<int>((yl / EPV) % BLOCK)) {
        const float wy = (SM && p.weight) ? p.weight[y] : 1.0f;
        if constexpr (GB) {
          __builtin_amdgcn_raw_buffer_store_b16(
              to_bf16(grad_one<SC, SM>(p, rs, sh.xy, wy, true) * gsc), rsrc_g,
              static_cast<int>(yl) * 2, 0, kStoreNT);
        } else {
          E::template st_buf<kStoreNT>(rsrc, static_cast<int>(yl),
                                       grad_one<SC, SM>(p, rs, sh.xy, wy, true));
        }
      }
    }
  }
}

// Persistent: as many workgroups as fit on the device at once (at most one
// per part; a multiple of G for rows split over G parts); each processes
// parts until the claims run out, then arrives once at the epilogue. The
// next part's loads are issued as soon as the current part's gradient
// stores are (they drain while the next part arrives).
// Four waves per SIMD: one 1024-thread workgroup or two 512-thread ones per
// CU, so at most 128 VGPRs.
template <class E, int BLOCK, int NREG, int PARTS, int SC, int SM>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) void wide_kernel(
    Params p) {
  static_assert(PARTS == 1 || PARTS == 2 || PARTS == 4, "whole, half or quarter rows");
  __shared__ WideShared<BLOCK> sh;
  __shared__ int s_last;
  // self_scales: every workgroup counts n and D once, before its parts
  // (kept out of the part loop, whose registers it would otherwise crowd)
  if (p.self_scales) compute_self_scales<BLOCK>(p);
  if (threadIdx.x == 0) sh.limit = p.spin_limit > 0 ? p.spin_limit : kGroupSpinLimit;
  // thread 0: the arrival count returned when the workgroup arrived with its
  // last part, else ~0
  uint32_t arrival = ~0u;
  if constexpr (PARTS > 1) {
    // group j = workgroups G j ... G j + G - 1 starts with row j (the grid
    // holds at most one group per row)
    const int h = static_cast<int>(blockIdx.x % PARTS);
    int64_t row = blockIdx.x / PARTS;
    int64_t y = p.target[row];
    while (row < p.rows) {
      int64_t nr, ny;
      wide_part<E, BLOCK, NREG, PARTS, SC, SM>(p, PARTS * row + h, y, sh, nr, ny, nullptr, 0,
                                               &arrival);
      row = nr;
      y = ny;
    }
  } else {
    const int64_t parts = p.rows;
    int64_t t = blockIdx.x;
    int64_t y = p.target[t];
    while (t < parts) {
      int64_t nt, ny;
      wide_part<E, BLOCK, NREG, PARTS, SC, SM>(p, t, y, sh, nt, ny, nullptr, 0, &arrival);
      t = nt;
      y = ny;
    }
  }
  if (p.epilogue) {
    if (threadIdx.x == 0)
      s_last = arrival != ~0u ? arrival == gridDim.x - 1u : arrive(p, gridDim.x);
    __syncthreads();
    if (s_last) epilogue_finish<BLOCK>(p);
  }
}

// The same on fp32 logits, with the gradient times gscale (one value, or one
// per row with gscale_per_row; null = 1) written as bf16 rows compacted in
// place (the linear layer's gradient products read it directly). The scale
// is an argument of its own, so wide_kernel's argument layout is left as it
// is; the part loop is written out again rather than shared through an
// inlined function, which changed wide_kernel's instruction schedule.
template <class E, int BLOCK, int NREG, int PARTS, int SC, int SM>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) void wide_kernel_gbf16(
    Params p, const float* gscale, int gscale_per_row) {
  static_assert(PARTS == 2 || PARTS == 4, "bf16 gradients: split rows");
  static_assert(E::EPV == 4, "bf16 gradients: fp32 logits");
  __shared__ WideShared<BLOCK> sh;
  __shared__ int s_last;
  if (p.self_scales) compute_self_scales<BLOCK>(p);
  if (threadIdx.x == 0) sh.limit = p.spin_limit > 0 ? p.spin_limit : kGroupSpinLimit;
  const int h = static_cast<int>(blockIdx.x % PARTS);
  int64_t row = blockIdx.x / PARTS;
  int64_t y = p.target[row];
  while (row < p.rows) {
    int64_t nr, ny;
    wide_part<E, BLOCK, NREG, PARTS, SC, SM, 1>(p, PARTS * row + h, y, sh, nr, ny, gscale,
                                                gscale_per_row);
    row = nr;
    y = ny;
  }
  if (p.epilogue) {
    if (threadIdx.x == 0) s_last = arrive(p, gridDim.x);
    __syncthreads();
    if (s_last) epilogue_finish<BLOCK>(p);
  }
}

}  // namespace cedev
