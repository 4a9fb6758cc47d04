// The linear layer fused with the cross-entropy, forward without gradients:
// logits = hidden @ weight^T computed tile by tile on the matrix cores
// (v_mfma_f32_32x32x16_bf16: bf16 products, fp32 sums) and reduced on chip
// to one partial per (row, block of 256 classes) -- max and sum of
// exponentials, smoothing sum, largest raw logit with its first index, the
// target logit -- so the fp32 logits never reach memory. The partials are
// then folded per row in class order by the vocabulary-shard finish kernel
// (each block of classes is one "shard"), which writes the loss outputs.
// The Liger-Kernel page "Kernel Profile: CrossEntropy (Tier 3 -
// Fused/Complex)", Classification, names the fused linear cross-entropy as
// the kernel this one extends with a linear layer.
//
// Tiles (one workgroup): 256 classes x 256 rows, the reduction dimension H
// in slices of 32 (H a multiple of 32), four slices in flight. The products
// are computed transposed, classes on the matrix instruction's M side
// (operand A = weight rows) and batch rows on its N side (operand B = hidden
// rows): both operands are then read H-contiguous, and each lane's
// accumulators hold 16 classes of one row, so the per-row reductions of the
// epilogue run mostly inside a lane. Eight waves: kLinWC groups of the
// classes x kLinWR groups of the rows, each wave 256 / kLinWC classes x
// 32 kLinNJ rows in tiles of 32 x 32 (two waves per SIMD, one workgroup
// per CU).
#pragma once

#include "ce_shard.hpp"

namespace cedev {

constexpr int kLinTileV = 256;    // classes per workgroup
constexpr int kLinWC = 2;         // waves along the classes (each 256 / kLinWC classes)
constexpr int kLinWR = 4;         // waves along the rows
constexpr int kLinNJ = 2;         // 32-row tiles per wave
constexpr int kLinNI = kLinTileV / kLinWC / 32;  // 32-class tiles per wave
constexpr int kLinTileR = 32 * kLinNJ * kLinWR;  // batch rows per workgroup
constexpr int kLinTileK = 32;     // H per stage (32: 64-byte rows of bf16, 64: 128-byte rows)
constexpr int kLinStages = 4;     // LDS stages in flight
constexpr int kLinWavesPerEU = 2;
constexpr int kLinWaves = kLinWC * kLinWR;
constexpr int kLinThreads = 64 * kLinWaves;
constexpr int kLinRowBytes = kLinTileK * 2;
constexpr int kLinChunks = kLinTileK / 8;   // 16-byte chunks per LDS row
constexpr int kLinLoadsA = kLinTileV * kLinRowBytes / 1024 / kLinWaves;  // 1 KiB loads per wave
constexpr int kLinLoadsB = kLinTileR * kLinRowBytes / 1024 / kLinWaves;  // per stage
// Position of chunk c of row R in LDS: c ^ lin_swz(R). Rows 16 / chunks
// apart share banks; the permutation spreads the rows of each such period.
__device__ __forceinline__ int lin_swz(int r) { return (r / (16 / kLinChunks)) % kLinChunks; }
// s_waitcnt immediate: vmcnt(n), expcnt and lgkmcnt left at their maxima
constexpr int lin_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct LinArgs {
  const uint16_t* hidden;  // bf16 (rows, ldh)
  const uint16_t* weight;  // bf16 (V, ldw)
  int64_t ldh, ldw;
  int H;
  int ncb;                 // class blocks: ceil(V / 256)
  int nrb;                 // row blocks: ceil(rows / 128)
  int cpx;                 // class blocks per XCD: ceil(ncb / 8)
  int npr;                 // row-block patches per XCD: ceil(nrb / 8)
  Partial* parts;          // (ncb, rows), shards by increasing class
};

// Work item of a workgroup. Workgroups are dispatched to the 8 XCDs in
// turn, so the workgroups running together on one XCD (and sharing its L2)
// are those with the same blockIdx.x mod 8: each XCD takes its own range of
// class blocks and walks it in patches of 4 class blocks x 8 row blocks, 32
// workgroups (one per CU of the XCD) that read 4 weight tiles and 8 hidden
// tiles between them.
__device__ __forceinline__ bool lin_work(const LinArgs& g, int& cb, int& rb) {
  const int xcd = blockIdx.x & 7;
  const int q = blockIdx.x >> 3;
  const int patch = q >> 5, within = q & 31;
  const int pc = patch / g.npr, pr = patch - pc * g.npr;
  const int cl = pc * 4 + (within >> 3);
  rb = pr * 8 + (within & 7);
  cb = xcd * g.cpx + cl;
  return cl < g.cpx && cb < g.ncb && rb < g.nrb;
}

template <int SC, int SM>
__global__ __launch_bounds__(kLinThreads) __attribute__((amdgpu_waves_per_eu(
    kLinWavesPerEU, kLinWavesPerEU))) void linear_partials_kernel(Params p, LinArgs g) {
  constexpr int NJ = kLinNJ;
  constexpr int NST = kLinStages;
  constexpr int NL = kLinLoadsA + kLinLoadsB;  // loads per thread per stage
  int cb, rb;
  if (!lin_work(g, cb, rb)) return;  // uniform: the grid is padded to whole patches
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wc = wave % kLinWC, wr = wave / kLinWC;  // class group, row group
  const int64_t c0 = static_cast<int64_t>(cb) * kLinTileV;
  const int64_t r0 = static_cast<int64_t>(rb) * kLinTileR;

  // NST LDS stages of the weight slice (256 rows) and the hidden slice
  // (kLinTileR rows), 64 bytes (32 H values) per row. The slices are loaded
  // straight into LDS (global_load_lds_dwordx4: lane l of a wave's load
  // writes 16 bytes at the load's LDS base + 16 l), each load filling 1 KiB,
  // i.e. 16 rows: row R of a block, 16-byte chunk position p = l % 4. The
  // chunks of row R are stored permuted, chunk c at position c ^ ((R / 4) %
  // 4), so the fragment reads below (16 lanes, 16 consecutive rows, one chunk
  // each) hit 16 distinct groups of 4 banks. Rows past V or past the batch
  // are read from the last valid row (their results are never used).
  // The stages, and after the products the epilogue's areas: per wave 32
  // rows x (CW + 4) floats, then the records of the class groups above the
  // first (kLinWC - 1) x 2 x 32 NJ rows.
  constexpr int NI = kLinNI;
  constexpr int CW = 32 * NI;  // classes per wave
  constexpr int kEP = CW + 4;
  constexpr int kStageBytes = NST * (kLinTileV + kLinTileR) * kLinRowBytes;
  constexpr int kEpilogueBytes =
      kLinWaves * 32 * kEP * 4 + (kLinWC - 1) * kLinWR * 32 * NJ * static_cast<int>(sizeof(Partial));
  __shared__ __attribute__((aligned(1024)))
  uint8_t smem[kStageBytes > kEpilogueBytes ? kStageBytes : kEpilogueBytes];
  constexpr int SA = kLinTileV * kLinRowBytes, SB = kLinTileR * kLinRowBytes;
  uint8_t (*sA)[SA] = reinterpret_cast<uint8_t (*)[SA]>(smem);
  uint8_t (*sB)[SB] = reinterpret_cast<uint8_t (*)[SB]>(smem + NST * SA);
  // A load fills 1 KiB = 1024 / kLinRowBytes rows: lane l writes row
  // l / chunks of the block at position l % chunks.
  constexpr int RPI = 1024 / kLinRowBytes;
  const int rl = lane / kLinChunks, pl = lane % kLinChunks;
  int64_t goa[kLinLoadsA], gob[kLinLoadsB];  // element offsets of the lane's loads
#pragma unroll
  for (int q = 0; q < kLinLoadsA; ++q) {
    const int R = (wave * kLinLoadsA + q) * RPI + rl;
    int64_t v = c0 + R;
    v = v < p.V ? v : p.V - 1;
    goa[q] = v * g.ldw + (pl ^ lin_swz(R)) * 8;
  }
#pragma unroll
  for (int q = 0; q < kLinLoadsB; ++q) {
    const int R = (wave * kLinLoadsB + q) * RPI + rl;
    int64_t r = r0 + R;
    r = r < p.rows ? r : p.rows - 1;
    gob[q] = r * g.ldh + (pl ^ lin_swz(R)) * 8;
  }
  auto load_stage = [&](int buf, int k0) {
#pragma unroll
    for (int q = 0; q < kLinLoadsA; ++q)
      __builtin_amdgcn_global_load_lds(g.weight + goa[q] + k0,
                                       &sA[buf][(wave * kLinLoadsA + q) * 1024], 16, 0, 0);
#pragma unroll
    for (int q = 0; q < kLinLoadsB; ++q)
      __builtin_amdgcn_global_load_lds(g.hidden + gob[q] + k0,
                                       &sB[buf][(wave * kLinLoadsB + q) * 1024], 16, 0, 0);
  };

  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

  // Fragment reads: lane l takes row l % 32 of a 32-row tile and, for the
  // 16 H values of step s, chunk 2 s + l / 32, at its permuted position.
  constexpr int NS = kLinTileK / 16;  // steps per stage
  const int sw = lin_swz(lane & 31);
  int fo[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st)
    fo[st] = (lane & 31) * kLinRowBytes + ((2 * st + (lane >> 5)) ^ sw) * 16;
  const int fa = wc * CW * kLinRowBytes, fb = wr * (32 * NJ) * kLinRowBytes;
  constexpr int TS = 32 * kLinRowBytes;  // bytes of a 32-row tile
  const int nk = g.H / kLinTileK;
  // stages 0 .. NST - 2 in flight before the loop
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nk) load_stage(st, st * kLinTileK);
  __builtin_amdgcn_s_waitcnt(lin_vmcnt(0));
  __syncthreads();
  // Fragments of the 16-wide steps of a stage: those of step 0 are read
  // before the stage's products start (right after the barrier), those of
  // each later step while the products of the step before run.
  bf16x8 fa_[2][NI], fb_[2][NJ];
  auto read_frags = [&](int buf, int off, bf16x8 (&a)[NI], bf16x8 (&b)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][fa + i * TS + off]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = *reinterpret_cast<const bf16x8*>(&sB[buf][fb + j * TS + off]);
  };
  auto products = [&](const bf16x8 (&a)[NI], const bf16x8 (&b)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  read_frags(0, fo[0], fa_[0], fb_[0]);
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks % NST;
#pragma unroll
    for (int st = 0; st + 1 < NS; ++st) {
      read_frags(buf, fo[st + 1], fa_[(st + 1) & 1], fb_[(st + 1) & 1]);
      products(fa_[st & 1], fb_[st & 1]);
      // interleave: one product, one fragment read of the next step
#pragma unroll
      for (int u = 0; u < NI + NJ; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (NI * NJ > NI + NJ)
        __builtin_amdgcn_sched_group_barrier(0x008, NI * NJ - (NI + NJ), 0);
    }
    // Stage ks + NST - 1 goes out after this stage's last fragment reads (in
    // program order, so the reads need not wait for it), into the buffer
    // that was last read before the previous barrier.
    __builtin_amdgcn_sched_barrier(0);
    const bool more = ks + NST - 1 < nk;
    if (more) load_stage((ks + NST - 1) % NST, (ks + NST - 1) * kLinTileK);
    __builtin_amdgcn_sched_barrier(0);
    products(fa_[(NS - 1) & 1], fb_[(NS - 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);  // the products are issued before the wait
    // stage ks + 1 has landed once at most the loads of the stages after it
    // are outstanding (the counter completes in order)
    if (more) {
      __builtin_amdgcn_s_waitcnt(lin_vmcnt((NST - 2) * NL));
    } else {
      __builtin_amdgcn_s_waitcnt(lin_vmcnt(0));
    }
    // Every wave's loads too, and every wave is done reading stage ks (its
    // products above waited for the reads). A bare s_barrier: the fence of
    // __syncthreads would also wait for the stages still in flight. LDS
    // accesses of one wave complete in order, and the compiler does not move
    // memory operations across the scheduling barriers.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (ks + 1 < nk) read_frags((ks + 1) % NST, fo[0], fa_[0], fb_[0]);
  }

  // ---- epilogue: per row, the partial over this wave's CW classes ----
  // Accumulator r of tile (i, j) in lane l holds row 32 j + l % 32 of the
  // wave's rows and class 32 i + 8 (r / 4) + 4 (l / 32) + r % 4 of its
  // classes. One 32-row tile at a time, the wave writes its CW x 32 logits
  // to its own LDS area (row-major, rows of CW + 4 floats so that the
  // 16-byte reads of 16 rows hit distinct banks); then lane l takes row
  // l % 32 and classes CW / 2 (l / 32) .. + CW / 2 - 1, and lanes l and
  // l ^ 32 combine.
  float* ep = reinterpret_cast<float*>(smem) + wave * 32 * kEP;
  const int er = lane & 31, eh = lane >> 5;
  const int64_t cbase = c0 + wc * CW + eh * (CW / 2);  // the lane's first class
  const int nv = static_cast<int>(p.V - cbase < CW / 2 ? (p.V - cbase > 0 ? p.V - cbase : 0)
                                                       : CW / 2);
  Partial rec[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f4*>(&ep[er * kEP + i * 32 + 8 * q + 4 * eh]) =
            f4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t row = r0 + wr * (32 * NJ) + j * 32 + er;
    const int64_t y = row < p.rows ? p.target[row] : p.ignore_index;
    const float* xr = &ep[er * kEP + eh * (CW / 2)];
    float bv = -__builtin_inff(), zmax = kLowest;
    int bi = kNoIndex;
    for (int e = 0; e < nv; ++e) {
      const float x = xr[e];
      arg_combine(bv, bi, x, static_cast<int>(cbase + e));
      zmax = __builtin_fmaxf(zmax, zval<SC>(p, x));
    }
    float s = 0.0f, sz = 0.0f;
    for (int e = 0; e < nv; ++e) {
      const float z = zval<SC>(p, xr[e]);  // recomputed, as the tanh of the first pass is not kept
      s += ex2((z - zmax) * kLog2e);
      if constexpr (SM) sz = p.weight ? __builtin_fmaf(p.weight[cbase + e], z, sz) : sz + z;
    }
    const bool here = y >= cbase && y < cbase + nv;
    float xy = here ? xr[y - cbase] : 0.0f;
    int has_y = here ? 1 : 0;
    // the other classes of the wave for this row, in lane l ^ 32
    float m2 = __shfl_xor(zmax, 32, 64), s2 = __shfl_xor(s, 32, 64);
    float sz2 = __shfl_xor(sz, 32, 64), bv2 = __shfl_xor(bv, 32, 64);
    int bi2 = __shfl_xor(bi, 32, 64);
    float xy2 = __shfl_xor(xy, 32, 64);
    int hy2 = __shfl_xor(has_y, 32, 64);
    // lower classes first: lanes 0..31 hold them
    ms_combine(zmax, s, m2, s2);
    sz += sz2;
    arg_combine(bv, bi, bv2, bi2);
    if (hy2) {
      xy = xy2;
      has_y = 1;
    }
    rec[j] = Partial{zmax, s, sz, bv, bi, xy, has_y, 0};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the area is written again by the next tile
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // The class groups of a row half: the groups above the first hand their
  // records to the first through LDS, which folds them in class order and
  // stores the block's partial.
  __syncthreads();
  Partial* sx = reinterpret_cast<Partial*>(smem + kLinWaves * 32 * kEP * 4);
  constexpr int RH = 32 * NJ;  // rows per row group
  if (wc > 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) sx[((wc - 1) * kLinWR + wr) * RH + j * 32 + lane] = rec[j];
  }
  __syncthreads();
  if (wc == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t row = r0 + wr * RH + j * 32 + lane;
      if (row < p.rows) {
        Partial q = rec[j];
        for (int c = 1; c < kLinWC; ++c) {
          const Partial u = sx[((c - 1) * kLinWR + wr) * RH + j * 32 + lane];
          ms_combine(q.m, q.s, u.m, u.s);
          q.sz += u.sz;
          arg_combine(q.bv, q.bi, u.bv, u.bi);
          if (u.has_y) {
            q.xy = u.xy;
            q.has_y = 1;
          }
        }
        g.parts[static_cast<int64_t>(cb) * p.rows + row] = q;
      }
    }
  }
}

}  // namespace cedev
