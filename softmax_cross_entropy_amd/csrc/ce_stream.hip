// HBM stream kernels for measurement (declared in include/ce_stream.h): read,
// write, in-place read-then-write, out-of-place copy and a cache flush, each
// over chunks of BLOCK threads x NREG 16-byte vectors with every load of a
// chunk issued before its first store (the layout of the fused cross-entropy
// kernels, without their arithmetic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ce_stream.h"

#define CE_API extern "C" __attribute__((visibility("default")))

namespace cestream {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data (gfx9 family)
constexpr int kNT = 2;                   // non-temporal (streaming) load / store

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kRsrcWord3);
}

// Chunk c of a buffer of nvec vectors: its descriptor (lanes past the end
// read 0 and their stores are dropped).
template <int CH>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk(const void* base, int64_t nvec,
                                                        int64_t c) {
  const int64_t v0 = c * CH;
  const int64_t n = nvec - v0 < CH ? nvec - v0 : CH;
  return rsrc(static_cast<const char*>(base) + v0 * 16, static_cast<int>(n) * 16);
}

// KIND: 0 read, 1 write, 2 in place, 3 copy, 4 flush (read, default policy).
// key is 0 in every launch; the compiler cannot see that, so loads feed the
// stores and the sink test and none can be dropped.
template <int KIND, int BLOCK, int NREG>
__global__ __launch_bounds__(BLOCK) void stream_kernel(char* dst, const char* src, int64_t nvec,
                                                       int64_t chunks, uint32_t key,
                                                       uint32_t* sink) {
  constexpr int CH = BLOCK * NREG;
  const int voff = threadIdx.x * 16;
  uint32_t acc = 0;
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    if constexpr (KIND == 1) {
      const __amdgpu_buffer_rsrc_t rd = chunk<CH>(dst, nvec, c);
      const u4 v = {key, key, key, key};
#pragma unroll
      for (int k = 0; k < NREG; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(v, rd, voff, k * BLOCK * 16, kNT);
    } else {
      const __amdgpu_buffer_rsrc_t rs = chunk<CH>(KIND == 2 ? dst : src, nvec, c);
      constexpr int pol = KIND == 4 ? 0 : kNT;
      u4 r[NREG];
#pragma unroll
      for (int k = 0; k < NREG; ++k)
        r[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, k * BLOCK * 16, pol);
      if constexpr (KIND == 0 || KIND == 4) {
#pragma unroll
        for (int k = 0; k < NREG; ++k) acc ^= r[k][0] ^ r[k][1] ^ r[k][2] ^ r[k][3];
      } else {
        const __amdgpu_buffer_rsrc_t rd = KIND == 2 ? rs : chunk<CH>(dst, nvec, c);
#pragma unroll
        for (int k = 0; k < NREG; ++k)
          __builtin_amdgcn_raw_buffer_store_b128(r[k] ^ key, rd, voff, k * BLOCK * 16, kNT);
      }
    }
  }
  if constexpr (KIND == 0 || KIND == 4) {
    // (acc == ~key is possible, so the loads stay; the store almost never runs)
    if (acc == ~key) sink[0] = acc;
  }
}

struct Config {
  int block, nreg;
};
constexpr Config kConfigs[] = {{256, 4},  {256, 8},  {256, 16}, {512, 4},  {512, 8},
                               {512, 16}, {1024, 4}, {1024, 8}, {1024, 16}};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

template <int KIND, int BLOCK, int NREG>
hipError_t launch(char* dst, const char* src, int64_t nvec, int64_t grid, uint32_t* sink,
                  hipStream_t st) {
  constexpr int64_t CH = static_cast<int64_t>(BLOCK) * NREG;
  const int64_t chunks = (nvec + CH - 1) / CH;
  const int64_t g = grid > 0 ? (grid < chunks ? grid : chunks) : chunks;
  if (g < 1) return hipSuccess;
  stream_kernel<KIND, BLOCK, NREG>
      <<<dim3(static_cast<unsigned>(g)), BLOCK, 0, st>>>(dst, src, nvec, chunks, 0u, sink);
  return hipGetLastError();
}

template <int KIND, int BLOCK, int NREG>
int64_t resident() {
  int per_cu = 0, ncu = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -6;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_kernel<KIND, BLOCK, NREG>,
                                                   BLOCK, 0) != hipSuccess)
    return -6;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -6;
  return static_cast<int64_t>(per_cu) * ncu;
}

// Dispatch on (kind, config) to the template instance F<KIND, BLOCK, NREG>.
template <int KIND, class F>
auto by_config(int config, F&& f) {
  switch (config) {
    case 0: return f.template operator()<KIND, 256, 4>();
    case 1: return f.template operator()<KIND, 256, 8>();
    case 2: return f.template operator()<KIND, 256, 16>();
    case 3: return f.template operator()<KIND, 512, 4>();
    case 4: return f.template operator()<KIND, 512, 8>();
    case 5: return f.template operator()<KIND, 512, 16>();
    case 6: return f.template operator()<KIND, 1024, 4>();
    case 7: return f.template operator()<KIND, 1024, 8>();
    default: return f.template operator()<KIND, 1024, 16>();
  }
}

template <class F>
auto by_kind(int kind, int config, F&& f) {
  switch (kind) {
    case 0: return by_config<0>(config, f);
    case 1: return by_config<1>(config, f);
    case 2: return by_config<2>(config, f);
    case 3: return by_config<3>(config, f);
    default: return by_config<4>(config, f);
  }
}

struct ResidentOf {
  template <int K, int B, int N>
  int64_t operator()() const { return resident<K, B, N>(); }
};

struct LaunchOf {
  char* d;
  const char* s;
  int64_t nvec, grid;
  uint32_t* sink;
  hipStream_t st;
  template <int K, int B, int N>
  hipError_t operator()() const { return launch<K, B, N>(d, s, nvec, grid, sink, st); }
};

}  // namespace cestream

CE_API int ce_stream_num_configs(void) { return cestream::kNumConfigs; }

CE_API int ce_stream_config(int config, int* block, int* nreg) {
  if (config < 0 || config >= cestream::kNumConfigs || block == nullptr || nreg == nullptr)
    return -4;
  *block = cestream::kConfigs[config].block;
  *nreg = cestream::kConfigs[config].nreg;
  return 0;
}

CE_API int64_t ce_stream_resident(int kind, int config) {
  if (kind < 0 || kind > 4 || config < 0 || config >= cestream::kNumConfigs) return -4;
  return cestream::by_kind(kind, config, cestream::ResidentOf{});
}

CE_API int ce_stream_run(int kind, int config, void* dst, const void* src, size_t bytes,
                         int64_t grid, uint32_t* sink, void* stream) {
  if (kind < 0 || kind > 4 || config < 0 || config >= cestream::kNumConfigs) return -4;
  const bool reads = kind == CE_STREAM_READ || kind == CE_STREAM_COPY || kind == CE_STREAM_FLUSH;
  const bool writes = kind == CE_STREAM_WRITE || kind == CE_STREAM_INPLACE || kind == CE_STREAM_COPY;
  if ((reads && src == nullptr) || (writes && dst == nullptr)) return -1;
  if ((kind == CE_STREAM_READ || kind == CE_STREAM_FLUSH) && sink == nullptr) return -1;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return -2;
  const int64_t nvec = static_cast<int64_t>(bytes / 16);
  const int64_t ch = static_cast<int64_t>(cestream::kConfigs[config].block) *
                     cestream::kConfigs[config].nreg;
  if (grid <= 0 && (nvec + ch - 1) / ch > 0x7fffffffLL) return -2;
  char* d = static_cast<char*>(dst);
  const char* s = static_cast<const char*>(src);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e =
      cestream::by_kind(kind, config, cestream::LaunchOf{d, s, nvec, grid, sink, st});
  return e == hipSuccess ? 0 : -6;
}
