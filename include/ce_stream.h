/* ce_stream.h -- C ABI of the HBM stream kernels the cross-entropy kernels are
 * measured against.
 *
 * The Liger-Kernel page "Kernel Profile: CrossEntropy (Tier 3 -
 * Fused/Complex)", Benchmarking, measures the fused kernel against other
 * providers on the same GPU; the memory traffic of the method (one read of
 * each counted logit, one write of each gradient element) is bounded by what
 * the GPU's memory can stream. These kernels measure that bound on the
 * machine itself, with the same access pattern, so that a kernel's time can
 * be stated as a fraction of a measured ceiling and not only of the data
 * sheet's peak:
 *   READ     every 16-byte vector of `src` read once (non-temporal);
 *   WRITE    every vector of `dst` written once (non-temporal);
 *   INPLACE  every vector of `dst` read, then written back unchanged at the
 *            same address (the read-then-overwrite pattern of the fused
 *            forward + gradient), a chunk at a time;
 *   COPY     `src` read, `dst` written (out of place);
 *   FLUSH    `src` read with the default cache policy, so that the caches
 *            hold it and not the data of the launch timed next.
 * A chunk is `block` threads x `nreg` 16-byte vectors per thread: every load
 * of a chunk is issued before its first store, as the fused kernels do.
 * grid = 0 launches one workgroup per chunk; grid > 0 launches that many
 * persistent workgroups, each taking chunks g, g + grid, ...
 *
 * Conventions: pointers are HIP device pointers owned by the caller; the
 * calls enqueue work on `stream` (a hipStream_t, NULL = null stream) and
 * return without waiting. Nothing is allocated.
 */
#ifndef CE_STREAM_MI355X_H
#define CE_STREAM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { CE_STREAM_READ = 0, CE_STREAM_WRITE = 1, CE_STREAM_INPLACE = 2, CE_STREAM_COPY = 3,
       CE_STREAM_FLUSH = 4 };

/* Number of compiled (block, nreg) chunk shapes; the shapes themselves
 * through ce_stream_config. */
int ce_stream_num_configs(void);

/* Shape `config` (0 <= config < ce_stream_num_configs()): threads per
 * workgroup and 16-byte vectors per thread. Returns 0, or -4 (CE_E_PARAM)
 * for an unknown index. */
int ce_stream_config(int config, int* block, int* nreg);

/* Workgroups of shape `config` of kernel `kind` resident on the current
 * device at once (occupancy x compute units), or a negative status. */
int64_t ce_stream_resident(int kind, int config);

/* One launch of kernel `kind`.
 *  dst     [device] destination (WRITE, INPLACE, COPY), else NULL.
 *  src     [device] source (READ, COPY, FLUSH), else NULL.
 *  bytes   multiple of 16; both pointers 16-byte aligned.
 *  sink    [device] one uint32, READ and FLUSH only (a workgroup writes
 *          the xor of what it read there if it equals a value it never
 *          takes in practice, so the loads cannot be dropped), or NULL.
 * Returns 0 (CE_OK), -1 (a pointer missing), -2 (bytes not a multiple of
 * 16, misaligned, or more chunks than a grid can hold), -4 (unknown kind
 * or config) or -6 (launch failure). */
int ce_stream_run(int kind, int config, void* dst, const void* src, size_t bytes, int64_t grid,
                  uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CE_STREAM_MI355X_H */
