/* ce.h -- C ABI of the MI355X (gfx950) fused softmax cross-entropy library.
 *
 * The operation is the one described on the Liger-Kernel page "Kernel
 * Profile: CrossEntropy (Tier 3 - Fused/Complex)":
 *   Forward Pass    -- inputs (logits (rows, V), target (rows,), optional
 *                      class weights (V,), ignore_index, label_smoothing,
 *                      reduction, softcap) and outputs (loss, z_loss,
 *                      token_accuracy, predicted tokens);
 *   Module Parameters -- lse_square_scale (z-loss), defaults;
 *   Key Patterns    -- online softmax, gradient-in-forward (the forward
 *                      overwrites the logits with d loss / d logits),
 *                      multiple loss components;
 *   Backward Pass   -- backward only scales the stored gradient by
 *                      grad_output.
 * The all-ignored mean (NaN loss, zero gradients) follows the tt-mlir pull
 * request page "[tt-crank] fuse cross entropy onto the ttml
 * cross_entropy_fw/bw composites" (#9324), Copilot comments on the mean
 * reduction.
 *
 * Definitions, with z = c tanh(x / c) for softcap c > 0 (else z = x),
 * lse_i = log sum_k exp(z_ik), eps = label_smoothing, w = class weights
 * (all ones when NULL), W = sum_k w_k, lam = lse_square_scale:
 *   l_i    = (1 - eps) w_y (lse_i - z_iy) + (eps / V) sum_k w_k (lse_i - z_ik)
 *   zeta_i = lam * lse_i^2
 * A row is counted when target != ignore_index and 0 <= target < V;
 * n = counted rows, D = sum over counted rows of w[target].
 *   mean: loss = sum l / D + sum zeta / n,  z_loss = sum zeta / n
 *   sum:  loss = sum l + sum zeta,          z_loss = sum zeta
 *   none: loss_i = l_i + zeta_i,            z_loss_i = zeta_i
 * token_accuracy = n_correct / n (mean, sum) or the per-row 0/1 (none);
 * argmax is over the raw logits, lowest index on ties, -1 on rows that are
 * not counted. Ignored rows are never read and get zero loss and a +0.0
 * gradient. The gradient is that of `loss` with grad_output = 1; for mean,
 * a zero D (or n) gives zero gradients and a NaN loss.
 * Rows whose target is outside [0, V) and not ignore_index get a NaN loss,
 * a zero gradient and argmax -1, are not counted, and set a device error
 * bit (see CE_F_CHECK_TARGETS).
 * Non-finite logits in counted rows follow IEEE arithmetic: a NaN or a +inf
 * makes the row's loss and gradient NaN; argmax ranks a NaN above every
 * number (the first NaN of the row), as numpy and torch order it.
 * Rows longer than one workgroup holds are split over a group of workgroups
 * that exchange partials and wait (a bounded number of polls) for each
 * other. If a wait gives up, which needs the group's workgroups not to be
 * resident together, nothing wrong is returned silently: the rows involved
 * get NaN loss and gradient, the reduced outputs are NaN, and
 * CE_F_CHECK_TARGETS returns CE_E_EXCHANGE.
 *
 * Conventions for every call:
 *  - Pointers marked [device] are HIP device pointers; the library never
 *    allocates, frees or keeps a pointer after returning.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream);
 *    the calls return without waiting for the GPU, except with
 *    CE_F_CHECK_TARGETS.
 *  - Arguments are validated on the host before anything is enqueued: on
 *    an error status nothing has been written.
 *  - Concurrent calls that share a workspace race; give each stream its
 *    own workspace. After its first zero fill a workspace needs no reset
 *    between calls: rows split over several workgroups exchange words
 *    stamped with a per-call number that repeats only after 2^30 - 1 calls
 *    in the process.
 */
#ifndef CE_MI355X_H
#define CE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CE_OK = 0,
  CE_E_NULL = -1,         /* a required pointer is NULL                        */
  CE_E_SHAPE = -2,        /* rows < 0, V < 1, row_stride < V, or too large     */
  CE_E_DTYPE = -3,        /* unknown dtype                                     */
  CE_E_PARAM = -4,        /* bad reduction, label_smoothing, softcap, scale    */
  CE_E_WORKSPACE = -5,    /* workspace NULL, too small or not 256-B aligned    */
  CE_E_HIP = -6,          /* a HIP runtime call or kernel launch failed        */
  CE_E_TARGET_RANGE = -7, /* CE_F_CHECK_TARGETS: a target outside [0, V)      */
  CE_E_EXCHANGE = -8,     /* CE_F_CHECK_TARGETS: a row split over workgroups   */
                          /* gave up waiting for one of its parts (its values */
                          /* and the reduced outputs are NaN)                 */
  CE_E_SCRATCH = -9       /* ce_forward_noalloc: ce_workspace_bytes(...) of   */
                          /* the problem exceeds CE_FORWARD_NOALLOC_MAX_BYTES */
} ce_status;

typedef enum { CE_F32 = 0, CE_BF16 = 1 } ce_dtype;

typedef enum { CE_RED_NONE = 0, CE_RED_MEAN = 1, CE_RED_SUM = 2 } ce_reduction;

enum {
  CE_F_GRAD = 1u << 0,          /* overwrite logits with d loss / d logits     */
  CE_F_CHECK_TARGETS = 1u << 4, /* wait for the GPU; CE_E_TARGET_RANGE if any  */
                                /* target is outside [0, V) and not ignored,   */
                                /* CE_E_EXCHANGE if a split row's wait gave up */
  CE_F_FORCE_FUSED = 1u << 5,   /* test hooks: pick the kernel path            */
  CE_F_FORCE_SPLITV = 1u << 6,
  CE_F_FORCE_SCALAR = 1u << 7,
  CE_F_SHAPE_ALT = 1u << 8,     /* test hook: the other fused layout where a   */
                                /* row size has two (rows of 2 K to 16 K       */
                                /* 16-byte vectors: 1024-thread workgroups vs  */
                                /* 256/512-thread ones; 16 K to 32 K: a pair   */
                                /* of 1024-thread workgroups per row vs four   */
                                /* 512-thread ones)                            */
  CE_F_EXCHANGE_ONE_POLL = 1u << 9, /* test hook: a row split over workgroups */
                                /* polls its parts' partials once before it    */
                                /* gives up (forces the failure path below)    */
  CE_F_LINEAR_ON_CHIP = 1u << 10 /* ce_linear_forward without gradients: the */
                                /* hand-written matrix-core kernel that keeps  */
                                /* the logits on chip (no logits workspace)    */
                                /* instead of the library GEMM and fp32 logits */
};

/* Kernel paths (ce_plan_path). */
enum {
  CE_PATH_FUSED = 1,   /* one workgroup per row, row kept on chip, 1 HBM read  */
  CE_PATH_SPLITV = 2,  /* row split over workgroups: partials, then combine    */
  CE_PATH_SCALAR = 3   /* rows not 16-byte aligned: element loads, two passes  */
};

/* Bytes of device workspace ce_forward needs for this problem (>= 256).
 * Returns 0 for invalid sizes or dtype. */
size_t ce_workspace_bytes(int64_t rows, int64_t V, int dtype, uint32_t flags);

/* The kernel path ce_forward would take (CE_PATH_*), or a negative
 * ce_status for invalid arguments. Host only; nothing is enqueued. */
int ce_plan_path(const void* logits, int dtype, int64_t rows, int64_t V, int64_t row_stride,
                 const float* weight, float label_smoothing, uint32_t flags);

/* Fused forward (+ gradient with CE_F_GRAD).
 *  logits     [device] (rows, row_stride) row-major, dtype `dtype`; the first V
 *             elements of each row are the logits. With CE_F_GRAD they are
 *             overwritten by the gradient in the same dtype (bf16: round to
 *             nearest even); otherwise they are only read.
 *  target     [device] int64 (rows).
 *  weight     [device] fp32 (V) class weights, or NULL.
 *  softcap    0 = off; else > 0 and finite.
 *  label_smoothing in [0, 1]; lse_square_scale finite, >= 0.
 *  loss       [device] fp32: 1 value (mean, sum) or rows values (none).
 *  z_loss     [device] fp32, same shape as loss, or NULL.
 *  token_accuracy [device] fp32, same shape as loss, or NULL.
 *  argmax     [device] int64 (rows), or NULL.
 *  counts     [device] int64 [n_counted, n_correct], or NULL.
 *  row_stats  [device] fp32 (rows, 2): per row the shift m = max z and
 *             log2 sum_k exp(z_k - m), kept for ce_backward_recompute; rows
 *             that are not counted get (0, 0). NULL = not written.
 *  workspace  [device] >= ce_workspace_bytes(...) bytes, 256-byte aligned,
 *             zero-filled before its first use (one hipMemset). Every call
 *             leaves it reusable: later calls on the same stream may pass it
 *             again without clearing. Two calls in flight at once must not
 *             share a workspace.
 */
ce_status ce_forward(void* logits, int dtype, int64_t rows, int64_t V, int64_t row_stride,
                     const int64_t* target, const float* weight, int64_t ignore_index,
                     float label_smoothing, float lse_square_scale, float softcap,
                     int reduction, uint32_t flags, float* loss, float* z_loss,
                     float* token_accuracy, int64_t* argmax, int64_t* counts, float* row_stats,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch ce_forward_noalloc holds per device (16 MiB). */
#define CE_FORWARD_NOALLOC_MAX_BYTES (16u << 20)

/* ce_forward for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, results and kernels without the workspace argument. The
 * workspace is a static device array of CE_FORWARD_NOALLOC_MAX_BYTES that
 * every device holds from the library's first use until the process ends;
 * the call allocates and frees nothing.
 *  - The first call on a device looks the array up for that device and
 *    enqueues one kernel that zero-fills it, ahead of its own work.
 *  - stream must belong to the current device (else CE_E_PARAM).
 *  - CE_E_SCRATCH if ce_workspace_bytes(rows, V, dtype, flags) exceeds
 *    CE_FORWARD_NOALLOC_MAX_BYTES (past 62598 rows at V = 131072 in fp32
 *    or V = 262144; 119832 rows of fp32 at V = 32768); nothing is enqueued
 *    then.
 *  - All calls on one device share the array and each leaves it ready for
 *    the next: calls in flight at the same time on one device (on different
 *    streams or host threads) race and must not overlap. */
ce_status ce_forward_noalloc(void* logits, int dtype, int64_t rows, int64_t V,
                             int64_t row_stride, const int64_t* target, const float* weight,
                             int64_t ignore_index, float label_smoothing,
                             float lse_square_scale, float softcap, int reduction,
                             uint32_t flags, float* loss, float* z_loss, float* token_accuracy,
                             int64_t* argmax, int64_t* counts, float* row_stats, void* stream);

/* Backward: grad (rows, row_stride) [device] *= grad_output in place.
 *  grad_output [device] fp32: one value, or rows values when per_row != 0
 *  (reduction none). Rows whose scale is exactly 1.0 are left untouched. */
ce_status ce_backward(void* grad, int dtype, int64_t rows, int64_t V, int64_t row_stride,
                      const float* grad_output, int per_row, void* stream);

/* Backward from kept logits: the gradient is recomputed instead of stored
 * by the forward. The tt-mlir PR #9324 page's cross_entropy_bw composite
 * (before/after table) takes the saved logits and target; here a forward
 * without CE_F_GRAD leaves the logits intact and fills row_stats, and this
 * call writes grad = grad_output * d loss / d logits (the same formula and
 * options as the fused forward's gradient) for every row, +0.0 for rows
 * that are not counted.
 *  logits, dtype, rows, V, row_stride, target, weight, ignore_index,
 *  label_smoothing, lse_square_scale, softcap, reduction
 *             as for the ce_forward call that produced row_stats.
 *  row_stats  [device] fp32 (rows, 2) from that ce_forward call.
 *  grad_output [device] fp32: one value, or rows values when per_row != 0.
 *  grad       [device] (rows, grad_stride), the logits' dtype; may be the
 *             logits themselves (in place, then grad_stride == row_stride),
 *             otherwise must not overlap them.
 *  workspace  [device] >= 256 bytes, 256-byte aligned; its first 256 bytes
 *             are overwritten (any ce_forward workspace will do).
 * Errors as ce_forward; CE_E_SHAPE also when grad_stride < V or when grad
 * is the logits with another stride. */
ce_status ce_backward_recompute(const void* logits, int dtype, int64_t rows, int64_t V,
                                int64_t row_stride, const int64_t* target, const float* weight,
                                int64_t ignore_index, float label_smoothing,
                                float lse_square_scale, float softcap, int reduction,
                                const float* row_stats, const float* grad_output, int per_row,
                                void* grad, int64_t grad_stride, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Linear layer fused with the cross-entropy. The Liger-Kernel page above,
 * Classification, names the fused linear cross-entropy as the kernel this
 * operation extends with a linear layer; read plainly, the logits are the
 * output of a bias-free linear layer (a language model head),
 *   logits = hidden @ weight^T,   hidden (rows, H), weight (V, H),
 * followed by exactly the cross-entropy of ce_forward (same options, same
 * outputs, same conventions), and the gradients follow by the chain rule
 * from G = d loss / d logits:
 *   d loss / d hidden = G @ weight,   d loss / d weight = G^T @ hidden.
 * The full (rows, V) logits are never held at once: rows are processed in
 * chunks of chunk_rows; each chunk's logits (fp32) live in the workspace,
 * are turned into G in place by the fused cross-entropy kernels, and feed
 * the two gradient products.
 *
 * Precision: hidden and weight are bf16; the products accumulate in fp32
 * (matrix cores, through rocBLAS); the logits and the cross-entropy are
 * fp32; G is scaled by grad_output and rounded to bf16 (nearest even)
 * before the two gradient products, whose fp32 results are returned.
 *
 * The GEMMs run through rocBLAS: the first call on a device creates that
 * device's rocBLAS handle (which allocates rocBLAS's own workspace); calls
 * after that allocate nothing.
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace ce_linear_forward needs (>= 256), or 0 for
 * invalid sizes. chunk_rows = 0 picks the default chunk: at most 2048 rows,
 * and at most 6 GiB of the chunk's fp32 logits, bf16 gradient and its
 * transpose (2.1 GB for 2048 rows at V = 128256). */
size_t ce_linear_workspace_bytes(int64_t rows, int64_t H, int64_t V, int64_t chunk_rows,
                                 uint32_t flags);

/* Forward of cross_entropy(hidden @ weight^T) and, when grad_hidden or
 * grad_weight is given, its gradients.
 *  hidden     [device] bf16 (rows, ld_hidden) row-major, first H used.
 *  weight     [device] bf16 (V, ld_weight) row-major (out x in), first H used.
 *  target, class_weight, ignore_index, label_smoothing, lse_square_scale,
 *  softcap, reduction, loss, z_loss, token_accuracy, argmax, counts
 *             as for ce_forward (class_weight: per-class weights, (V,)).
 *  flags      CE_F_CHECK_TARGETS and the kernel-path test hooks of
 *             ce_forward; CE_F_GRAD is implied by a gradient output.
 *  grad_output [device] fp32: one value, or rows values when per_row != 0;
 *             NULL = 1. The gradients are those of grad_output * loss (per
 *             row for reduction none).
 *  grad_hidden [device] fp32 (rows, ld_grad_hidden), or NULL; overwritten.
 *  grad_weight [device] fp32 (V, ld_grad_weight), or NULL; overwritten.
 *  chunk_rows rows per chunk (> 0), or 0 for the default; the workspace
 *             must have been sized with the same value.
 *  workspace  [device] >= ce_linear_workspace_bytes(...) bytes, 256-byte
 *             aligned; any contents (each call clears the part it needs
 *             with a kernel on `stream`). Two calls in flight at once must
 *             not share a workspace.
 * Errors as ce_forward; CE_E_DTYPE if dtype is not CE_BF16; CE_E_SHAPE also
 * for H < 1 or a leading dimension below H. */
ce_status ce_linear_forward(const void* hidden, int64_t ld_hidden, const void* weight,
                            int64_t ld_weight, int dtype, int64_t rows, int64_t H, int64_t V,
                            const int64_t* target, const float* class_weight,
                            int64_t ignore_index, float label_smoothing, float lse_square_scale,
                            float softcap, int reduction, uint32_t flags,
                            const float* grad_output, int per_row, int64_t chunk_rows,
                            float* loss, float* z_loss, float* token_accuracy, int64_t* argmax,
                            int64_t* counts, float* grad_hidden, int64_t ld_grad_hidden,
                            float* grad_weight, int64_t ld_grad_weight, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Vocabulary-parallel cross-entropy: the part one device runs when the V_total
 * classes are split over num_shards devices, this one holding the columns
 * [v_offset, v_offset + V) of every row. The Liger-Kernel page above, Tiling
 * Strategy, processes a row of any length in chunks; here the chunks live on
 * different devices (the tt-mlir PR #9324 page's commit list moves the
 * composites towards multi-chip sharding).
 *  1. ce_shard_partials reduces this device's columns of each row to one
 *     32-byte partial (max, sum of exponentials, smoothing sum, largest raw
 *     logit with its first global index, the target logit when the target is
 *     one of these columns).
 *  2. The caller gathers the num_shards partial arrays, in increasing
 *     v_offset order, into partials_all (num_shards, rows) x 32 bytes (an
 *     all-gather between devices; on one device, the arrays side by side).
 *  3. ce_shard_finish combines each row's partials in that order (every
 *     shard gets bitwise identical row scalars), writes the outputs of
 *     ce_forward (each shard the same values) and overwrites this device's
 *     columns with their gradient.
 * Conventions of ce_forward; target and weight are global: target (rows)
 * holds class indices in [0, V_total), weight is (V_total) or NULL (with
 * label smoothing and weights, weight + v_offset must be 16-byte aligned
 * for the vector path). Argmax and token accuracy are over all V_total
 * classes, lowest global index on ties.
 * ------------------------------------------------------------------------ */

/* Workspace bytes ce_shard_finish needs (>= 256), or 0 for invalid rows. */
size_t ce_shard_workspace_bytes(int64_t rows);

/* Stage 1.
 *  logits     [device] (rows, row_stride): this device's V columns, read only.
 *  partials   [device] rows x 32 bytes, written.
 * Errors: CE_E_SHAPE also when v_offset < 0 or v_offset + V > V_total. */
ce_status ce_shard_partials(const void* logits, int dtype, int64_t rows, int64_t V,
                            int64_t row_stride, int64_t v_offset, int64_t V_total,
                            const int64_t* target, const float* weight, int64_t ignore_index,
                            float label_smoothing, float softcap, void* partials, void* stream);

/* Stage 3 (after the gather).
 *  logits        [device] this device's columns, overwritten by the gradient.
 *  partials_all  [device] (num_shards, rows) partials, shards by increasing
 *                v_offset; this device's own are among them.
 *  flags         CE_F_CHECK_TARGETS only.
 *  loss, z_loss, token_accuracy, argmax, counts as for ce_forward.
 *  workspace     >= ce_shard_workspace_bytes(rows), 256-byte aligned, zero
 *                filled before its first use; reusable across calls. */
ce_status ce_shard_finish(void* logits, int dtype, int64_t rows, int64_t V, int64_t row_stride,
                          int64_t v_offset, int64_t V_total, const int64_t* target,
                          const float* weight, int64_t ignore_index, float label_smoothing,
                          float lse_square_scale, float softcap, int reduction, uint32_t flags,
                          const void* partials_all, int num_shards, float* loss, float* z_loss,
                          float* token_accuracy, int64_t* argmax, int64_t* counts,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable text of a ce_status value. */
const char* ce_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CE_MI355X_H */
