/* Host-side checks of the C ABI, run against the library built with its host
 * code under AddressSanitizer and UndefinedBehaviorSanitizer (no call below
 * reaches a kernel launch or any HIP call). Every entry point
 * declared in include/ce.h and include/ce_stream.h is called with invalid
 * arguments, and the host-only functions (workspace sizes, path planning,
 * status strings) over a grid of sizes up to the int64 limits, so an
 * out-of-bounds access or an overflowing size computation stops the
 * program with the sanitizer's report. Prints "ABI HOST CHECKS OK". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ce.h"
#include "ce_stream.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

/* Never dereferenced: every call that gets it fails validation first. */
#define FAKE ((void*)(uintptr_t)(1u << 20))
#define FAKE_OFF(b) ((void*)((uintptr_t)(1u << 20) + (b)))

static const int64_t kRows[] = {-5, -1, 0, 1, 7, 255, 256, 1023, 4096, 65536, 2147483647LL,
                                2147483648LL, 1LL << 40, INT64_MAX};
static const int64_t kV[] = {-1, 0, 1, 3, 4, 7, 8, 9, 1000, 4096, 32768, 128256, 131072, 262144,
                             1LL << 20, 1LL << 24, 2147483647LL, 2147483648LL, INT64_MAX};
static const uint32_t kFlags[] = {0u, CE_F_GRAD, CE_F_FORCE_FUSED, CE_F_FORCE_SPLITV,
                                  CE_F_FORCE_SCALAR, CE_F_SHAPE_ALT, 0x3FFu};
#define N(a) (sizeof(a) / sizeof((a)[0]))

static void status_strings(void) {
  for (int s = -100; s <= 100; ++s) {
    const char* t = ce_status_string(s);
    EXPECT(t != NULL && strlen(t) > 0);
    if (s >= CE_E_SCRATCH && s <= 0) EXPECT(strcmp(t, "unknown status") != 0);
  }
}

static void workspace_sizes(void) {
  for (size_t i = 0; i < N(kRows); ++i)
    for (size_t j = 0; j < N(kV); ++j)
      for (int dt = -1; dt <= 2; ++dt)
        for (size_t f = 0; f < N(kFlags); ++f) {
          const size_t b = ce_workspace_bytes(kRows[i], kV[j], dt, kFlags[f]);
          const int valid = kRows[i] >= 0 && kV[j] >= 1 && kRows[i] <= 2147483647LL &&
                            kV[j] <= 2147483647LL && (dt == CE_F32 || dt == CE_BF16);
          if (!valid) EXPECT(b == 0);
          if (b != 0) EXPECT(b >= 256 && b % 256 == 0);
        }
  for (size_t i = 0; i < N(kRows); ++i) {
    const size_t b = ce_shard_workspace_bytes(kRows[i]);
    if (kRows[i] < 0 || kRows[i] > 2147483647LL) EXPECT(b == 0);
    else EXPECT(b >= 256);
  }
  const int64_t H[] = {-1, 0, 1, 4096, 2147483647LL, 2147483648LL};
  const int64_t chunk[] = {-1, 0, 1, 64, 4096, INT64_MAX};
  for (size_t i = 0; i < N(kRows); ++i)
    for (size_t j = 0; j < N(kV); ++j)
      for (size_t h = 0; h < N(H); ++h)
        for (size_t c = 0; c < N(chunk); ++c) {
          const size_t b = ce_linear_workspace_bytes(kRows[i], H[h], kV[j], chunk[c], 0u);
          if (b != 0) EXPECT(b >= 256);
        }
}

static void plan_paths(void) {
  void* ptrs[] = {FAKE, FAKE_OFF(4), FAKE_OFF(8), NULL};
  for (size_t i = 0; i < N(kRows); ++i)
    for (size_t j = 0; j < N(kV); ++j)
      for (size_t q = 0; q < N(ptrs); ++q)
        for (size_t f = 0; f < N(kFlags); ++f) {
          const int64_t stride = kV[j];
          const int r = ce_plan_path(ptrs[q], CE_BF16, kRows[i], kV[j], stride,
                                     (const float*)FAKE_OFF(4), 0.1f, kFlags[f]);
          EXPECT(r < 0 || r == CE_PATH_FUSED || r == CE_PATH_SPLITV || r == CE_PATH_SCALAR);
        }
  EXPECT(ce_plan_path(FAKE, 5, 8, 64, 64, NULL, 0.0f, 0u) == CE_E_DTYPE);
  EXPECT(ce_plan_path(FAKE, CE_F32, 8, 64, 32, NULL, 0.0f, 0u) == CE_E_SHAPE);
}

/* ce_forward / ce_forward_noalloc with one argument made invalid at a time. */
typedef struct {
  void* logits; int dtype; int64_t rows, V, stride; const int64_t* target; const float* weight;
  float eps, lam, cap; int red; uint32_t flags; float* loss; void* ws; size_t wsb;
} Fwd;

static Fwd fwd_default(void) {
  Fwd a = {FAKE, CE_F32, 4, 16, 16, (const int64_t*)FAKE, NULL, 0.0f, 0.0f, 0.0f, CE_RED_MEAN,
           0u, (float*)FAKE, NULL, 0};
  return a;
}

static int fwd(Fwd a) {
  return ce_forward(a.logits, a.dtype, a.rows, a.V, a.stride, a.target, a.weight, -100, a.eps,
                    a.lam, a.cap, a.red, a.flags, a.loss, NULL, NULL, NULL, NULL, NULL, a.ws,
                    a.wsb, NULL);
}

static int fwd_noalloc(Fwd a) {
  return ce_forward_noalloc(a.logits, a.dtype, a.rows, a.V, a.stride, a.target, a.weight, -100,
                            a.eps, a.lam, a.cap, a.red, a.flags, a.loss, NULL, NULL, NULL, NULL,
                            NULL, NULL);
}

static void forward_validation(void) {
  Fwd a;
  a = fwd_default(); a.dtype = 7; EXPECT(fwd(a) == CE_E_DTYPE); EXPECT(fwd_noalloc(a) == CE_E_DTYPE);
  a = fwd_default(); a.rows = -1; EXPECT(fwd(a) == CE_E_SHAPE);
  a = fwd_default(); a.V = 0; EXPECT(fwd(a) == CE_E_SHAPE);
  a = fwd_default(); a.stride = 15; EXPECT(fwd(a) == CE_E_SHAPE);
  a = fwd_default(); a.V = a.stride = 1LL << 31; EXPECT(fwd(a) == CE_E_SHAPE);
  a = fwd_default(); a.red = 3; EXPECT(fwd(a) == CE_E_PARAM);
  a = fwd_default(); a.eps = 1.5f; EXPECT(fwd(a) == CE_E_PARAM);
  a = fwd_default(); a.eps = NAN; EXPECT(fwd(a) == CE_E_PARAM);
  a = fwd_default(); a.cap = -1.0f; EXPECT(fwd(a) == CE_E_PARAM);
  a = fwd_default(); a.cap = INFINITY; EXPECT(fwd(a) == CE_E_PARAM);
  a = fwd_default(); a.lam = NAN; EXPECT(fwd(a) == CE_E_PARAM);
  a = fwd_default(); a.lam = -1.0f; EXPECT(fwd(a) == CE_E_PARAM);
  a = fwd_default(); a.loss = NULL; EXPECT(fwd(a) == CE_E_NULL); EXPECT(fwd_noalloc(a) == CE_E_NULL);
  a = fwd_default(); a.logits = NULL; EXPECT(fwd(a) == CE_E_NULL);
  a = fwd_default(); a.target = NULL; EXPECT(fwd(a) == CE_E_NULL);
  a = fwd_default(); a.wsb = 1u << 20; EXPECT(fwd(a) == CE_E_WORKSPACE);
  a = fwd_default(); a.ws = FAKE_OFF(8); a.wsb = 1u << 20; EXPECT(fwd(a) == CE_E_WORKSPACE);
  a = fwd_default(); a.ws = FAKE; a.wsb = 64; EXPECT(fwd(a) == CE_E_WORKSPACE);
  /* every valid size without a workspace: CE_E_WORKSPACE (or a shape error
   * for rows x chunks past the int range), never a launch */
  for (size_t i = 0; i < N(kRows); ++i)
    for (size_t j = 0; j < N(kV); ++j)
      for (size_t f = 0; f < N(kFlags); ++f) {
        a = fwd_default();
        a.rows = kRows[i]; a.V = a.stride = kV[j]; a.flags = kFlags[f]; a.dtype = CE_BF16;
        const int s = fwd(a);
        EXPECT(s == CE_E_WORKSPACE || s == CE_E_SHAPE);
        /* the no-alloc variant: problems past its scratch are refused on the
         * host (vector paths: the layout ce_workspace_bytes sizes) */
        if (s == CE_E_WORKSPACE && a.V % 8 == 0 && !(a.flags & CE_F_FORCE_SCALAR) &&
            ce_workspace_bytes(a.rows, a.V, a.dtype, a.flags) > CE_FORWARD_NOALLOC_MAX_BYTES)
          EXPECT(fwd_noalloc(a) == CE_E_SCRATCH);
      }
}

static void backward_validation(void) {
  EXPECT(ce_backward(FAKE, 2, 4, 16, 16, (const float*)FAKE, 0, NULL) == CE_E_DTYPE);
  EXPECT(ce_backward(FAKE, CE_BF16, -3, 16, 16, (const float*)FAKE, 0, NULL) == CE_E_SHAPE);
  EXPECT(ce_backward(FAKE, CE_BF16, 4, 16, 3, (const float*)FAKE, 0, NULL) == CE_E_SHAPE);
  EXPECT(ce_backward(FAKE, CE_BF16, 4, 16, 16, NULL, 0, NULL) == CE_E_NULL);
  EXPECT(ce_backward(NULL, CE_BF16, 4, 16, 16, (const float*)FAKE, 0, NULL) == CE_E_NULL);
  EXPECT(ce_backward(NULL, CE_BF16, 0, 16, 16, (const float*)FAKE, 0, NULL) == CE_OK);
  EXPECT(ce_backward(FAKE, CE_F32, INT64_MAX, INT64_MAX, INT64_MAX, (const float*)FAKE, 0,
                     NULL) == CE_E_SHAPE);
  const float* go = (const float*)FAKE;
  const float* st = (const float*)FAKE;
  EXPECT(ce_backward_recompute(FAKE, 3, 4, 16, 16, (const int64_t*)FAKE, NULL, -100, 0.0f, 0.0f,
                               0.0f, CE_RED_MEAN, st, go, 0, FAKE_OFF(4096), 16, FAKE, 256,
                               NULL) == CE_E_DTYPE);
  EXPECT(ce_backward_recompute(FAKE, CE_F32, 4, 16, 16, (const int64_t*)FAKE, NULL, -100, 0.0f,
                               0.0f, 0.0f, CE_RED_MEAN, st, go, 0, FAKE, 32, FAKE, 256,
                               NULL) == CE_E_SHAPE);
  EXPECT(ce_backward_recompute(FAKE, CE_F32, 4, 16, 16, (const int64_t*)FAKE, NULL, -100, 0.0f,
                               0.0f, 0.0f, CE_RED_MEAN, NULL, go, 0, FAKE_OFF(4096), 16, FAKE,
                               256, NULL) == CE_E_NULL);
  EXPECT(ce_backward_recompute(FAKE, CE_F32, 4, 16, 16, (const int64_t*)FAKE, NULL, -100, 0.0f,
                               0.0f, 0.0f, CE_RED_MEAN, st, go, 0, FAKE_OFF(4096), 16, FAKE, 128,
                               NULL) == CE_E_WORKSPACE);
  EXPECT(ce_backward_recompute(NULL, CE_F32, 0, 16, 16, (const int64_t*)FAKE, NULL, -100, 0.0f,
                               0.0f, 0.0f, CE_RED_MEAN, NULL, go, 0, NULL, 16, FAKE, 256,
                               NULL) == CE_OK);
}

static void linear_validation(void) {
  float* loss = (float*)FAKE;
#define LIN(dtype, rows, H, V, ldh, ldw, red, per_row, chunk, lossp, ws, wsb)                  \
  ce_linear_forward(FAKE, ldh, FAKE, ldw, dtype, rows, H, V, (const int64_t*)FAKE, NULL, -100, \
                    0.0f, 0.0f, 0.0f, red, 0u, NULL, per_row, chunk, lossp, NULL, NULL, NULL, \
                    NULL, NULL, 0, NULL, 0, ws, wsb, NULL)
  EXPECT(LIN(CE_F32, 4, 64, 128, 64, 64, CE_RED_MEAN, 0, 0, loss, FAKE, 1u << 30) == CE_E_DTYPE);
  EXPECT(LIN(CE_BF16, 4, 0, 128, 64, 64, CE_RED_MEAN, 0, 0, loss, FAKE, 1u << 30) == CE_E_SHAPE);
  EXPECT(LIN(CE_BF16, 4, 64, 128, 32, 64, CE_RED_MEAN, 0, 0, loss, FAKE, 1u << 30) == CE_E_SHAPE);
  EXPECT(LIN(CE_BF16, 4, 64, 128, 64, 32, CE_RED_MEAN, 0, 0, loss, FAKE, 1u << 30) == CE_E_SHAPE);
  EXPECT(LIN(CE_BF16, 4, 64, 128, 64, 64, CE_RED_MEAN, 0, -1, loss, FAKE, 1u << 30) == CE_E_SHAPE);
  EXPECT(LIN(CE_BF16, 4, 64, 128, 64, 64, CE_RED_MEAN, 0, 0, NULL, FAKE, 1u << 30) == CE_E_NULL);
  EXPECT(LIN(CE_BF16, 4, 64, 128, 64, 64, CE_RED_MEAN, 1, 0, loss, FAKE, 1u << 30) == CE_E_PARAM);
  EXPECT(LIN(CE_BF16, 4, 64, 128, 64, 64, CE_RED_MEAN, 0, 0, loss, NULL, 1u << 30) ==
         CE_E_WORKSPACE);
  EXPECT(LIN(CE_BF16, 4, 64, 128, 64, 64, CE_RED_MEAN, 0, 0, loss, FAKE, 16) == CE_E_WORKSPACE);
  EXPECT(LIN(CE_BF16, INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX, CE_RED_MEAN, 0, 0,
             loss, FAKE, 16) == CE_E_SHAPE);
#undef LIN
}

static void shard_validation(void) {
  void* f = FAKE;
  const int64_t* t = (const int64_t*)FAKE;
  EXPECT(ce_shard_partials(f, CE_F32, 4, 100, 100, 950, 1000, t, NULL, -100, 0.0f, 0.0f, f,
                           NULL) == CE_E_SHAPE);
  EXPECT(ce_shard_partials(f, CE_F32, 4, 100, 100, -1, 1000, t, NULL, -100, 0.0f, 0.0f, f,
                           NULL) == CE_E_SHAPE);
  EXPECT(ce_shard_partials(f, CE_F32, 4, 100, 100, INT64_MAX, INT64_MAX, t, NULL, -100, 0.0f,
                           0.0f, f, NULL) == CE_E_SHAPE);
  EXPECT(ce_shard_partials(f, 9, 4, 100, 100, 0, 1000, t, NULL, -100, 0.0f, 0.0f, f, NULL) ==
         CE_E_DTYPE);
  EXPECT(ce_shard_partials(NULL, CE_F32, 4, 100, 100, 0, 1000, t, NULL, -100, 0.0f, 0.0f, f,
                           NULL) == CE_E_NULL);
  EXPECT(ce_shard_partials(NULL, CE_F32, 0, 100, 100, 0, 1000, NULL, NULL, -100, 0.0f, 0.0f,
                           NULL, NULL) == CE_OK);
#define FIN(shards, eps, lossp, ws, wsb)                                                       \
  ce_shard_finish(f, CE_F32, 4, 100, 100, 0, 1000, t, NULL, -100, eps, 0.0f, 0.0f, CE_RED_SUM, \
                  0u, f, shards, lossp, NULL, NULL, NULL, NULL, ws, wsb, NULL)
  EXPECT(FIN(0, 0.0f, (float*)f, f, 1u << 20) == CE_E_PARAM);
  EXPECT(FIN(2, 1.5f, (float*)f, f, 1u << 20) == CE_E_PARAM);
  EXPECT(FIN(2, 0.0f, (float*)f, f, 8) == CE_E_WORKSPACE);
  EXPECT(FIN(2, 0.0f, (float*)f, FAKE_OFF(8), 1u << 20) == CE_E_WORKSPACE);
  EXPECT(FIN(2, 0.0f, NULL, f, 1u << 20) == CE_E_NULL);
#undef FIN
}

static void stream_validation(void) {
  const int n = ce_stream_num_configs();
  EXPECT(n > 0);
  for (int c = -3; c < n + 3; ++c) {
    int b = -1, r = -1;
    const int s = ce_stream_config(c, &b, &r);
    if (c < 0 || c >= n) {
      EXPECT(s == -4);
    } else {
      EXPECT(s == 0 && b > 0 && r > 0);
    }
    EXPECT(ce_stream_config(c, NULL, &r) == -4);
  }
  EXPECT(ce_stream_resident(-1, 0) == -4);
  EXPECT(ce_stream_resident(5, 0) == -4);
  EXPECT(ce_stream_resident(0, n) == -4);
  uint32_t* sink = (uint32_t*)FAKE;
  EXPECT(ce_stream_run(9, 0, FAKE, FAKE, 1024, 0, sink, NULL) == -4);
  EXPECT(ce_stream_run(CE_STREAM_READ, 0, NULL, NULL, 1024, 0, sink, NULL) == -1);
  EXPECT(ce_stream_run(CE_STREAM_READ, 0, NULL, FAKE, 1024, 0, NULL, NULL) == -1);
  EXPECT(ce_stream_run(CE_STREAM_WRITE, 0, NULL, NULL, 1024, 0, NULL, NULL) == -1);
  EXPECT(ce_stream_run(CE_STREAM_COPY, 0, FAKE, FAKE, 1000, 0, NULL, NULL) == -2);
  EXPECT(ce_stream_run(CE_STREAM_COPY, 0, FAKE_OFF(4), FAKE, 1024, 0, NULL, NULL) == -2);
  EXPECT(ce_stream_run(CE_STREAM_INPLACE, 0, FAKE, NULL, (size_t)1 << 62, 0, NULL, NULL) == -2);
}

int main(void) {
  status_strings();
  workspace_sizes();
  plan_paths();
  forward_validation();
  backward_validation();
  linear_validation();
  shard_validation();
  stream_validation();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("ABI HOST CHECKS OK\n");
  return 0;
}
