// Host-side checks of the C ABI's argument validation and workspace queries,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
// (tests/test_sanitize.py).  Every call here is rejected, or is a pure size
// query, before the library makes any HIP call, so no GPU is needed.  Exit
// status 0 when every status matches; the sanitizers abort on the first
// report.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "gram_select.h"
#include "rope_attn.h"

static int g_fail = 0, g_n = 0;

#define EXPECT(expr, want)                                                            \
  do {                                                                                \
    const long long got_ = (long long)(expr);                                         \
    ++g_n;                                                                            \
    if (got_ != (long long)(want)) {                                                  \
      fprintf(stderr, "line %d: %s = %lld, expected %lld\n", __LINE__, #expr, got_,   \
              (long long)(want));                                                     \
      ++g_fail;                                                                       \
    }                                                                                 \
  } while (0)

#define EXPECT_TRUE(cond)                                                 \
  do {                                                                    \
    ++g_n;                                                                \
    if (!(cond)) {                                                        \
      fprintf(stderr, "line %d: %s is false\n", __LINE__, #cond);         \
      ++g_fail;                                                           \
    }                                                                     \
  } while (0)

int main() {
  // Stand-in device pointers: 16-byte aligned, never dereferenced, since
  // validation fails first.
  void* A = (void*)(uintptr_t)4096;
  float* F = (float*)A;
  void* M = (void*)(uintptr_t)(4096 + 2);  // misaligned
  const double b = 1e4;
  const size_t big = (size_t)1 << 30;

  // workspace queries: valid shapes give a size, invalid ones 0; extreme
  // arguments must not overflow
  EXPECT_TRUE(rope_attn_fwd_workspace_bytes(1, 32, 8192, 128, ROPE_ATTN_BF16, 1) > 0);
  EXPECT_TRUE(rope_attn_bwd_workspace_bytes(1, 32, 8192, 128, ROPE_ATTN_BF16, 1) >
              rope_attn_bwd_workspace_bytes_min(1, 32, 8192, 128, ROPE_ATTN_BF16, 1));
  EXPECT_TRUE(rope_attn_bwd_workspace_bytes(1, 8, 32768, 64, ROPE_ATTN_BF16, 1) ==
              rope_attn_bwd_workspace_bytes_min(1, 8, 32768, 64, ROPE_ATTN_BF16, 1));
  EXPECT_TRUE(rope_attn_bwd_workspace_bytes(1, 1, 128, 64, ROPE_ATTN_FP32, 1) > 0);
  EXPECT(rope_attn_fwd_workspace_bytes(1, 1, 16, 96, ROPE_ATTN_BF16, 1), 0);
  EXPECT(rope_attn_bwd_workspace_bytes(0, 1, 16, 64, ROPE_ATTN_BF16, 1), 0);
  EXPECT(rope_attn_bwd_workspace_bytes(1, 1, 16, 64, 7, 1), 0);
  EXPECT(rope_attn_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 128, ROPE_ATTN_BF16, 1), 0);
  EXPECT(rope_attn_fwd_workspace_bytes(INT_MIN, 1, 1, 64, ROPE_ATTN_BF16, 0), 0);
  EXPECT(rope_attn_bwd_workspace_bytes_min(1, 1 << 20, 1 << 20, 128, ROPE_ATTN_BF16, 1), 0);
  EXPECT_TRUE(rope_attn_bwd_workspace_bytes(1, 1, 1 << 24, 64, ROPE_ATTN_BF16, 1) > 0);
  EXPECT_TRUE(rope_attn_bwd_workspace_bytes(1 << 12, 1 << 12, 1, 64, ROPE_ATTN_FP32, 0) > 0);

  // forward
  EXPECT(rope_attn_fwd(nullptr, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_NULL);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 1, 16, 96, 1, b, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_SHAPE);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 0, 16, 64, 1, b, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_SHAPE);
  EXPECT(rope_attn_fwd(A, A, A, F, F, INT_MAX, INT_MAX, INT_MAX, 64, 1, b, nullptr, 1, A, big,
                       nullptr),
         ROPE_ATTN_ERR_SHAPE);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 1, 16, 64, 5, b, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_DTYPE);
  EXPECT(rope_attn_fwd(M, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_ALIGN);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1, A, 16, nullptr),
         ROPE_ATTN_ERR_WORKSPACE);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 1, 16, 64, 1, 0.0, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 1, 16, 64, 1, NAN, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 1, 16, 64, 1, INFINITY, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 2, A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  EXPECT(rope_attn_fwd(A, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1, nullptr, big, nullptr),
         ROPE_ATTN_ERR_NULL);
  EXPECT(rope_attn_fwd_stages(ROPE_ATTN_STAGE_ALL, A, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1,
                              M, big, nullptr),
         ROPE_ATTN_ERR_ALIGN);

  // options
  rope_attn_options o = {};
  o.unrotated_pairs = 33;
  EXPECT(rope_attn_fwd_ex(ROPE_ATTN_STAGE_ALL, &o, A, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1,
                          A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  o = rope_attn_options{};
  o.scale = -0.5f;
  EXPECT(rope_attn_fwd_ex(ROPE_ATTN_STAGE_ALL, &o, A, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1,
                          A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  o = rope_attn_options{};
  o.pos_offset = INT_MAX;
  EXPECT(rope_attn_fwd_ex(ROPE_ATTN_STAGE_ALL, &o, A, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1,
                          A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  o = rope_attn_options{};
  o.block_ptr = (const int*)A;
  o.block_nnz = 3;  // block_idx missing
  EXPECT(rope_attn_fwd_ex(ROPE_ATTN_STAGE_ALL, &o, A, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1,
                          A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  o.block_idx = (const int*)((uintptr_t)4096 + 1);
  EXPECT(rope_attn_bwd_ex(ROPE_ATTN_STAGE_ALL, &o, A, A, A, F, A, F, F, F, F, F, 1, 1, 16, 64, 1,
                          b, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_ALIGN);
  o = rope_attn_options{};
  o.block_ptr = (const int*)A;
  EXPECT(rope_attn_fwd_ex(ROPE_ATTN_STAGE_ALL, &o, A, A, A, F, F, 1, 1, 65537, 64, 1, b, nullptr,
                          1, A, big, nullptr),
         ROPE_ATTN_ERR_SHAPE);

  // backward
  EXPECT(rope_attn_bwd(A, A, A, F, A, F, F, F, nullptr, F, 1, 1, 16, 64, 1, b, nullptr, 1, A, big,
                       nullptr),
         ROPE_ATTN_ERR_NULL);
  EXPECT(rope_attn_bwd(A, A, A, F, A, F, F, F, F, F, 1, 1, 16, 128, 1, b, nullptr, 1, A, 1000,
                       nullptr),
         ROPE_ATTN_ERR_WORKSPACE);
  EXPECT(rope_attn_bwd(A, A, A, F, M, F, F, F, F, F, 1, 1, 16, 64, 1, b, nullptr, 1, A, big,
                       nullptr),
         ROPE_ATTN_ERR_ALIGN);
  EXPECT(rope_attn_bwd_stages(ROPE_ATTN_STAGE_ALL, A, A, A, F, A, F, F, F, F, F, 1, 1, 16, 64, 3,
                              b, nullptr, 1, A, big, nullptr),
         ROPE_ATTN_ERR_DTYPE);
  EXPECT(rope_attn_bwd(A, A, A, F, A, F, F, F, F, F, 1, 1, 16, 64, 1, -1.0, nullptr, 1, A, big,
                       nullptr),
         ROPE_ATTN_ERR_ARG);

  // range flags and the no-allocation forward
  unsigned flags = 0;
  EXPECT(rope_attn_workspace_flags(nullptr, big, &flags, nullptr), ROPE_ATTN_ERR_NULL);
  EXPECT(rope_attn_workspace_flags(A, big, nullptr, nullptr), ROPE_ATTN_ERR_NULL);
  EXPECT(rope_attn_workspace_flags(M, big, &flags, nullptr), ROPE_ATTN_ERR_ALIGN);
  EXPECT(rope_attn_workspace_flags(A, 2, &flags, nullptr), ROPE_ATTN_ERR_WORKSPACE);
  EXPECT(rope_attn_fwd_noalloc(A, A, A, F, F, 1, 1, 16, 96, 1, b, nullptr, 1, nullptr),
         ROPE_ATTN_ERR_SHAPE);
  EXPECT(rope_attn_fwd_noalloc(nullptr, A, A, F, F, 1, 1, 16, 64, 1, b, nullptr, 1, nullptr),
         ROPE_ATTN_ERR_NULL);
  EXPECT(rope_attn_fwd_noalloc(A, A, A, F, F, 1, 1, 16, 64, 1, NAN, nullptr, 1, nullptr),
         ROPE_ATTN_ERR_ARG);
  EXPECT(rope_attn_fwd_noalloc(A, A, A, F, F, 1, 64, 8192, 128, 1, b, nullptr, 1, nullptr),
         ROPE_ATTN_ERR_WORKSPACE);

  // Gram selection
  EXPECT_TRUE(gram_select_workspace_bytes(2, 512, 768) > 0);
  EXPECT(gram_select_workspace_bytes(0, 512, 768), 0);
  EXPECT(gram_select_workspace_bytes(INT_MAX, INT_MAX, 64), 0);
  EXPECT(gram_cascade_workspace_bytes(512, 100), 0);
  unsigned char* U = (unsigned char*)A;
  int* I = (int*)A;
  EXPECT(gram_select(nullptr, 1, 64, 64, GRAM_BF16, 0.3f, F, U, I, A, big, nullptr),
         ROPE_ATTN_ERR_NULL);
  EXPECT(gram_select(A, 1, 64, 64, 9, 0.3f, F, U, I, A, big, nullptr), ROPE_ATTN_ERR_DTYPE);
  EXPECT(gram_select(A, 1, 64, 64, GRAM_BF16, NAN, F, U, I, A, big, nullptr), ROPE_ATTN_ERR_ARG);
  EXPECT(gram_select(A, 1, 64, 64, GRAM_BF16, 0.3f, F, U, I, A, 8, nullptr),
         ROPE_ATTN_ERR_WORKSPACE);
  EXPECT(gram_select_stages(GRAM_STAGE_ALL, A, 1, 64, 96, GRAM_BF16, 0.3f, F, U, I, A, big,
                            nullptr),
         ROPE_ATTN_ERR_SHAPE);
  EXPECT(gram_cascade(A, 64, 64, GRAM_FP16, -1.0f, U, F, U, I, A, big, nullptr),
         ROPE_ATTN_ERR_ARG);
  EXPECT(gram_cascade(A, 64, 64, GRAM_FP16, 0.3f, nullptr, F, U, I, A, big, nullptr),
         ROPE_ATTN_ERR_NULL);

  // status strings: every code, and unknown ones, give a static string
  for (int s = -9; s <= 2; ++s) EXPECT_TRUE(rope_attn_status_string(s) != nullptr);
  EXPECT_TRUE(rope_attn_status_string(INT_MIN) != nullptr);

  printf("%d checks, %d failed\n", g_n, g_fail);
  return g_fail ? 1 : 0;
}
