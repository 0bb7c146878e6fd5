// Host-side checks of the C ABI's validation and workspace planning, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the
// device code is not instrumented).  No call here reaches a kernel launch:
// every entry point is either a pure host query or called with arguments it
// rejects before enqueueing anything.  Exit status 0 means every check held
// and no sanitizer fired (the sanitizers abort on their first report).
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "grpo.h"

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static void* const FAKE = (void*)0x1000;   // never dereferenced

static void workspace_queries() {
  const int64_t Ns[] = {1, 7, 255, 256, 257, 4096, 32768, 163840, 1 << 22};
  const int64_t ds[] = {8, 16, 64, 1536, 2880, 4096, 8192, 16384};
  const int64_t Vs[] = {1, 3, 255, 256, 257, 1000, 128256, 151936, 201088, 262144};
  const int64_t chunks[] = {1, 128, 256, 300, 4096, 8192, 16384, 1 << 20};
  for (int64_t N : Ns)
    for (int64_t d : ds)
      for (int64_t V : Vs)
        for (int64_t c : chunks)
          for (int dt = 0; dt <= 2; ++dt) {
            size_t w[4];
            for (int op = 0; op < 4; ++op) w[op] = grpo_workspace_bytes(op, N, d, V, dt, c);
            CHECK(w[0] == w[1]);
            // the backward's minimum never exceeds its default plan
            CHECK(w[3] <= w[2]);
            if (w[2] != 0) CHECK(w[3] != 0);
          }
  CHECK(grpo_workspace_bytes(4, 512, 256, 1024, 0, 128) == 0);
  CHECK(grpo_workspace_bytes(-1, 512, 256, 1024, 0, 128) == 0);
  CHECK(grpo_workspace_bytes(1, 0, 256, 1024, 0, 128) == 0);
  CHECK(grpo_workspace_bytes(1, 512, 255, 1024, 0, 128) == 0);
  CHECK(grpo_workspace_bytes(1, 512, 256, 1024, 7, 128) == 0);
  CHECK(grpo_workspace_bytes(1, INT64_MAX, 256, 1024, 0, 128) == 0);
  CHECK(grpo_workspace_bytes(2, 512, 256, INT64_MAX, 1, 128) == 0);
  CHECK(grpo_workspace_bytes(2, 512, INT64_MAX - 7, 1024, 1, 128) == 0);
}

static void auto_chunk() {
  const int64_t shapes[][4] = {{32, 1024, 1536, 151936}, {8, 20480, 4096, 128256},
                               {4, 16384, 2880, 201088}, {1, 7, 16, 3}, {3, 100, 64, 500}};
  const size_t budgets[] = {0, 1, 1 << 20, 1ull << 30, 12ull << 30, SIZE_MAX};
  for (auto& s : shapes)
    for (size_t b : budgets)
      for (int dt = 0; dt <= 2; ++dt) {
        const int64_t c = grpo_auto_chunk(s[0], s[1], s[2], s[3], dt, b);
        if (dt == 0 && s[2] % 4) continue;
        CHECK(c == 0 || (c % 256 == 0 && c >= 256 && c <= 8192));
      }
  CHECK(grpo_auto_chunk(0, 8, 16, 32, 1, 1 << 30) == 0);
  CHECK(grpo_auto_chunk(INT64_MAX, 2, 16, 32, 1, 1 << 30) == 0);
  CHECK(grpo_auto_chunk(2, 8, 16, 32, 9, 1 << 30) == 0);
}

static void rejected_calls() {
  float f;
  grpo_opts bad = {};
  bad.temperature = NAN;
  // forward: each argument error is caught before a launch
  CHECK(grpo_loss_fwd(nullptr, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, 2, 4, 16, 32, 0,
                      0.04f, 8, &f, &f, &f, &f, FAKE, 1 << 20, nullptr) == GRPO_ERR_INVALID_ARG);
  CHECK(grpo_loss_fwd(FAKE, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, 2, 4, 16, 32, 0, NAN, 8,
                      &f, &f, &f, &f, FAKE, 1 << 20, nullptr) == GRPO_ERR_INVALID_ARG);
  CHECK(grpo_loss_fwd(FAKE, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, 2, 4, 16, 32, 0, 0.04f,
                      8, &f, &f, &f, &f, FAKE, 16, nullptr) == GRPO_ERR_WORKSPACE);
  CHECK(grpo_loss_fwd(FAKE, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, INT64_MAX, 4, 16, 32, 0,
                      0.04f, 8, &f, &f, &f, &f, FAKE, 1 << 20, nullptr) == GRPO_ERR_UNSUPPORTED);
  CHECK(grpo_loss_fwd_ex(FAKE, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, 2, 4, 16, 32, 0,
                         0.04f, 8, &bad, &f, &f, &f, &f, FAKE, 1 << 20, nullptr) ==
        GRPO_ERR_INVALID_ARG);
  CHECK(strlen(grpo_last_error()) > 0);
  // backward: a workspace below the minimum plans the slab and is refused
  for (int dt = 0; dt <= 1; ++dt) {
    const size_t least = grpo_workspace_bytes(GRPO_OP_BWD_MIN, 32768, 1536, 151936, dt, 4096);
    CHECK(least > 0);
    for (size_t w : {(size_t)0, (size_t)1, least / 2, least - 1})
      CHECK(grpo_loss_bwd(FAKE, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, &f, &f, 32, 1024,
                          1536, 151936, dt, 0.04f, 1.0f, 4096, FAKE, &f, FAKE, w, nullptr) ==
            GRPO_ERR_WORKSPACE);
  }
  CHECK(grpo_loss_bwd(FAKE, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, &f, &f, 2, 4, 16, 32, 0,
                      0.04f, INFINITY, 8, FAKE, &f, FAKE, 1 << 20, nullptr) == GRPO_ERR_INVALID_ARG);
  CHECK(grpo_loss_bwd(FAKE, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, &f, &f, 2, 4, 16, 32, 0,
                      0.04f, 1.0f, 8, FAKE, nullptr, FAKE, 1 << 20, nullptr) == GRPO_ERR_INVALID_ARG);
  {
    const size_t least = grpo_workspace_bytes(GRPO_OP_BWD_MIN, 32768, 1536, 151936, 2, 4096);
    CHECK(grpo_loss_bwd_fp8((uint8_t*)FAKE, &f, (uint8_t*)FAKE, &f, (int32_t*)FAKE, (uint8_t*)FAKE,
                            &f, &f, &f, &f, 32, 1024, 1536, 151936, 0.04f, 1.0f, 4096, nullptr, FAKE,
                            &f, FAKE, least - 1, nullptr) == GRPO_ERR_WORKSPACE);
  }
  // reference, advantages, fp8 helpers, the tile GEMM, the forward without allocation
  CHECK(grpo_ref_logprobs(FAKE, FAKE, nullptr, 512, 256, 1024, 0, 128, &f, FAKE, 1 << 20,
                          nullptr) == GRPO_ERR_INVALID_ARG);
  CHECK(grpo_advantages(&f, 0, 4, 1e-4f, &f, nullptr) == GRPO_ERR_INVALID_ARG);
  CHECK(grpo_advantages(&f, 2, 4, -1.0f, &f, nullptr) == GRPO_ERR_INVALID_ARG);
  CHECK(grpo_quantize_fp8(FAKE, 1, 4, 15, 1, (uint8_t*)FAKE, &f, nullptr, 0, nullptr) ==
        GRPO_ERR_UNSUPPORTED);
  CHECK(grpo_quantize_fp8(FAKE, 1, 4, 16, 0, (uint8_t*)FAKE, &f, nullptr, 0, nullptr) ==
        GRPO_ERR_WORKSPACE);
  CHECK(grpo_dequantize_fp8((uint8_t*)FAKE, &f, 4, 16, 2, FAKE, nullptr) == GRPO_ERR_INVALID_ARG);
  CHECK(grpo_gemm_nt(FAKE, FAKE, 4, 4, 6, 1, &f, nullptr) == GRPO_ERR_UNSUPPORTED);
  CHECK(grpo_loss_fwd_noalloc(FAKE, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE, &f, &f, 8, 4096, 1536,
                              151936, 1, 0.04f, 16384, nullptr, &f, &f, &f, &f, nullptr) ==
        GRPO_ERR_WORKSPACE);
  CHECK(grpo_noalloc_scratch_bytes() == (64u << 20));
  for (int code = -5; code <= 1; ++code) CHECK(grpo_strerror(code) != nullptr);
}

int main() {
  workspace_queries();
  auto_chunk();
  rejected_calls();
  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
